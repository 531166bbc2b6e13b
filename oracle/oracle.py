"""ctypes marshalling for the fp64 C oracle (test infrastructure only).

Nothing here computes attention: arrays are converted to contiguous float64, the mask's
broadcast is described by element strides (0 on a broadcast dimension), and the C library
does the arithmetic.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "sdpa_oracle.c"


def oracle_lib_path() -> Path:
    return _HERE / "liboracle.so"


def build_oracle(out: Path | None = None, src: Path | None = None, extra_flags=()) -> Path:
    """Compile the oracle with gcc (fp64, IEEE semantics: no fast-math)."""
    out = Path(out) if out is not None else oracle_lib_path()
    src = Path(src) if src is not None else _SRC
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", f"-I{_HERE}",
           *extra_flags, "-o", str(tmp), str(src), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Lq", ctypes.c_int32), ("Lk", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32),
        ("mask_stride", ctypes.c_int64 * 4),
        ("scale", ctypes.c_double),
        ("is_causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)


# Causal modes (the ``is_causal`` argument): False/0 none, True/1 top-left diagonal,
# 2 bottom-right diagonal (aligned with the per-batch actual lengths).
CAUSAL_TOP_LEFT = 1
CAUSAL_BOTTOM_RIGHT = 2


def causal_mode(is_causal) -> int:
    mode = int(is_causal)
    if mode not in (0, 1, 2):
        raise ValueError("is_causal must be False/True (0/1) or 2 (bottom-right)")
    return mode


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, kind=_DP):
    return None if a is None else a.ctypes.data_as(kind)


class Oracle:
    """Handle on one build of the oracle library (the default build, or a test variant)."""

    def __init__(self, path: Path | str | None = None):
        path = Path(path) if path is not None else oracle_lib_path()
        self.path = path
        self.lib = ctypes.CDLL(str(path))
        for name in ("oracle_sdpa_forward", "oracle_sdpa_forward_rows", "oracle_sdpa_backward"):
            getattr(self.lib, name).restype = ctypes.c_int
        self.lib.oracle_num_threads.restype = ctypes.c_int

    @property
    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    # ---- marshalling -------------------------------------------------------------
    @staticmethod
    def _problem(q, k, v, mask, scale, is_causal, window=0):
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("oracle expects (B, H, L, D) arrays")
        B, Hq, Lq, Dk = q.shape
        Bk, Hkv, Lk, Dk2 = k.shape
        Bv, Hv, Lv, Dv = v.shape
        if Bk != B or Bv != B or Dk2 != Dk or Hv != Hkv or Lv != Lk:
            raise ValueError("inconsistent q/k/v shapes")
        p = _Problem()
        p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.Dk, p.Dv = B, Hq, Hkv, Lq, Lk, Dk, Dv
        p.scale = math.nan if scale is None else float(scale)
        p.is_causal = causal_mode(is_causal)
        p.window = int(window)
        m = None
        if mask is not None:
            m = _f64(mask)
            if m.ndim != 4:
                raise ValueError("mask must be 4-D, broadcastable to (B, Hq, Lq, Lk)")
            full = (B, Hq, Lq, Lk)
            for ax in range(4):
                if m.shape[ax] not in (1, full[ax]):
                    raise ValueError(f"mask dim {ax} = {m.shape[ax]} does not broadcast to {full[ax]}")
            st = [s // 8 for s in m.strides]
            for ax in range(4):
                p.mask_stride[ax] = 0 if (m.shape[ax] == 1 and full[ax] != 1) else st[ax]
        return p, m

    @staticmethod
    def _lens(lens, B):
        if lens is None:
            return None
        a = np.ascontiguousarray(lens, dtype=np.int32).reshape(-1)
        if a.shape[0] != B:
            raise ValueError("lengths must have one entry per batch")
        return a

    @staticmethod
    def _check(rc):
        if rc == -1:
            raise ValueError("oracle: invalid problem")
        if rc == -2:
            raise ValueError("oracle: mask holds NaN or +inf")
        if rc != 0:
            raise RuntimeError(f"oracle: status {rc}")

    # ---- calls ---------------------------------------------------------------------
    def forward(self, q, k, v, mask=None, scale=None, is_causal=False, len_q=None, len_kv=None,
                window=0):
        """``window`` W > 0 (with a causal diagonal): a row also sees only the last W keys
        up to its diagonal (the sliding window)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        p, m = self._problem(q, k, v, mask, scale, is_causal, window)
        lq, lk = self._lens(len_q, p.B), self._lens(len_kv, p.B)
        o = np.zeros((p.B, p.Hq, p.Lq, p.Dv))
        lse = np.zeros((p.B, p.Hq, p.Lq))
        rc = self.lib.oracle_sdpa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                                          _ptr(lq, _IP), _ptr(lk, _IP), _ptr(o), _ptr(lse))
        self._check(rc)
        return o, lse

    def forward_rows(self, q, k, v, rows, mask=None, scale=None, is_causal=False, len_q=None,
                     len_kv=None, window=0):
        """Forward on an explicit list of (b, h, i) rows; returns (o_rows, lse_rows)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        p, m = self._problem(q, k, v, mask, scale, is_causal, window)
        lq, lk = self._lens(len_q, p.B), self._lens(len_kv, p.B)
        r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
        o = np.zeros((r.shape[0], p.Dv))
        lse = np.zeros((r.shape[0],))
        rc = self.lib.oracle_sdpa_forward_rows(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                                               _ptr(lq, _IP), _ptr(lk, _IP),
                                               ctypes.c_int64(r.shape[0]), _ptr(r, _IP),
                                               _ptr(o), _ptr(lse))
        self._check(rc)
        return o, lse

    def backward(self, q, k, v, dO, mask=None, scale=None, is_causal=False, len_q=None,
                 len_kv=None, window=0):
        """Returns (dq, dk, dv, D) with D_i = sum_j P_ij dP_ij."""
        q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
        p, m = self._problem(q, k, v, mask, scale, is_causal, window)
        if dO.shape != (p.B, p.Hq, p.Lq, p.Dv):
            raise ValueError("dO must have the output's shape")
        lq, lk = self._lens(len_q, p.B), self._lens(len_kv, p.B)
        dq = np.zeros(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        dsum = np.zeros((p.B, p.Hq, p.Lq))
        rc = self.lib.oracle_sdpa_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(m),
                                           _ptr(lq, _IP), _ptr(lk, _IP), _ptr(dO), _ptr(dq),
                                           _ptr(dk), _ptr(dv), _ptr(dsum))
        self._check(rc)
        return dq, dk, dv, dsum


_DEFAULT: Oracle | None = None


def load_oracle(build_if_missing: bool = True) -> Oracle:
    """The default oracle build; compiled on first use if it is not there yet."""
    global _DEFAULT
    if _DEFAULT is None:
        if not oracle_lib_path().exists():
            if not build_if_missing:
                raise FileNotFoundError(oracle_lib_path())
            build_oracle()
        _DEFAULT = Oracle()
    return _DEFAULT
