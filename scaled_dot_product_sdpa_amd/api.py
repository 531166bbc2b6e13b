"""ctypes binding of libsdpa.so (include/sdpa.h).

Argument marshalling only: shapes and strides are read off torch tensors, outputs and the
workspace are allocated with torch on the inputs' device, and the call is forwarded to the
C ABI on torch's current stream.  Every step of the attention itself runs in the HIP
kernels; there is no fallback path.  If the library is missing the call fails.
"""

from __future__ import annotations

import ctypes
import math
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libsdpa.so"

SDPA_OK = 0
SDPA_ERR_INVALID_ARGUMENT = 1
SDPA_ERR_UNSUPPORTED = 2
SDPA_ERR_WORKSPACE_TOO_SMALL = 3
SDPA_ERR_HIP = 4
SDPA_DTYPE_F32 = 0
SDPA_DTYPE_BF16 = 1

EXPORTS = (
    "sdpa_forward_workspace_bytes", "sdpa_backward_workspace_bytes", "sdpa_forward",
    "sdpa_backward", "sdpa_status_string", "sdpa_last_error", "sdpa_version",
)


class Problem(ctypes.Structure):
    """Mirror of ``sdpa_problem``."""

    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Lq", ctypes.c_int32), ("Lk", ctypes.c_int32), ("Dqk", ctypes.c_int32),
        ("Dv", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("mask_stride", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float),
        ("is_causal", ctypes.c_int32),
    ]


class SdpaError(RuntimeError):
    pass


_LIB = None


def load_library(path: Path | str | None = None):
    """Load libsdpa.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with `python -m scaled_dot_product_sdpa_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pp = ctypes.POINTER(Problem)
    lib.sdpa_forward_workspace_bytes.argtypes = [pp]
    lib.sdpa_forward_workspace_bytes.restype = sz
    lib.sdpa_backward_workspace_bytes.argtypes = [pp]
    lib.sdpa_backward_workspace_bytes.restype = sz
    lib.sdpa_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_forward.restype = ctypes.c_int
    lib.sdpa_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_backward.restype = ctypes.c_int
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_version.restype = ctypes.c_int
    if path is None:
        _LIB = lib
    return lib


def _raise(lib, status: int):
    msg = lib.sdpa_last_error().decode()
    name = lib.sdpa_status_string(status).decode()
    text = f"sdpa: {name}: {msg}"
    if status == SDPA_ERR_INVALID_ARGUMENT:
        raise ValueError(text)
    if status == SDPA_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    raise SdpaError(text)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SDPA_DTYPE_BF16
    if t.dtype == torch.float32:
        return SDPA_DTYPE_F32
    raise NotImplementedError(f"sdpa: dtype {t.dtype} is not supported (bfloat16, float32)")


def _as4d(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dim() == 3:
        return t.unsqueeze(0)
    if t.dim() != 4:
        raise ValueError(f"sdpa: {name} must be (B, H, L, D) or (H, L, D), got {tuple(t.shape)}")
    return t


def _strides3(t: torch.Tensor, name: str):
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise NotImplementedError(f"sdpa: {name} must have unit stride along its last dim")
    return tuple(int(s) for s in t.stride()[:3])


def _mask4d(mask, B, Hq, Lq, Lk):
    if mask is None:
        return None, (0, 0, 0)
    m = mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if m.dim() != 4:
        raise ValueError(f"sdpa: mask must broadcast to (B, Hq, Lq, Lk), got {tuple(mask.shape)}")
    if m.shape[-2] != Lq or m.shape[-1] != Lk:
        raise ValueError(f"sdpa: mask's last dims {tuple(m.shape[-2:])} must be (Lq, Lk) = ({Lq}, {Lk})")
    for ax, full in ((0, B), (1, Hq)):
        if m.shape[ax] not in (1, full):
            raise ValueError(f"sdpa: mask dim {ax} = {m.shape[ax]} does not broadcast to {full}")
    if m.stride(-1) != 1 and Lk > 1:
        raise NotImplementedError("sdpa: mask must have unit stride along keys")
    st = [int(s) for s in m.stride()[:3]]
    if m.shape[0] == 1:
        st[0] = 0
    if m.shape[1] == 1:
        st[1] = 0
    return m, tuple(st)


def _lens(x, B, device, name):
    if x is None:
        return None
    if not torch.is_tensor(x):
        x = torch.tensor(x, dtype=torch.int32)
    x = x.reshape(-1)
    if x.numel() != B:
        raise ValueError(f"sdpa: {name} needs one length per batch ({B}), got {x.numel()}")
    return x.to(device=device, dtype=torch.int32).contiguous()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_problem(q, k, v, o_strides, mask_strides, scale, is_causal) -> Problem:
    B, Hq, Lq, Dqk = q.shape
    Bk, Hkv, Lk, Dk2 = k.shape
    Bv, Hv, Lv, Dv = v.shape
    if Bk != B or Bv != B:
        raise ValueError("sdpa: q, k and v must have the same batch size")
    if Dk2 != Dqk:
        raise ValueError(f"sdpa: q and k widths differ ({Dqk} vs {Dk2})")
    if Hv != Hkv or Lv != Lk:
        raise ValueError("sdpa: k and v must have the same heads and length")
    p = Problem()
    p.dtype = _dtype_code(q)
    p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.Dqk, p.Dv = B, Hq, Hkv, Lq, Lk, Dqk, Dv
    for field, t, name in (("q_stride", q, "q"), ("k_stride", k, "k"), ("v_stride", v, "v")):
        getattr(p, field)[:] = _strides3(t, name)
    p.o_stride[:] = o_strides
    p.mask_stride[:] = mask_strides
    p.scale = math.nan if scale is None else float(scale)
    p.is_causal = 1 if is_causal else 0
    return p


def _check_io(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("sdpa: tensors must be on a GPU device")
    for t in ts:
        if t.device != dev:
            raise ValueError("sdpa: all tensors must be on the same device")
        if t.dtype != ts[0].dtype:
            raise ValueError("sdpa: q, k, v (and o, dO, mask) must share one dtype")


def sdpa_forward(q, k, v, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                 seq_lens_kv=None, return_lse=True):
    """O (and LSE) of scaled dot-product attention.  q (B,Hq,Lq,D), k/v (B,Hkv,Lk,D)."""
    lib = load_library()
    squeeze = q.dim() == 3
    q, k, v = _as4d(q, "q"), _as4d(k, "k"), _as4d(v, "v")
    _check_io(q, k, v, *([mask] if mask is not None else []))
    B, Hq, Lq, _ = q.shape
    Lk, Dv = k.shape[2], v.shape[3]
    o = torch.empty((B, Hq, Lq, Dv), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if return_lse else None
    m, mst = _mask4d(mask, B, Hq, Lq, Lk)
    p = make_problem(q, k, v, _strides3(o, "o"), mst, scale, is_causal)
    lq = _lens(seq_lens_q, B, q.device, "seq_lens_q")
    lk = _lens(seq_lens_kv, B, q.device, "seq_lens_kv")
    nws = lib.sdpa_forward_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.sdpa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(lq), _ptr(lk),
                          _ptr(o), _ptr(lse), _ptr(ws), nws, ctypes.c_void_p(stream))
    if st != SDPA_OK:
        _raise(lib, st)
    if squeeze:
        o = o.squeeze(0)
        lse = lse.squeeze(0) if lse is not None else None
    return (o, lse) if return_lse else o


def sdpa_backward(q, k, v, o, dO, lse, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                  seq_lens_kv=None):
    """(dQ, dK, dV) from the forward's o and lse and the output gradient dO."""
    lib = load_library()
    squeeze = q.dim() == 3
    q, k, v, o, dO = (_as4d(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO")))
    if lse.dim() == 2:
        lse = lse.unsqueeze(0)
    _check_io(q, k, v, o, dO, *([mask] if mask is not None else []))
    B, Hq, Lq, _ = q.shape
    Lk = k.shape[2]
    if tuple(o.shape) != (B, Hq, Lq, v.shape[3]) or dO.shape != o.shape:
        raise ValueError("sdpa: o and dO must be (B, Hq, Lq, Dv)")
    if o.stride() != dO.stride():
        dO = dO.contiguous()
        o = o.contiguous()
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("sdpa: lse must be float32 (B, Hq, Lq)")
    lse = lse.contiguous()
    m, mst = _mask4d(mask, B, Hq, Lq, Lk)
    p = make_problem(q, k, v, _strides3(o, "o"), mst, scale, is_causal)
    lq = _lens(seq_lens_q, B, q.device, "seq_lens_q")
    lk = _lens(seq_lens_kv, B, q.device, "seq_lens_kv")
    dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
    dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    nws = lib.sdpa_backward_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = lib.sdpa_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dO), _ptr(lse),
                           _ptr(m), _ptr(lq), _ptr(lk), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nws,
                           ctypes.c_void_p(stream))
    if st != SDPA_OK:
        _raise(lib, st)
    if squeeze:
        dq, dk, dv = dq.squeeze(0), dk.squeeze(0), dv.squeeze(0)
    return dq, dk, dv
