"""ctypes binding of libsdpa.so (include/sdpa.h).

Argument marshalling only: shapes and strides are read off torch tensors, outputs and the
workspace are allocated with torch on the inputs' device, and the call is forwarded to the
C ABI on torch's current stream.  Every step of the attention itself runs in the HIP
kernels; there is no fallback path.  If the library is missing the call fails.

``ForwardCall`` / ``BackwardCall`` marshal once and then launch with the cached
arguments (used for timing and for capture into HIP graphs); ``sdpa_forward`` /
``sdpa_backward`` are the one-shot forms.
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
    "sdpa_forward_workspace_bytes", "sdpa_backward_workspace_bytes",
    "sdpa_backward_workspace_bytes_min", "sdpa_forward",
    "sdpa_backward", "sdpa_backward_prep", "sdpa_backward_dkdv", "sdpa_backward_dq",
    "sdpa_backward_main",
    "sdpa_status_string", "sdpa_last_error", "sdpa_version", "sdpa_decode_paged_workspace_bytes",
    "sdpa_decode_paged", "sdpa_forward_ragged", "sdpa_backward_ragged", "sdpa_forward_noalloc",
)
BACKWARD_STAGES = ("prep", "dkdv", "dq", "main")


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
        ("sliding_window", ctypes.c_int32),
    ]


class PagedDecode(ctypes.Structure):
    """Mirror of ``sdpa_paged_decode``."""

    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 2), ("o_stride", ctypes.c_int64 * 2),
        ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float), ("sliding_window", ctypes.c_int32),
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
    lib.sdpa_backward_workspace_bytes_min.argtypes = [pp]
    lib.sdpa_backward_workspace_bytes_min.restype = sz
    lib.sdpa_forward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_forward.restype = ctypes.c_int
    lib.sdpa_forward_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sdpa_forward_noalloc.restype = ctypes.c_int
    for name in ("sdpa_backward", "sdpa_backward_prep", "sdpa_backward_dkdv", "sdpa_backward_dq",
                 "sdpa_backward_main"):
        f = getattr(lib, name)
        f.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        f.restype = ctypes.c_int
    lib.sdpa_forward_ragged.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_forward_ragged.restype = ctypes.c_int
    lib.sdpa_backward_ragged.argtypes = [pp] + [vp] * 15 + [sz, vp]
    lib.sdpa_backward_ragged.restype = ctypes.c_int
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_version.restype = ctypes.c_int
    lib.sdpa_decode_paged_workspace_bytes.argtypes = [ctypes.POINTER(PagedDecode)]
    lib.sdpa_decode_paged_workspace_bytes.restype = sz
    lib.sdpa_decode_paged.argtypes = [ctypes.POINTER(PagedDecode), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sdpa_decode_paged.restype = ctypes.c_int
    if path is None:
        _LIB = lib
    return lib


def raise_status(lib, status: int):
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


class _Layout:
    """Logical (B, H, L, D) shape and (b, h, l) element strides of one operand: a padded
    (B, H, L, D) / (H, L, D) tensor, or with row offsets a packed (T, H, D) one whose batch
    stride is unused."""

    def __init__(self, t, name, offsets=None, max_len=None, B=None):
        if offsets is None:
            t4 = _as4d(t, name)
            self.shape = tuple(int(x) for x in t4.shape)
            self.strides = _strides3(t4, name)
            self.tensor = t4
            return
        if t.dim() != 3:
            raise ValueError(f"sdpa: packed {name} must be (T, H, D), got {tuple(t.shape)}")
        if t.stride(-1) != 1 and t.shape[-1] > 1:
            raise NotImplementedError(f"sdpa: {name} must have unit stride along its last dim")
        self.shape = (B, int(t.shape[1]), int(max_len), int(t.shape[2]))
        self.strides = (0, int(t.stride(1)), int(t.stride(0)))
        self.tensor = t


def _offsets(x, device, name):
    if x is None:
        return None
    if not torch.is_tensor(x):
        x = torch.tensor(x, dtype=torch.int32)
    x = x.reshape(-1)
    if x.numel() < 2:
        raise ValueError(f"sdpa: {name} needs B + 1 >= 2 entries, got {x.numel()}")
    return x.to(device=device, dtype=torch.int32).contiguous()


def _max_len(max_len, lens, offsets):
    """The padded length of a ragged side: given, or the longest batch (read back from the
    device, which synchronises)."""
    if max_len is not None:
        return int(max_len)
    ls = lens if lens is not None else offsets[1:] - offsets[:-1]
    return max(int(ls.max().item()), 0)


def _ragged_batch(q, offsets_q, offsets_kv):
    B = None
    for off in (offsets_q, offsets_kv):
        if off is not None:
            if B is not None and off.numel() - 1 != B:
                raise ValueError("sdpa: offsets_q and offsets_kv give different batch sizes")
            B = off.numel() - 1
    return B


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


def _unaliased(t: torch.Tensor) -> torch.Tensor:
    """t itself, or a contiguous copy when a dimension of size > 1 has stride 0."""
    if any(st == 0 and n > 1 for st, n in zip(t.stride(), t.shape)):
        return t.contiguous()
    return t


def _grad_like(t: torch.Tensor, zero: bool) -> torch.Tensor:
    """A gradient buffer with t's shape and strides, zero-filled when ``zero``."""
    g = torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)
    return g.zero_() if zero else g


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ``is_causal`` values (the C ABI's sdpa_causal): False/0 none, True/1 top-left diagonal
# (key j visible to query i iff j <= i), 2 bottom-right diagonal (iff j <= i + len_kv - len_q
# of the batch: a prefill chunk against its KV cache).
CAUSAL_TOP_LEFT = 1
CAUSAL_BOTTOM_RIGHT = 2


def causal_code(is_causal) -> int:
    code = int(is_causal)
    if code not in (0, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT):
        raise ValueError("sdpa: is_causal must be False/True (0/1) or 2 (bottom-right)")
    return code


def make_problem(q, k, v, o_strides, mask_strides, scale, is_causal, sliding_window=0) -> Problem:
    """q, k, v are tensors (B, H, L, D) or ``_Layout``s."""
    q, k, v = (x if isinstance(x, _Layout) else _Layout(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v")))
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
    p.dtype = _dtype_code(q.tensor)
    p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.Dqk, p.Dv = B, Hq, Hkv, Lq, Lk, Dqk, Dv
    p.q_stride[:] = q.strides
    p.k_stride[:] = k.strides
    p.v_stride[:] = v.strides
    p.o_stride[:] = o_strides
    p.mask_stride[:] = mask_strides
    p.scale = math.nan if scale is None else float(scale)
    p.is_causal = causal_code(is_causal)
    p.sliding_window = int(sliding_window)
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


class ForwardCall:
    """Marshalled forward: outputs ``o``, ``lse`` and the workspace are allocated once;
    ``launch()`` enqueues the kernels on the current stream with the cached arguments.

    Ragged (packed) sequences: with ``offsets_q`` ((B + 1) starting rows) q is a packed
    (T, Hq, D) tensor and o is returned packed the same way; with ``offsets_kv`` k and v are
    packed (T, Hkv, D).  Lengths are ``seq_lens_*`` when given, else the offset differences;
    ``max_seqlen_*`` is the padded length (computed from the lengths, with a device read,
    when not given).  Rows of ``o`` outside every batch are left as allocated."""

    def __init__(self, q, k, v, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                 seq_lens_kv=None, return_lse=True, offsets_q=None, offsets_kv=None,
                 max_seqlen_q=None, max_seqlen_kv=None, sliding_window=0, noalloc=False):
        self.lib = load_library()
        self.ragged = offsets_q is not None or offsets_kv is not None
        if noalloc and self.ragged:
            raise ValueError("sdpa: the no-allocation forward takes padded (B, H, L, D) tensors")
        self.squeeze = q.dim() == 3 and not self.ragged
        _check_io(q, k, v, *([mask] if mask is not None else []))
        dev = q.device
        oq, ok = _offsets(offsets_q, dev, "offsets_q"), _offsets(offsets_kv, dev, "offsets_kv")
        B = _ragged_batch(q, oq, ok)
        lq = _lens(seq_lens_q, B if B is not None else _as4d(q, "q").shape[0], dev, "seq_lens_q")
        lk = _lens(seq_lens_kv, B if B is not None else _as4d(q, "q").shape[0], dev, "seq_lens_kv")
        qL = _Layout(q, "q", oq, _max_len(max_seqlen_q, lq, oq) if oq is not None else None, B)
        kL = _Layout(k, "k", ok, _max_len(max_seqlen_kv, lk, ok) if ok is not None else None, B)
        vL = _Layout(v, "v", ok, kL.shape[2], B)
        B, Hq, Lq, _ = qL.shape
        Lk, Dv = kL.shape[2], vL.shape[3]
        if oq is not None:
            # rows outside every batch are not written by the library: zeros there
            self.o = torch.zeros((q.shape[0], Hq, Dv), dtype=q.dtype, device=dev)
            o_st = (0, Dv, Hq * Dv)
        else:
            self.o = torch.empty((B, Hq, Lq, Dv), dtype=q.dtype, device=dev)
            o_st = _strides3(self.o, "o")
        self.lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=dev) if return_lse else None
        m, mst = _mask4d(mask, B, Hq, Lq, Lk)
        self.p = make_problem(qL, kL, vL, o_st, mst, scale, is_causal, sliding_window)
        self._keep = (qL.tensor, kL.tensor, vL.tensor, m, lq, lk, oq, ok)
        self.device = dev
        ptrs = [_vp(qL.tensor), _vp(kL.tensor), _vp(vL.tensor), _vp(m), _vp(lq), _vp(lk)]
        if noalloc:
            # sdpa_forward_noalloc: the library's built-in scratch replaces the workspace
            self.ws = None
            self.args = [ctypes.byref(self.p), *ptrs, _vp(self.o), _vp(self.lse)]
            self.fn = self.lib.sdpa_forward_noalloc
            return
        nws = self.lib.sdpa_forward_workspace_bytes(ctypes.byref(self.p))
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        if self.ragged:
            ptrs += [_vp(oq), _vp(ok)]
        self.args = [ctypes.byref(self.p), *ptrs, _vp(self.o), _vp(self.lse), _vp(self.ws), nws]
        self.fn = self.lib.sdpa_forward_ragged if self.ragged else self.lib.sdpa_forward

    def launch(self):
        stream = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        st = self.fn(*self.args, stream)
        if st != SDPA_OK:
            raise_status(self.lib, st)

    def result(self):
        o, lse = self.o, self.lse
        if self.squeeze:
            o = o.squeeze(0)
            lse = lse.squeeze(0) if lse is not None else None
        return o, lse


class BackwardCall:
    """Marshalled backward: dq, dk, dv and the workspace are allocated once; ``launch()``
    runs all stages, ``launch(stage)`` one of "prep", "dkdv", "dq", "main" (dkdv and dq in
    one call; prep must precede the others).  Ragged arguments as in ``ForwardCall`` (o and dO then packed like q; only
    the whole backward is offered)."""

    def __init__(self, q, k, v, o, dO, lse, mask=None, scale=None, is_causal=False,
                 seq_lens_q=None, seq_lens_kv=None, offsets_q=None, offsets_kv=None,
                 max_seqlen_q=None, max_seqlen_kv=None, sliding_window=0, ds_buffer=True):
        self.lib = load_library()
        self.ragged = offsets_q is not None or offsets_kv is not None
        self.squeeze = q.dim() == 3 and not self.ragged
        _check_io(q, k, v, o, dO, *([mask] if mask is not None else []))
        dev = q.device
        oq, ok = _offsets(offsets_q, dev, "offsets_q"), _offsets(offsets_kv, dev, "offsets_kv")
        B = _ragged_batch(q, oq, ok)
        lq = _lens(seq_lens_q, B if B is not None else _as4d(q, "q").shape[0], dev, "seq_lens_q")
        lk = _lens(seq_lens_kv, B if B is not None else _as4d(q, "q").shape[0], dev, "seq_lens_kv")
        # dq, dk, dv take the strides of q, k, v: an operand that repeats memory along a
        # dimension (stride 0, an expanded view) is copied first, or several heads or
        # batches would write their gradients into the same elements
        q, k, v = _unaliased(q), _unaliased(k), _unaliased(v)
        qL = _Layout(q, "q", oq, _max_len(max_seqlen_q, lq, oq) if oq is not None else None, B)
        kL = _Layout(k, "k", ok, _max_len(max_seqlen_kv, lk, ok) if ok is not None else None, B)
        vL = _Layout(v, "v", ok, kL.shape[2], B)
        B, Hq, Lq, _ = qL.shape
        Lk, Dv = kL.shape[2], vL.shape[3]
        if oq is not None:
            want = (q.shape[0], Hq, Dv)
        else:
            o, dO = _as4d(o, "o"), _as4d(dO, "dO")
            want = (B, Hq, Lq, Dv)
        if tuple(o.shape) != want or dO.shape != o.shape:
            raise ValueError(f"sdpa: o and dO must be {want}")
        if o.stride() != dO.stride():
            dO = dO.contiguous()
            o = o.contiguous()
        if lse.dim() == 2:
            lse = lse.unsqueeze(0)
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq):
            raise ValueError("sdpa: lse must be float32 (B, Hq, Lq)")
        lse = lse.contiguous()
        if oq is not None:
            if o.stride(-1) != 1:
                raise NotImplementedError("sdpa: o must have unit stride along its last dim")
            o_st = (0, int(o.stride(1)), int(o.stride(0)))
        else:
            o_st = _strides3(o, "o")
        m, mst = _mask4d(mask, B, Hq, Lq, Lk)
        self.p = make_problem(qL, kL, vL, o_st, mst, scale, is_causal, sliding_window)
        qt, kt, vt = qL.tensor, kL.tensor, vL.tensor
        # a packed (ragged) side leaves the rows outside every batch unwritten: zeros there
        self.dq = _grad_like(qt, oq is not None)
        self.dk = _grad_like(kt, ok is not None)
        self.dv = _grad_like(vt, ok is not None)
        # the full workspace holds the dS buffer (d = 128, bf16): dQ is then formed from the
        # dK/dV pass's dS; ds_buffer=False passes the least workspace (dQ recomputed)
        ws_bytes = (self.lib.sdpa_backward_workspace_bytes if ds_buffer
                    else self.lib.sdpa_backward_workspace_bytes_min)
        nws = ws_bytes(ctypes.byref(self.p))
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self._keep = (qt, kt, vt, o, dO, lse, m, lq, lk, oq, ok)
        self.device = dev
        ptrs = [_vp(qt), _vp(kt), _vp(vt), _vp(o), _vp(dO), _vp(lse), _vp(m), _vp(lq), _vp(lk)]
        if self.ragged:
            ptrs += [_vp(oq), _vp(ok)]
        self.args = [ctypes.byref(self.p), *ptrs, _vp(self.dq), _vp(self.dk), _vp(self.dv),
                     _vp(self.ws), nws]
        if self.ragged:
            self.fns = {"all": self.lib.sdpa_backward_ragged}
        else:
            self.fns = {"all": self.lib.sdpa_backward, "prep": self.lib.sdpa_backward_prep,
                        "dkdv": self.lib.sdpa_backward_dkdv, "dq": self.lib.sdpa_backward_dq,
                        "main": self.lib.sdpa_backward_main}

    def launch(self, stage: str = "all"):
        if stage not in self.fns:
            raise ValueError(f"sdpa: backward stage {stage!r} is not offered here ({sorted(self.fns)})")
        stream = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        st = self.fns[stage](*self.args, stream)
        if st != SDPA_OK:
            raise_status(self.lib, st)

    def result(self):
        g = (self.dq, self.dk, self.dv)
        if self.squeeze:
            g = tuple(t.squeeze(0) for t in g)
        return g


def sdpa_forward(q, k, v, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                 seq_lens_kv=None, return_lse=True, offsets_q=None, offsets_kv=None,
                 max_seqlen_q=None, max_seqlen_kv=None, sliding_window=0):
    """O (and LSE) of scaled dot-product attention.  q (B,Hq,Lq,D), k/v (B,Hkv,Lk,D), or
    packed (T, H, D) with ``offsets_q`` / ``offsets_kv`` (see ``ForwardCall``).
    ``sliding_window`` W > 0 (with a causal diagonal): each row sees the last W keys up to
    its diagonal."""
    call = ForwardCall(q, k, v, mask, scale, is_causal, seq_lens_q, seq_lens_kv, return_lse,
                       offsets_q, offsets_kv, max_seqlen_q, max_seqlen_kv, sliding_window)
    call.launch()
    o, lse = call.result()
    return (o, lse) if return_lse else o


def sdpa_forward_noalloc(q, k, v, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                         seq_lens_kv=None, sliding_window=0):
    """(O, LSE) like ``sdpa_forward``, through the C ABI's ``sdpa_forward_noalloc``: the
    library uses its built-in per-GPU scratch where the decode needs a workspace (see
    include/sdpa.h for its limit); only the outputs are allocated here."""
    call = ForwardCall(q, k, v, mask, scale, is_causal, seq_lens_q, seq_lens_kv,
                       sliding_window=sliding_window, noalloc=True)
    call.launch()
    return call.result()


def sdpa_backward(q, k, v, o, dO, lse, mask=None, scale=None, is_causal=False, seq_lens_q=None,
                  seq_lens_kv=None, offsets_q=None, offsets_kv=None, max_seqlen_q=None,
                  max_seqlen_kv=None, sliding_window=0):
    """(dQ, dK, dV) from the forward's o and lse and the output gradient dO (same
    problem, mask, causal flag, window and lengths as the forward)."""
    call = BackwardCall(q, k, v, o, dO, lse, mask, scale, is_causal, seq_lens_q, seq_lens_kv,
                        offsets_q, offsets_kv, max_seqlen_q, max_seqlen_kv, sliding_window)
    call.launch()
    return call.result()


class PagedDecodeCall:
    """Marshalled single-query decode against a paged KV cache (see ``sdpa_decode_paged`` in
    include/sdpa.h): q (B, Hq, D); k_pages, v_pages (num_pages, Hkv, page_size, D);
    page_table (B, max_pages) int32; seq_lens_kv (B) int32; all on one GPU.
    ``sliding_window`` W > 0 attends to the last W keys of each sequence only."""

    def __init__(self, q, k_pages, v_pages, page_table, seq_lens_kv, scale=None, return_lse=True,
                 sliding_window=0):
        self.lib = load_library()
        if q.dim() == 4 and q.shape[2] == 1:
            q = q[:, :, 0]
        if q.dim() != 3 or k_pages.dim() != 4 or v_pages.dim() != 4:
            raise ValueError("sdpa_decode_paged: q (B, Hq, D), k/v pages (num_pages, Hkv, page_size, D)")
        _check_io(q, k_pages, v_pages)
        B, Hq, D = q.shape
        num_pages, Hkv, page_size, Dk = k_pages.shape
        if tuple(v_pages.shape) != tuple(k_pages.shape) or Dk != D:
            raise ValueError("sdpa_decode_paged: k/v pages must share one shape with width D")
        if page_table.dim() != 2 or page_table.shape[0] != B:
            raise ValueError("sdpa_decode_paged: page_table must be (B, max_pages)")
        for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages")):
            if t.stride(-1) != 1:
                raise ValueError(f"sdpa_decode_paged: {n} must have unit stride along D")
        self.page_table = page_table.to(device=q.device, dtype=torch.int32).contiguous()
        self.lens = _lens(seq_lens_kv, B, q.device, "seq_lens_kv")
        if self.lens is None:
            raise ValueError("sdpa_decode_paged: seq_lens_kv is required")
        self.o = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
        p = PagedDecode()
        p.B, p.Hq, p.Hkv, p.D = B, Hq, Hkv, D
        p.page_size, p.num_pages, p.max_pages = page_size, num_pages, self.page_table.shape[1]
        p.q_stride[:] = (q.stride(0), q.stride(1))
        p.o_stride[:] = (self.o.stride(0), self.o.stride(1))
        p.k_stride[:] = (k_pages.stride(0), k_pages.stride(1), k_pages.stride(2))
        p.v_stride[:] = (v_pages.stride(0), v_pages.stride(1), v_pages.stride(2))
        p.scale = math.nan if scale is None else float(scale)
        p.sliding_window = int(sliding_window)
        self.p = p
        nws = self.lib.sdpa_decode_paged_workspace_bytes(ctypes.byref(p))
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device)
        self._keep = (q, k_pages, v_pages)
        self.device = q.device
        self.args = [ctypes.byref(p), _vp(q), _vp(k_pages), _vp(v_pages), _vp(self.page_table),
                     _vp(self.lens), _vp(self.o), _vp(self.lse), _vp(self.ws), nws]

    def launch(self):
        stream = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        st = self.lib.sdpa_decode_paged(*self.args, stream)
        if st != SDPA_OK:
            raise_status(self.lib, st)

    def result(self):
        return self.o, self.lse


def sdpa_decode_paged(q, k_pages, v_pages, page_table, seq_lens_kv, scale=None, return_lse=True,
                      sliding_window=0):
    """O (B, Hq, D) (and LSE (B, Hq)) of single-query attention over a paged KV cache
    (the last ``sliding_window`` keys of each sequence only, when it is > 0)."""
    call = PagedDecodeCall(q, k_pages, v_pages, page_table, seq_lens_kv, scale, return_lse,
                           sliding_window)
    call.launch()
    o, lse = call.result()
    return (o, lse) if return_lse else o
