"""C ABI checks that need no GPU: the library loads and exports every function that
include/sdpa.h declares, workspace sizes follow their documented formulas, and every
host-checkable bad argument returns its status code before anything is launched."""

import ctypes
import math
import re
from pathlib import Path

import pytest

import scaled_dot_product_sdpa_amd as sd
from scaled_dot_product_sdpa_amd.api import (SDPA_DTYPE_BF16, SDPA_DTYPE_F32,
                                             SDPA_ERR_INVALID_ARGUMENT, SDPA_ERR_UNSUPPORTED,
                                             SDPA_ERR_WORKSPACE_TOO_SMALL, Problem)

HEADER = Path(__file__).resolve().parent.parent / "include" / "sdpa.h"


@pytest.fixture(scope="module")
def lib():
    if not sd.LIB_PATH.exists():
        from scaled_dot_product_sdpa_amd.build import build
        build()
    return sd.load_library()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "sdpa_forward" in names and "sdpa_backward" in names
    for n in names:
        assert hasattr(lib, n), f"libsdpa.so does not export {n}"
    assert set(names) == set(sd.EXPORTS)


def _problem(dtype=SDPA_DTYPE_BF16, B=2, Hq=4, Hkv=2, Lq=16, Lk=16, D=64, scale=math.nan, causal=0):
    p = Problem()
    p.dtype = dtype
    p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.Dqk, p.Dv = B, Hq, Hkv, Lq, Lk, D, D
    p.q_stride[:] = (Hq * Lq * D, Lq * D, D)
    p.k_stride[:] = (Hkv * Lk * D, Lk * D, D)
    p.v_stride[:] = (Hkv * Lk * D, Lk * D, D)
    p.o_stride[:] = (Hq * Lq * D, Lq * D, D)
    p.mask_stride[:] = (0, 0, Lk)
    p.scale = scale
    p.is_causal = causal
    return p


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def _fwd(lib, p, q=FAKE, k=FAKE, v=FAKE, mask=None, o=FAKE, lse=FAKE, ws=None, nws=0):
    return lib.sdpa_forward(ctypes.byref(p), q, k, v, mask, None, None, o, lse, ws, nws, None)


def _bwd(lib, p, lse=FAKE, dq=FAKE, ws=FAKE, nws=1 << 20, stage="sdpa_backward"):
    f = getattr(lib, stage)
    return f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, lse, None, None, None, dq, FAKE, FAKE,
             ws, nws, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "dtype", 7), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "B", 0), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "Hq", 3), SDPA_ERR_INVALID_ARGUMENT),          # Hq % Hkv != 0
    (lambda p: setattr(p, "Lk", -1), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "scale", -0.5), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "scale", 0.0), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "scale", math.inf), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "Dv", 32), SDPA_ERR_UNSUPPORTED),              # Dqk != Dv
    (lambda p: (setattr(p, "Dqk", 96), setattr(p, "Dv", 96)), SDPA_ERR_UNSUPPORTED),
    (lambda p: p.k_stride.__setitem__(2, 60), SDPA_ERR_UNSUPPORTED),     # not a multiple of 8
    (lambda p: p.q_stride.__setitem__(1, -64), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: p.o_stride.__setitem__(2, 32), SDPA_ERR_INVALID_ARGUMENT),  # rows overlap
    (lambda p: p.v_stride.__setitem__(2, 1 << 24), SDPA_ERR_UNSUPPORTED),  # 64-row tile > 2 GiB
    (lambda p: p.mask_stride.__setitem__(2, 1 << 24), SDPA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "is_causal", 3), SDPA_ERR_INVALID_ARGUMENT),    # 0, 1 or 2 only
    (lambda p: setattr(p, "is_causal", -1), SDPA_ERR_INVALID_ARGUMENT),
    # a sliding window is a count of keys and needs a causal diagonal to end at
    (lambda p: (setattr(p, "is_causal", 1), setattr(p, "sliding_window", -1)), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: (setattr(p, "is_causal", 0), setattr(p, "sliding_window", 16)), SDPA_ERR_INVALID_ARGUMENT),
])
def test_forward_rejects(lib, mutate, status):
    p = _problem()
    mutate(p)
    assert _fwd(lib, p) == status, lib.sdpa_last_error()
    assert lib.sdpa_last_error().decode() != ""


def test_forward_rejects_pointers(lib):
    p = _problem()
    assert _fwd(lib, p, q=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _fwd(lib, p, k=FAKE + 8) == SDPA_ERR_UNSUPPORTED       # bf16 io needs 16-byte alignment
    assert _fwd(lib, p, lse=FAKE + 2) == SDPA_ERR_UNSUPPORTED     # fp32 lse needs 4-byte alignment
    pf = _problem(dtype=SDPA_DTYPE_F32, D=32)
    assert _fwd(lib, pf, o=None) == SDPA_ERR_INVALID_ARGUMENT


def test_decode_workspace(lib):
    p = _problem(B=64, Hq=32, Hkv=8, Lq=1, Lk=8192, D=128)
    need = lib.sdpa_forward_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert _fwd(lib, p, ws=FAKE, nws=need - 1) == SDPA_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(lib, p, ws=None, nws=need) == SDPA_ERR_WORKSPACE_TOO_SMALL
    # a top-left causal single-query problem runs on the prefill kernel and needs none; a
    # bottom-right one sees its whole cache, so it is a decode and needs the same workspace
    pc = _problem(B=64, Hq=32, Hkv=8, Lq=1, Lk=8192, D=128, causal=1)
    assert lib.sdpa_forward_workspace_bytes(ctypes.byref(pc)) == 0
    pb = _problem(B=64, Hq=32, Hkv=8, Lq=1, Lk=8192, D=128, causal=2)
    assert lib.sdpa_forward_workspace_bytes(ctypes.byref(pb)) == need


def test_prefill_and_backward_workspace(lib):
    p = _problem(B=4, Hq=16, Hkv=16, Lq=1024, Lk=1024, D=64)
    assert lib.sdpa_forward_workspace_bytes(ctypes.byref(p)) == 0
    nb = lib.sdpa_backward_workspace_bytes(ctypes.byref(p))
    assert nb >= 4 * 16 * 1024 * 4 and nb % 256 == 0
    # no dS buffer at d = 64: the full and the least workspace agree
    assert lib.sdpa_backward_workspace_bytes_min(ctypes.byref(p)) == nb
    bad = _problem(Hq=3)
    assert lib.sdpa_backward_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.sdpa_backward_workspace_bytes_min(ctypes.byref(bad)) == 0


def test_backward_ds_buffer_size(lib):
    """At d = 128 (bf16) the backward workspace adds the dS block buffer: 2 KB per 32 x 32
    block, over whole 64-row query tiles and 128-key groups of every (batch, query head)."""
    p = _problem(B=2, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128, causal=1)
    nmin = lib.sdpa_backward_workspace_bytes_min(ctypes.byref(p))
    assert nmin == 2 * 2 * 32 * 4096 * 4
    assert lib.sdpa_backward_workspace_bytes(ctypes.byref(p)) == nmin + 2 * 32 * 128 * 128 * 2048
    # ragged tails round up to whole query tiles (64 rows) and key groups (128 keys)
    p = _problem(B=3, Hq=4, Hkv=2, Lq=90, Lk=130, D=128)
    nmin = lib.sdpa_backward_workspace_bytes_min(ctypes.byref(p))
    assert lib.sdpa_backward_workspace_bytes(ctypes.byref(p)) == nmin + 3 * 4 * 4 * 8 * 2048
    # over 8 GiB of blocks: no buffer (dQ is recomputed)
    p = _problem(B=8, Hq=32, Hkv=8, Lq=16384, Lk=16384, D=128, causal=1)
    assert lib.sdpa_backward_workspace_bytes(ctypes.byref(p)) == \
        lib.sdpa_backward_workspace_bytes_min(ctypes.byref(p))


@pytest.mark.parametrize("stage", ["sdpa_backward", "sdpa_backward_prep", "sdpa_backward_dkdv",
                                   "sdpa_backward_dq", "sdpa_backward_main"])
def test_backward_rejects(lib, stage):
    p = _problem()
    assert _bwd(lib, p, lse=None, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
    assert _bwd(lib, p, dq=None, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
    assert _bwd(lib, p, nws=16, stage=stage) == SDPA_ERR_WORKSPACE_TOO_SMALL
    bad = _problem(Hq=3)
    assert _bwd(lib, bad, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
    nowin = _problem()
    nowin.is_causal, nowin.sliding_window = 0, 16
    assert _bwd(lib, nowin, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
    # gradients take the strides of q, k, v: a zero batch or head stride would alias them
    for t, ax in (("q_stride", 1), ("k_stride", 0), ("v_stride", 1)):
        alias = _problem()
        getattr(alias, t)[ax] = 0
        assert _bwd(lib, alias, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
        assert "alias" in lib.sdpa_last_error().decode()
    # ... but a dimension of size 1 may have any stride
    one = _problem(B=1, Hq=1, Hkv=1)
    one.q_stride[0] = one.q_stride[1] = one.k_stride[0] = one.k_stride[1] = 0
    assert _bwd(lib, one, lse=None, stage=stage) == SDPA_ERR_INVALID_ARGUMENT
    assert "lse" in lib.sdpa_last_error().decode()


def test_noalloc_forward_rejects_before_launch(lib):
    """The no-allocation forward validates like sdpa_forward and refuses a decode whose
    partial results would not fit its built-in 16 MiB scratch, before any HIP call."""
    p = _problem(Hq=3)
    assert lib.sdpa_forward_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE,
                                    None) == SDPA_ERR_INVALID_ARGUMENT
    big = _problem(B=512, Hq=32, Hkv=8, Lq=1, Lk=8192, D=128)
    need = lib.sdpa_forward_workspace_bytes(ctypes.byref(big))
    assert need > (16 << 20)
    assert lib.sdpa_forward_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE,
                                    None) == SDPA_ERR_UNSUPPORTED
    assert "scratch" in lib.sdpa_last_error().decode()


def test_status_strings_and_version(lib):
    assert lib.sdpa_status_string(0) == b"ok"
    assert lib.sdpa_status_string(SDPA_ERR_WORKSPACE_TOO_SMALL) == b"workspace too small"
    assert lib.sdpa_version() >= 100


def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sd.sdpa_forward(q, q, q)


def _paged(B=2, Hq=8, Hkv=2, D=128, page_size=64, num_pages=10, max_pages=4):
    p = sd.PagedDecode()
    p.B, p.Hq, p.Hkv, p.D = B, Hq, Hkv, D
    p.page_size, p.num_pages, p.max_pages = page_size, num_pages, max_pages
    p.q_stride[:] = (Hq * D, D)
    p.o_stride[:] = (Hq * D, D)
    p.k_stride[:] = (Hkv * page_size * D, page_size * D, D)
    p.v_stride[:] = (Hkv * page_size * D, page_size * D, D)
    p.scale = math.nan
    return p


def _dec(lib, p, table=FAKE, lens=FAKE, ws=FAKE, nws=1 << 20):
    return lib.sdpa_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, table, lens, FAKE, FAKE, ws, nws, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda p: setattr(p, "page_size", 48), SDPA_ERR_UNSUPPORTED),   # not a multiple of 32
    (lambda p: setattr(p, "page_size", 0), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "num_pages", 0), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: setattr(p, "Hq", 3), SDPA_ERR_INVALID_ARGUMENT),      # Hq % Hkv != 0
    (lambda p: setattr(p, "Hq", 64), SDPA_ERR_UNSUPPORTED),          # 32 heads per KV head
    (lambda p: setattr(p, "D", 96), SDPA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "scale", -1.0), SDPA_ERR_INVALID_ARGUMENT),
    (lambda p: p.k_stride.__setitem__(2, 60), SDPA_ERR_UNSUPPORTED),
    (lambda p: p.v_stride.__setitem__(2, 64), SDPA_ERR_INVALID_ARGUMENT),  # rows overlap
    (lambda p: setattr(p, "sliding_window", -1), SDPA_ERR_INVALID_ARGUMENT),
])
def test_paged_decode_rejects(lib, mutate, status):
    p = _paged()
    mutate(p)  # every case fails validation, so the FAKE pointers are never used
    assert _dec(lib, p) == status
    assert lib.sdpa_decode_paged_workspace_bytes(ctypes.byref(p)) == 0


def test_paged_decode_pointers_and_workspace(lib):
    p = _paged()
    need = lib.sdpa_decode_paged_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert _dec(lib, p, table=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _dec(lib, p, lens=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _dec(lib, p, ws=FAKE, nws=need - 1) == SDPA_ERR_WORKSPACE_TOO_SMALL
    assert _dec(lib, p, ws=None, nws=need) == SDPA_ERR_WORKSPACE_TOO_SMALL


def _fwd_ragged(lib, p, off_q=FAKE, off_kv=FAKE, q=FAKE, lse=FAKE):
    return lib.sdpa_forward_ragged(ctypes.byref(p), q, FAKE, FAKE, None, None, None, off_q, off_kv,
                                   FAKE, lse, None, 0, None)


def _bwd_ragged(lib, p, off_q=FAKE, off_kv=FAKE, lse=FAKE, ws=FAKE, nws=1 << 20):
    return lib.sdpa_backward_ragged(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, lse, None, None,
                                    None, off_q, off_kv, FAKE, FAKE, FAKE, ws, nws, None)


def test_ragged_rejects(lib):
    p = _problem()
    # at least one side ragged; offsets 4-byte aligned
    assert _fwd_ragged(lib, p, off_q=None, off_kv=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _bwd_ragged(lib, p, off_q=None, off_kv=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _fwd_ragged(lib, p, off_q=FAKE + 2) == SDPA_ERR_UNSUPPORTED
    assert _bwd_ragged(lib, p, off_kv=FAKE + 1) == SDPA_ERR_UNSUPPORTED
    # the common checks still apply
    assert _fwd_ragged(lib, _problem(Hq=3)) == SDPA_ERR_INVALID_ARGUMENT
    assert _bwd_ragged(lib, p, lse=None) == SDPA_ERR_INVALID_ARGUMENT
    assert _bwd_ragged(lib, p, nws=16) == SDPA_ERR_WORKSPACE_TOO_SMALL
    assert _fwd_ragged(lib, p, q=None) == SDPA_ERR_INVALID_ARGUMENT
    assert lib.sdpa_last_error().decode() != ""


def test_ragged_backward_accepts_unused_batch_stride(lib):
    """A ragged side's batch stride is zeroed (unused); that is no gradient alias."""
    p = _problem()
    assert _bwd_ragged(lib, p, off_kv=None, lse=None) == SDPA_ERR_INVALID_ARGUMENT
    assert "lse" in lib.sdpa_last_error().decode()


def test_binding_copies_aliased_operands():
    """An expanded (stride-0) operand is copied before its gradient buffer is laid out, so
    the buffer's strides never repeat memory; packed gradients start as zeros."""
    import torch
    from scaled_dot_product_sdpa_amd.api import _grad_like, _unaliased
    k = torch.randn(1, 1, 8, 64).expand(2, 3, 8, 64)
    assert k.stride()[:2] == (0, 0)
    k2 = _unaliased(k)
    assert k2.is_contiguous() and torch.equal(k2, k)
    q = torch.randn(2, 3, 8, 64)
    assert _unaliased(q) is q
    g = _grad_like(torch.randn(10, 2, 64)[:, :, :], True)
    assert torch.count_nonzero(g) == 0


def test_ragged_ignores_batch_strides_of_ragged_sides(lib):
    """A batch stride that the padded call rejects is unused (and not checked) on a ragged
    side; the call then fails on the null q instead, before any launch."""
    p = _problem()
    p.q_stride[0] = 3
    p.o_stride[0] = 5
    assert _fwd(lib, p, q=None) == SDPA_ERR_UNSUPPORTED
    assert _fwd_ragged(lib, p, off_kv=None, q=None) == SDPA_ERR_INVALID_ARGUMENT
    p = _problem()
    p.k_stride[0] = 3
    assert _fwd(lib, p, q=None) == SDPA_ERR_UNSUPPORTED
    assert _fwd_ragged(lib, p, off_q=None, q=None) == SDPA_ERR_INVALID_ARGUMENT
    # the query side's batch stride is still checked when only the keys are ragged
    p = _problem()
    p.q_stride[0] = 3
    assert _fwd_ragged(lib, p, off_q=None, q=None) == SDPA_ERR_UNSUPPORTED
