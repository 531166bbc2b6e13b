"""The forward without allocation (sdpa_forward_noalloc in include/sdpa.h), on the GPU
through the C ABI: its results equal sdpa_forward's bit for bit (same kernels; the decode
partials live in the library's built-in scratch instead of a caller workspace), on two
calls in a row, the second smaller than the first, and on a prefill problem (no
workspace at all).  The scratch keeps the last call's contents, which must not leak into
a later, smaller call."""

import pytest
import torch

from gpu_common import banner, to_dev
from scaled_dot_product_sdpa_amd import sdpa_forward, sdpa_forward_noalloc
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _both(inp):
    args = dict(scale=inp["scale"], is_causal=inp["is_causal"], seq_lens_q=inp["len_q"],
                seq_lens_kv=inp["len_kv"], sliding_window=inp.get("window", 0))
    o1, l1 = sdpa_forward(inp["q"], inp["k"], inp["v"], mask=inp["mask"], **args)
    o2, l2 = sdpa_forward_noalloc(inp["q"], inp["k"], inp["v"], mask=inp["mask"], **args)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_decode_two_calls_second_smaller():
    big = WORKLOADS["gqa_decode_8k"].scaled(B=16, Hq=32, Hkv=8, Lk=4096, len_range=(1000, 4096), seed=201)
    small = WORKLOADS["gqa_decode_8k"].scaled(B=3, Hq=8, Hkv=2, Lk=700, len_range=(1, 700), seed=202)
    for name, w in (("large", big), ("small", small)):
        banner(f"noalloc decode {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lk={w.Lk}")
        inp = to_dev(make_inputs(w))
        o1, l1, o2, l2 = _both(inp)
        assert torch.isfinite(o2).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), name


def test_noalloc_prefill_and_full_decode():
    w = WORKLOADS["gqa_causal_4k"].scaled(B=1, Hq=4, Hkv=2, Lq=300, Lk=300, seed=203)
    banner("noalloc prefill")
    o1, l1, o2, l2 = _both(to_dev(make_inputs(w)))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the full-size decode workload fits the scratch
    banner("noalloc decode at full size")
    inp = make_inputs(WORKLOADS["gqa_decode_8k"], device="cuda")
    o1, l1, o2, l2 = _both(inp)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
