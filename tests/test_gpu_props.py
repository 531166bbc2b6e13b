"""GPU properties and edge cases of the HIP path (through the C ABI)."""

import numpy as np
import pytest
import torch

from gpu_common import (banner, check_grad, compare_forward, f64, gpu_backward, gpu_forward,
                        oracle_backward, oracle_forward, rel_fro, to_dev)
from scaled_dot_product_sdpa_amd import BackwardCall, ForwardCall, sdpa_backward, sdpa_forward
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

MID = WORKLOADS["gqa_causal_4k"].scaled(B=2, Hq=8, Hkv=2, Lq=700, Lk=700, seed=31)


def test_forward_and_backward_are_bitwise_repeatable():
    banner("repeatability")
    d = to_dev(make_inputs(MID))
    o1, l1 = gpu_forward(d)
    o2, l2 = gpu_forward(d)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = gpu_backward(d, o1, l1)
    g2 = gpu_backward(d, o1, l1)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_causal_equals_tril_mask():
    """is_causal and an explicit additive mask built from tril give the same result."""
    banner("causal == tril mask")
    w = MID.scaled(Hq=4, Hkv=4, D=64, Lq=300, Lk=300)
    d = to_dev(make_inputs(w))
    o1, l1 = gpu_forward(d)
    tril = torch.ones(w.Lq, w.Lk, dtype=torch.bool, device="cuda").tril()
    m = torch.zeros(w.Lq, w.Lk, device="cuda").masked_fill(~tril, float("-inf")).to(torch.bfloat16)
    d2 = dict(d, is_causal=False, mask=m.view(1, 1, w.Lq, w.Lk))
    o2, l2 = gpu_forward(d2)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4
    g1 = gpu_backward(d, o1, l1)
    g2 = gpu_backward(d2, o2, l2)
    for a, b in zip(g1, g2):
        assert rel_fro(f64(a), f64(b)) <= 1e-2


def test_gqa_equals_repeat_interleave():
    """GQA equals MHA on K/V expanded in repeat_interleave order; a shared head's dK/dV is
    the sum of the expanded heads' gradients."""
    banner("GQA == repeat_interleave")
    d = to_dev(make_inputs(MID))
    G = MID.Hq // MID.Hkv
    de = dict(d, k=d["k"].repeat_interleave(G, dim=1).contiguous(),
              v=d["v"].repeat_interleave(G, dim=1).contiguous())
    o1, l1 = gpu_forward(d)
    o2, l2 = gpu_forward(de)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    dq1, dk1, dv1 = gpu_backward(d, o1, l1)
    dq2, dk2, dv2 = gpu_backward(de, o2, l2)
    assert torch.equal(dq1, dq2)
    sk = dk2.float().view(MID.B, MID.Hkv, G, MID.Lk, MID.D).sum(2)
    sv = dv2.float().view(MID.B, MID.Hkv, G, MID.Lk, MID.D).sum(2)
    assert rel_fro(f64(dk1), f64(sk)) <= 1e-2 and rel_fro(f64(dv1), f64(sv)) <= 1e-2


def test_padding_is_never_read(orc):
    """With length arrays, NaN in q/k/v/dO rows past the lengths changes nothing."""
    banner("NaN-poisoned padding (prefill, fwd + bwd)")
    w = MID.scaled(lens="qkv", len_range=(50, 700), causal=False, seed=33)
    inp = make_inputs(w)
    d = to_dev(inp)
    o1, l1 = gpu_forward(d)
    g1 = gpu_backward(d, o1, l1)
    pois = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in d.items()}
    for b, n in enumerate(inp["len_kv"].tolist()):
        for name in ("q", "k", "v", "dO"):
            pois[name][b, :, n:] = float("nan")
    o2, l2 = gpu_forward(pois)
    g2 = gpu_backward(pois, o2, l2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o1, l1, o_ref, lse_ref)


def test_zero_lengths_and_empty_batches(orc):
    """A batch with length 0 gives O = 0, LSE = -inf and zero gradients."""
    banner("zero lengths")
    w = MID.scaled(B=3, lens="qkv", len_range=(0, 0), seed=34, causal=True)
    inp = make_inputs(w)
    inp["len_q"] = torch.tensor([0, 300, 700], dtype=torch.int32)
    inp["len_kv"] = torch.tensor([0, 123, 700], dtype=torch.int32)
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    dq, dk, dv = gpu_backward(d, o, lse)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(dq[0] == 0) and torch.all(dk[0] == 0) and torch.all(dv[0] == 0)
    assert torch.all(dk[1, :, 123:] == 0) and torch.all(dq[1, :, 300:] == 0)
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o, lse, o_ref, lse_ref)
    rq, rk, rv, _ = oracle_backward(orc, inp)
    for g, r, n in zip((dq, dk, dv), (rq, rk, rv), ("dQ", "dK", "dV")):
        check_grad(f64(g), r, torch.bfloat16, n)


def test_empty_key_sequence():
    """Lk = 0: every row is empty (O = 0, LSE = -inf); Lq = 0 is a no-op."""
    banner("Lk = 0 / Lq = 0")
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = sdpa_forward(q, k, k)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    kk = torch.randn(1, 2, 7, 64, device="cuda").to(torch.bfloat16)
    o0, l0 = sdpa_forward(q0, kk, kk)
    dq, dk, dv = sdpa_backward(q0, kk, kk, o0, o0, l0)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.all(dk == 0) and torch.all(dv == 0)


def test_strided_bshd_layout(orc):
    """Inputs in (B, S, H, D) memory order (strided views) give the same result, forward and
    backward (the gradients are written with the strides of q, k, v; at d = 128 the backward
    forms dQ from the stored dS)."""
    banner("BSHD strided layout")
    w = MID.scaled(Hq=4, Hkv=2, Lq=200, Lk=200, seed=35)
    inp = make_inputs(w)
    d = to_dev(inp)
    o1, l1 = gpu_forward(d)
    ds = dict(d)
    for n in ("q", "k", "v", "dO"):
        ds[n] = d[n].transpose(1, 2).contiguous().transpose(1, 2)  # BSHD storage, BHSD view
    o2, l2 = gpu_forward(ds)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = gpu_backward(d, o1, l1)
    g2 = gpu_backward(ds, o2, l2)
    for a, b in zip(g1, g2):
        assert a.shape == b.shape and torch.equal(a, b.contiguous())
    assert g2[0].stride() == ds["q"].stride() and g2[1].stride() == ds["k"].stride()


def test_graph_replay_matches_eager():
    """A HIP graph of the forward and backward replays to the eager result every time,
    with eager work and synchronisations between replays."""
    banner("graph replay")
    d = to_dev(make_inputs(MID))
    fc = ForwardCall(d["q"], d["k"], d["v"], None, d["scale"], True)
    fc.launch()
    torch.cuda.synchronize()
    bc = BackwardCall(d["q"], d["k"], d["v"], fc.o, d["dO"], fc.lse, None, d["scale"], True)

    def step():
        fc.launch()
        bc.launch()

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (fc.o, fc.lse, bc.dq, bc.dk, bc.dv)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (fc.o, fc.lse, bc.dq, bc.dk, bc.dv):
            t.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (fc.o, fc.lse, bc.dq, bc.dk, bc.dv)):
            assert torch.equal(a, b), f"replay {rep} differs"


@pytest.mark.parametrize("D,mask", [(64, False), (64, True), (128, False), (128, True)])
def test_backward_stages_equal_whole(D, mask):
    """prep + dkdv + dq as separate calls, prep + main, and the whole backward give the same
    gradients bit for bit (at d = 64 without a mask "main" runs both passes in one launch).
    At d = 128 with the full workspace the dkdv stage stores dS and the dq stage forms dQ
    from it; with the least workspace dq recomputes S, P and dP: the stages equal the whole
    call in either mode, and dK, dV are the same bits in both."""
    banner(f"backward stages d={D} mask={mask}")
    base = WORKLOADS["padded_mask_2k"] if mask else WORKLOADS["gqa_causal_4k"]
    w = base.scaled(B=2, Hq=4, Hkv=2, Lq=300, Lk=300, D=D, seed=36, len_range=(100, 300))
    d = to_dev(make_inputs(w))
    fc = ForwardCall(d["q"], d["k"], d["v"], d["mask"], d["scale"], w.causal, d["len_q"], d["len_kv"])
    fc.launch()
    bc = BackwardCall(d["q"], d["k"], d["v"], fc.o, d["dO"], fc.lse, d["mask"], d["scale"], w.causal,
                      d["len_q"], d["len_kv"])
    bmin = BackwardCall(d["q"], d["k"], d["v"], fc.o, d["dO"], fc.lse, d["mask"], d["scale"], w.causal,
                        d["len_q"], d["len_kv"], ds_buffer=False)
    for call in (bc, bmin):
        results = []
        for stages in (["all"], ["prep", "dkdv", "dq"], ["prep", "main"]):
            for t in (call.dq, call.dk, call.dv):
                t.fill_(7.0)
            for st in stages:
                call.launch(st)
            torch.cuda.synchronize()
            results.append([t.clone() for t in (call.dq, call.dk, call.dv)])
        for r in results[1:]:
            for a, b in zip(results[0], r):
                assert torch.equal(a, b)
    # dK, dV do not depend on how dQ is formed (at d = 64 nothing differs)
    for a, b in zip((bc.dk, bc.dv) if D == 128 else (bc.dq, bc.dk, bc.dv),
                    (bmin.dk, bmin.dv) if D == 128 else (bmin.dq, bmin.dk, bmin.dv)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
def test_stale_lds_does_not_leak(D):
    """LDS left full of NaN by an earlier launch of the same kernels (all-NaN inputs, so
    every tile buffer holds NaN rows) changes nothing in the next launch: the gradients
    equal those computed after an all-zero launch, bit for bit, and are finite.  The
    pipelined backward kernels multiply zero weights by a buffer that no tile has filled
    yet in their first block, so that buffer must not hold NaN or Inf."""
    banner(f"stale LDS (D={D})")
    w = MID.scaled(D=D, Hq=8, Hkv=2, Lq=700, Lk=700, seed=36)
    d = to_dev(make_inputs(w))
    shape = (8, 16, 1024, D)  # many workgroups per CU, several query/key tiles each

    def fill(value):
        t = torch.full(shape, value, device="cuda", dtype=torch.bfloat16)
        f = dict(q=t, k=t, v=t, dO=t, scale=D ** -0.5, is_causal=False)
        o, lse = gpu_forward(f)
        gpu_backward(f, o, lse)

    fill(0.0)
    o1, l1 = gpu_forward(d)
    g1 = gpu_backward(d, o1, l1)
    fill(float("nan"))
    o2, l2 = gpu_forward(d)
    g2 = gpu_backward(d, o2, l2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.isfinite(a).all() and torch.equal(a, b)


def test_bottom_right_chunk_equals_full_causal_rows():
    """A prefill chunk (the last c queries against the whole KV cache, bottom-right
    diagonal) reproduces the last c rows of the top-left causal forward over the full
    sequence, and their dQ; dK, dV equal the full backward's when the other rows carry no
    output gradient."""
    banner("bottom-right chunk == rows of the full causal problem")
    for D, n, c, Hq, Hkv in ((64, 700, 180, 4, 4), (128, 520, 130, 8, 2)):
        w = MID.scaled(B=2, Hq=Hq, Hkv=Hkv, Lq=n, Lk=n, D=D, seed=50 + D)
        d = to_dev(make_inputs(w))
        o_f, l_f = gpu_forward(d)
        dO_c = d["dO"].clone()
        dO_c[:, :, : n - c] = 0
        gq_f, gk_f, gv_f = gpu_backward(dict(d, dO=dO_c), o_f, l_f)
        dc = dict(d, q=d["q"][:, :, n - c:].contiguous(), dO=d["dO"][:, :, n - c:].contiguous(),
                  is_causal=2)
        o, l = gpu_forward(dc)
        gq, gk, gv = gpu_backward(dc, o, l)
        assert (o.float() - o_f[:, :, n - c:].float()).abs().max().item() <= 1e-2
        assert (l - l_f[:, :, n - c:]).abs().max().item() <= 1e-4
        assert rel_fro(f64(gq), f64(gq_f[:, :, n - c:])) <= 1e-2
        assert rel_fro(f64(gk), f64(gk_f)) <= 1e-2 and rel_fro(f64(gv), f64(gv_f)) <= 1e-2


@pytest.mark.parametrize("causal", [0, 2])
def test_decode_with_query_lengths(orc, causal):
    """Single-query decode (non-causal, or bottom-right, which sees the whole cache) with a
    query-length array: batches of query length 0 give O = 0 and LSE = -inf; the others
    match the oracle."""
    banner(f"decode with query lengths (is_causal={causal})")
    w = WORKLOADS["gqa_decode_8k"].scaled(B=4, Hq=8, Hkv=2, Lk=900, len_range=(100, 900),
                                          causal=causal, seed=55)
    inp = make_inputs(w)
    inp["len_q"] = torch.tensor([1, 0, 1, 0], dtype=torch.int32)
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    assert torch.all(o[1] == 0) and torch.all(o[3] == 0)
    assert torch.all(torch.isneginf(lse[1])) and torch.all(torch.isneginf(lse[3]))
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("D,dtype,causal,Lq", [(64, "bf16", 1, 500), (128, "bf16", 2, 300),
                                               (64, "f32", 1, 130), (128, "bf16", 2, 1)])
def test_window_covering_every_key_changes_nothing(D, dtype, causal, Lq):
    """A sliding window at least as wide as the key sequence skips no tile and cuts no key,
    so every output is bit-identical to the plain causal problem's (prefill, fp32, decode)."""
    banner(f"window >= Lk is the causal problem: D={D} {dtype} causal={causal} Lq={Lq}")
    w = MID.scaled(B=2, Hq=4, Hkv=2, Lq=Lq, Lk=500, D=D, dtype=dtype, causal=causal, seed=59,
                   backward=Lq > 1)
    d = to_dev(make_inputs(w))
    o1, l1 = gpu_forward(d)
    dw = dict(d, window=w.Lk)
    o2, l2 = gpu_forward(dw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if w.backward:
        for a, b in zip(gpu_backward(d, o1, l1), gpu_backward(dw, o2, l2)):
            assert torch.equal(a, b)


def test_window_equals_band_mask():
    """is_causal with a sliding window of W keys and an explicit additive band mask
    (-inf outside i - W < j <= i) give the same result."""
    banner("window == band mask")
    w = MID.scaled(Hq=2, Hkv=2, D=128, Lq=400, Lk=400, seed=60)
    W = 97
    d = to_dev(make_inputs(w))
    dw = dict(d, window=W)
    o1, l1 = gpu_forward(dw)
    i = torch.arange(w.Lq, device="cuda").view(-1, 1)
    j = torch.arange(w.Lk, device="cuda").view(1, -1)
    band = (j <= i) & (j > i - W)
    m = torch.zeros(w.Lq, w.Lk, device="cuda").masked_fill(~band, float("-inf")).to(torch.bfloat16)
    d2 = dict(d, is_causal=False, mask=m.view(1, 1, w.Lq, w.Lk))
    o2, l2 = gpu_forward(d2)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2
    assert (l1 - l2).abs().max().item() <= 1e-4
    for a, b in zip(gpu_backward(dw, o1, l1), gpu_backward(d2, o2, l2)):
        assert rel_fro(f64(a), f64(b)) <= 1e-2
