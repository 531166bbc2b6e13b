"""The backward's dS buffer (d = 128, bf16): with the full workspace the dK/dV pass stores
bf16 dS blocks and dQ = scale dS K is formed from them; with the least workspace dQ runs as
its own pass, recomputing S, P and dP.  dK and dV are the same bits either way, dQ agrees
within rounding, both agree with the oracle, and the reader touches no block the dK/dV pass
did not write (a workspace filled with NaN changes nothing)."""

import pytest
import torch

from gpu_common import banner, compare_backward, f64, oracle_backward, rel_fro, to_dev
from scaled_dot_product_sdpa_amd import BackwardCall, ForwardCall
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

GQA = WORKLOADS["gqa_causal_4k"]
PAD = WORKLOADS["padded_mask_2k"]

# (name, workload): top-left and bottom-right diagonals, sliding windows, lengths with a
# mask, no diagonal with Lq != Lk, ragged tails of the 32-row blocks and 128-key groups
CASES = [
    ("causal_gqa", GQA.scaled(B=2, Hq=8, Hkv=2, Lq=333, Lk=333, seed=61)),
    ("br_chunk", GQA.scaled(B=2, Hq=4, Hkv=1, Lq=90, Lk=517, causal=2, seed=62)),
    ("br_long_q", GQA.scaled(B=1, Hq=4, Hkv=2, Lq=300, Lk=130, causal=2, seed=63)),
    ("window_tl", GQA.scaled(B=1, Hq=4, Hkv=2, Lq=400, Lk=400, window=45, seed=64)),
    ("window_br", GQA.scaled(B=2, Hq=4, Hkv=4, Lq=200, Lk=450, causal=2, window=100, seed=65)),
    ("padded_mask", PAD.scaled(B=3, Hq=4, Hkv=4, Lq=260, Lk=260, len_range=(1, 260), seed=66)),
    ("noncausal", GQA.scaled(B=1, Hq=4, Hkv=2, Lq=100, Lk=270, causal=0, seed=67)),
]


def _run(d, o, lse, w, ds_buffer, poison=False):
    bc = BackwardCall(d["q"], d["k"], d["v"], o, d["dO"], lse, d["mask"], d["scale"], d["is_causal"],
                      d["len_q"], d["len_kv"], sliding_window=w.window, ds_buffer=ds_buffer)
    if poison:
        bc.ws.fill_(255)  # every bf16 of the dS buffer reads as NaN until written
    bc.launch()
    torch.cuda.synchronize()
    return [t.clone() for t in bc.result()], bc.ws.numel()


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_ds_buffer_matches_recompute_and_oracle(orc, name, w):
    banner(f"dS buffer vs recomputed dQ: {name}")
    d = to_dev(make_inputs(w))
    fc = ForwardCall(d["q"], d["k"], d["v"], d["mask"], d["scale"], d["is_causal"], d["len_q"],
                     d["len_kv"], sliding_window=w.window)
    fc.launch()
    torch.cuda.synchronize()
    (dq1, dk1, dv1), n1 = _run(d, fc.o, fc.lse, w, True, poison=True)
    (dq2, dk2, dv2), n2 = _run(d, fc.o, fc.lse, w, False)
    assert n1 > n2  # the full workspace holds the buffer
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    assert torch.isfinite(dq1.float()).all()
    assert rel_fro(f64(dq1), f64(dq2)) <= 2e-3
    refs = oracle_backward(orc, d)[:3]
    # (rows with no visible key: dQ exactly 0, checked through the forward's -inf LSE)
    compare_backward(d, (dq1, dk1, dv1), refs, lse_ref=f64(fc.lse))


def test_ds_buffer_poisoned_workspace_is_bitwise_clean():
    """A NaN-filled and a zero-filled workspace give the same gradients bit for bit: every
    dS block the dQ pass reads was written by the dK/dV pass of the same call."""
    banner("dS buffer: NaN-filled workspace")
    for name, w in CASES:
        d = to_dev(make_inputs(w))
        fc = ForwardCall(d["q"], d["k"], d["v"], d["mask"], d["scale"], d["is_causal"], d["len_q"],
                         d["len_kv"], sliding_window=w.window)
        fc.launch()
        bc = BackwardCall(d["q"], d["k"], d["v"], fc.o, d["dO"], fc.lse, d["mask"], d["scale"],
                          d["is_causal"], d["len_q"], d["len_kv"], sliding_window=w.window)
        outs = []
        for fill in (0, 255):
            bc.ws.fill_(fill)
            bc.launch()
            torch.cuda.synchronize()
            outs.append([t.clone() for t in bc.result()])
        for a, b in zip(*outs):
            assert torch.equal(a, b), name


@pytest.mark.parametrize("causal,window", [(1, 0), (2, 300)])
def test_ds_buffer_eight_wave_grid(causal, window):
    """A grid large enough for the eight-wave dQ-from-dS workgroups (256 rows each, ragged
    last tile): the same gradients as the recomputing path (dK, dV bit for bit, dQ within
    rounding), with the workspace NaN-filled first.  (The oracle checks the recomputing path
    on the same shapes at reduced size; this size is beyond a quick fp64 run.)"""
    banner(f"dS buffer, eight-wave grid: causal={causal} window={window}")
    w = GQA.scaled(B=4, Hq=32, Hkv=8, Lq=1000, Lk=1000, causal=causal, window=window, seed=68)
    d = to_dev(make_inputs(w))
    fc = ForwardCall(d["q"], d["k"], d["v"], d["mask"], d["scale"], d["is_causal"], d["len_q"],
                     d["len_kv"], sliding_window=w.window)
    fc.launch()
    torch.cuda.synchronize()
    (dq1, dk1, dv1), _ = _run(d, fc.o, fc.lse, w, True, poison=True)
    (dq2, dk2, dv2), _ = _run(d, fc.o, fc.lse, w, False)
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    assert torch.isfinite(dq1.float()).all()
    assert rel_fro(f64(dq1), f64(dq2)) <= 2e-3
