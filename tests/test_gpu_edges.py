"""GPU parity on the edge cases of "Scaled dot-product attention (forward and backward)",
section 4 (the interface's test table): scores of order 1e4 give a clean one-hot row
(test_large_scores_do_not_overflow), the default scale is 1/sqrt(d)
(test_default_scale_is_inverse_sqrt_d), and keys that every row masks get exactly zero
weight and gradient (test_masked_keys_get_no_weight_or_gradient).  Each runs the HIP path
through the C ABI and compares it with the fp64 oracle on the same inputs."""

import numpy as np
import pytest
import torch

from gpu_common import (TOL_BF16_LSE, banner, check_grad, check_lse, compare_backward,
                        compare_forward, f64, gpu_backward, gpu_forward, oracle_backward,
                        oracle_forward, to_dev)
from scaled_dot_product_sdpa_amd import sdpa_forward
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _one_hot_inputs(B, Hq, Hkv, Lq, Lk, D, seed):
    """Scores of order 1e4 with one clear winner per row.  With scale 1/8, q carries +-800
    in its first coordinate and each key a distinct integer in [-100, 100] there (all exact
    in bf16), so a row's scores are 100 * key value (+- the O(1) dot product of the other
    coordinates): the best visible key beats the next by about 100."""
    assert Lk <= 201
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, Lq, D, generator=g) * 0.05
    k = torch.randn(B, Hkv, Lk, D, generator=g) * 0.05
    v = torch.randn(B, Hkv, Lk, D, generator=g)
    sign = torch.where(torch.rand(B, Hq, Lq, generator=g) < 0.5, -1.0, 1.0)
    q[..., 0] = 800.0 * sign
    for b in range(B):
        for h in range(Hkv):
            k[b, h, :, 0] = (torch.randperm(201, generator=g)[:Lk] - 100).float()
    dO = torch.randn(B, Hq, Lq, D, generator=g)
    bf = lambda t: t.to(torch.bfloat16)
    return dict(q=bf(q), k=bf(k), v=bf(v), dO=bf(dO), mask=None, len_q=None, len_kv=None,
                scale=0.125, is_causal=False, window=0)


def _lse_tol(lse_ref):
    """1e-3, widened by four fp32 ulps of the LSE itself: at |LSE| ~ 1e4 one ulp of the
    fp32 output is already 1e-3."""
    fin = np.abs(lse_ref[np.isfinite(lse_ref)])
    big = fin.max() if fin.size else 0.0
    return TOL_BF16_LSE + 4 * float(np.spacing(np.float32(big)))


@pytest.mark.parametrize("D,causal,Lq", [(64, False, 200), (128, False, 200), (64, True, 200),
                                         (128, True, 200), (128, False, 1), (64, False, 1)])
def test_large_scores_give_one_hot(orc, D, causal, Lq):
    """Lq = 1 runs the split-KV decode kernels, the others the prefill kernels."""
    inp = _one_hot_inputs(B=2, Hq=4, Hkv=2, Lq=Lq, Lk=200, D=D, seed=80 + D + Lq)
    inp["is_causal"] = causal
    banner(f"one-hot D={D} causal={causal} Lq={Lq}")
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    o_ref, lse_ref = oracle_forward(orc, inp)
    # the oracle's rows are one-hot: O is the winning key's value row itself, exactly
    G = inp["q"].shape[1] // inp["k"].shape[1]
    v = f64(inp["v"])
    q0 = f64(inp["q"])[..., 0]
    k0 = f64(inp["k"])[..., 0]
    og = f64(o)
    for b in range(o_ref.shape[0]):
        for h in range(o_ref.shape[1]):
            for i in range(o_ref.shape[2]):
                vis = k0[b, h // G, : (i + 1 if causal else k0.shape[2])]
                j = int(np.argmax(vis * np.sign(q0[b, h, i])))
                assert np.abs(o_ref[b, h, i] - v[b, h // G, j]).max() < 1e-12
                assert np.array_equal(og[b, h, i], v[b, h // G, j]), (b, h, i, j)
    check_lse(f64(lse), lse_ref, _lse_tol(lse_ref))
    if Lq > 1:
        grads = gpu_backward(d, o, lse)
        for t in grads:
            assert torch.isfinite(t).all()
        _, _, dv_ref, _ = oracle_backward(orc, inp)
        # P is one-hot, so dS = P o (dP - D) vanishes and dV = P^T dO is the only gradient
        check_grad(f64(grads[2]), dv_ref, torch.bfloat16, "dV")
        assert float(grads[0].float().abs().max()) < 1e-2 and float(grads[1].float().abs().max()) < 1e-2


DEFAULT_SCALE_CASES = {
    "d64_causal": WORKLOADS["mha_causal_1k"].scaled(B=2, Hq=2, Hkv=2, Lq=150, Lk=150, seed=90),
    "d128_gqa_causal": WORKLOADS["gqa_causal_4k"].scaled(B=1, Hq=4, Hkv=2, Lq=200, Lk=200, seed=91),
    "d128_mask_lens": WORKLOADS["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=2, Lq=140, Lk=140,
                                                         len_range=(40, 140), seed=92),
    "decode_d128": WORKLOADS["gqa_decode_8k"].scaled(B=3, Hq=8, Hkv=2, Lk=900, len_range=(1, 900), seed=93),
    "decode_d64": WORKLOADS["gqa_decode_8k"].scaled(B=2, Hq=4, Hkv=4, Lk=500, D=64, len_range=(30, 500),
                                                    seed=94),
    "fp32_d64": WORKLOADS["tiny_fp32"].scaled(B=1, Hq=2, Hkv=1, Lq=70, Lk=90, D=64, seed=95),
}


@pytest.mark.parametrize("name", list(DEFAULT_SCALE_CASES))
def test_default_scale_matches_oracle(orc, name):
    """scale=None passes the ABI's NaN sentinel; both sides must use 1/sqrt(d)."""
    w = DEFAULT_SCALE_CASES[name]
    inp = make_inputs(w)
    inp["scale"] = None
    banner(f"default scale {name}: D={w.D} Lq={w.Lq} Lk={w.Lk} {w.dtype}")
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o, lse, o_ref, lse_ref)
    # and bit for bit the same as passing 1/sqrt(d) itself (the fp32 value the library
    # resolves the sentinel to: a correctly rounded square root, then division)
    explicit = float(np.float32(1.0) / np.sqrt(np.float32(w.D)))
    o2, lse2 = sdpa_forward(d["q"], d["k"], d["v"], mask=d["mask"], scale=explicit,
                            is_causal=w.causal, seq_lens_q=d["len_q"], seq_lens_kv=d["len_kv"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    if w.backward:
        grads = gpu_backward(d, o, lse)
        dq, dk, dv, _ = oracle_backward(orc, inp)
        compare_backward(inp, grads, (dq, dk, dv), lse_ref)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lens", [False, True])
def test_blocked_keys_get_exactly_zero_gradient(orc, D, lens):
    """Keys that every row of a batch masks (past the batch's length, in the padded
    workload's additive mask) receive dK = dV = 0 exactly, element by element, whether the
    mask alone blocks them or the length arrays also do."""
    w = WORKLOADS["padded_mask_2k"].scaled(B=3, Hq=4, Hkv=2, Lq=230, Lk=230, D=D,
                                           len_range=(50, 200), seed=96 + D)
    inp = make_inputs(w)
    if not lens:
        inp["len_q"] = inp["len_kv"] = None
    banner(f"blocked keys D={D} lens={lens}")
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    grads = gpu_backward(d, o, lse)
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o, lse, o_ref, lse_ref)
    dq_r, dk_r, dv_r, _ = oracle_backward(orc, inp)
    compare_backward(inp, grads, (dq_r, dk_r, dv_r), lse_ref)
    m = inp["mask"].float()  # (B, 1, Lq, Lk)
    blocked = torch.isneginf(m).all(dim=2)[:, 0]  # (B, Lk): masked in every row
    dk, dv = f64(grads[1]), f64(grads[2])
    n = 0
    for b, j in blocked.nonzero().tolist():
        assert np.all(dk[b, :, j] == 0.0) and np.all(dv[b, :, j] == 0.0), (b, j)
        assert np.all(dk_r[b, :, j] == 0.0) and np.all(dv_r[b, :, j] == 0.0)
        n += 1
    assert n >= 3 * 30  # every batch has at least 30 keys past its length


BF16_MIN = float(torch.finfo(torch.bfloat16).min)


@pytest.mark.parametrize("D,causal", [(64, False), (128, False), (128, True)])
def test_rows_masked_at_bf16_min_keep_equal_weights(orc, D, causal):
    """Additive masks built from a dtype's minimum carry the most negative finite bf16, a
    finite number: a row holding it for every key has equal weights (O = mean of the
    visible values, LSE = that number), a row holding it for some keys gives them weight
    0, and -inf still empties a row.  The kernels keep masked scores in natural units, where
    the value times log2(e) would overflow to -inf.

    The backward recovers P from LSE, and at that magnitude LSE absorbs ln(n): a row held
    at the minimum for every key gets P = 1 per key there.  Its dO is zero here, as for the
    padding rows such masks mark, which makes its gradient terms zero on both sides."""
    B, Hq, Hkv, L = 2, 4, 2, 150
    g = torch.Generator().manual_seed(120 + D + causal)
    bf = lambda t: t.to(torch.bfloat16)
    q = bf(torch.randn(B, Hq, L, D, generator=g))
    k = bf(torch.randn(B, Hkv, L, D, generator=g))
    v = bf(torch.randn(B, Hkv, L, D, generator=g))
    dO = torch.randn(B, Hq, L, D, generator=g)
    m = torch.zeros(B, 1, L, L)
    m[torch.rand(B, 1, L, L, generator=g) < 0.05] = BF16_MIN
    full_row, half_row, empty_row = 5, 40, 77
    m[:, :, full_row, :] = BF16_MIN
    m[:, :, half_row, ::2] = BF16_MIN
    m[:, :, empty_row, :] = float("-inf")
    dO[:, :, full_row, :] = 0.0
    inp = dict(q=q, k=k, v=v, dO=bf(dO), mask=bf(m), len_q=None, len_kv=None,
               scale=1.0 / np.sqrt(D), is_causal=causal, window=0)
    banner(f"bf16-min mask rows D={D} causal={causal}")
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    o_ref, lse_ref = oracle_forward(orc, inp)
    G = Hq // Hkv
    nvis = full_row + 1 if causal else L
    vmean = f64(v)[:, :, :nvis].mean(axis=2)  # (B, Hkv, D)
    for h in range(Hq):
        assert np.abs(o_ref[:, h, full_row] - vmean[:, h // G]).max() < 1e-9
    assert np.all(f64(lse)[:, :, full_row] == BF16_MIN)
    assert np.all(lse_ref[:, :, full_row] == BF16_MIN)
    assert np.all(np.isneginf(lse_ref[:, :, empty_row]))
    compare_forward(inp, o, lse, o_ref, lse_ref)
    grads = gpu_backward(d, o, lse)
    refs = oracle_backward(orc, inp)[:3]
    compare_backward(inp, grads, refs, lse_ref)
