"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every ``check_*`` takes an ``Oracle`` handle and raises AssertionError on a mismatch.
``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py`` runs them
on deliberately broken builds of it and requires each broken build to fail at least one.

None of these checks re-types the oracle's formula: each compares it with something
else — the worked example's printed numbers, a closed form, an invariant, a brute-force
finite difference, a library routine, or a statistical property.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _randn(rng, *shape):
    return rng.standard_normal(shape)


def _rand_mask(rng, B, H, Lq, Lk, p_block=0.3):
    m = rng.standard_normal((B, H, Lq, Lk)) * 0.5
    m[rng.random((B, H, Lq, Lk)) < p_block] = -np.inf
    return m


# ---------------------------------------------------------------------------------
# Worked example ("Scaled dot-product attention (forward and backward)", section 3)
# ---------------------------------------------------------------------------------
def _hand():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float).reshape(1, 1, 1, 4)
    k = np.array(g["k"], float).reshape(1, 1, 3, 4)
    v = np.array(g["v"], float).reshape(1, 1, 3, 2)
    dO = np.array(g["dO"], float).reshape(1, 1, 1, 2)
    return g, q, k, v, dO


def check_hand_forward(orc):
    """P, O of the worked example; P read out through V = I (then O_i = P_i)."""
    g, q, k, v, dO = _hand()
    tol = g["tolerance_abs"]
    e = g["expected"]
    # default scale: d = 4 gives alpha = 1/2, the example's scale
    o, lse = orc.forward(q, k, v)
    assert np.abs(o.reshape(-1) - e["O"]).max() <= tol, o
    o_p, _ = orc.forward(q, k, np.eye(3).reshape(1, 1, 3, 3), scale=g["scale"])
    assert np.abs(o_p.reshape(-1) - e["P"]).max() <= tol, o_p
    # S from P: S_j - S_0 = ln(P_j / P_0); the page's S = (1, 0, 2)
    s = np.log(o_p.reshape(-1) / o_p.reshape(-1)[0]) + e["S"][0]
    assert np.abs(s - e["S"]).max() <= 1e-9, s


def check_hand_lse(orc):
    """LSE of the worked example equals the closed form ln(1 + e + e^2)."""
    g, q, k, v, dO = _hand()
    _, lse = orc.forward(q, k, v, scale=g["scale"])
    assert abs(lse.item() - math.log(1 + math.e + math.e ** 2)) <= 1e-12, lse


def check_hand_backward(orc):
    g, q, k, v, dO = _hand()
    tol = g["tolerance_abs"]
    e = g["expected"]
    dq, dk, dv, D = orc.backward(q, k, v, dO, scale=g["scale"])
    assert np.abs(dv.reshape(3, 2) - np.array(e["dV"])).max() <= tol, dv
    assert np.abs(dq.reshape(-1) - e["dQ"]).max() <= tol, dq
    assert np.abs(dk.reshape(3, 4) - np.array(e["dK"])).max() <= tol, dk
    assert abs(D.item() - e["D"]) <= tol, D
    # the example's q/2 = (1,0,0,0), so dK row j carries dS_j in its first entry
    assert np.abs(dk.reshape(3, 4)[:, 0] - e["dS"]).max() <= tol


# ---------------------------------------------------------------------------------
# Identities and invariants
# ---------------------------------------------------------------------------------
def _case(seed, B=2, Hq=4, Hkv=2, Lq=7, Lk=9, Dk=5, Dv=3, mask=True, causal=False, lens=False):
    rng = _rng(seed)
    q = _randn(rng, B, Hq, Lq, Dk)
    k = _randn(rng, B, Hkv, Lk, Dk)
    v = _randn(rng, B, Hkv, Lk, Dv)
    dO = _randn(rng, B, Hq, Lq, Dv)
    m = _rand_mask(rng, B, Hq, Lq, Lk) if mask else None
    lq = lk = None
    if lens:
        lq = rng.integers(0, Lq + 1, B).astype(np.int32)
        lk = rng.integers(0, Lk + 1, B).astype(np.int32)
        lq[0], lk[0] = Lq, Lk
    return dict(q=q, k=k, v=v, dO=dO, mask=m, len_q=lq, len_kv=lk, is_causal=causal)


def _fwd(orc, c, **kw):
    a = dict(mask=c["mask"], is_causal=c["is_causal"], len_q=c["len_q"], len_kv=c["len_kv"])
    a.update(kw)
    return orc.forward(c["q"], c["k"], c["v"], **a)


def _bwd(orc, c, **kw):
    a = dict(mask=c["mask"], is_causal=c["is_causal"], len_q=c["len_q"], len_kv=c["len_kv"])
    a.update(kw)
    return orc.backward(c["q"], c["k"], c["v"], c["dO"], **a)


def check_rowsum_identity(orc):
    """D_i = sum_j P_ij dP_ij (backward) equals dO_i . O_i (forward output)."""
    for seed, causal, lens in ((11, False, False), (12, True, False), (13, True, True)):
        c = _case(seed, causal=causal, lens=lens)
        o, _ = _fwd(orc, c)
        *_, D = _bwd(orc, c)
        assert np.abs(D - (c["dO"] * o).sum(-1)).max() <= 1e-12


def check_rows_sum_to_one(orc):
    """With V = 1 every non-empty row's output is sum_j P_ij = 1; empty rows give 0."""
    c = _case(21, causal=True, lens=True)
    v1 = np.ones_like(c["v"])
    o, lse = orc.forward(c["q"], c["k"], v1, mask=c["mask"], is_causal=True,
                         len_q=c["len_q"], len_kv=c["len_kv"])
    nonempty = np.isfinite(lse)
    assert np.abs(o[nonempty] - 1.0).max() <= 1e-12
    assert np.all(o[~nonempty] == 0.0)
    assert nonempty.sum() > 0 and (~nonempty).sum() > 0


def check_key_shift_invariance(orc):
    """Adding one vector c to every key shifts each score row by a constant (q_i . c):
    O, dV are unchanged and dQ is unchanged because sum_j dS_ij = 0."""
    c = _case(31, mask=True, causal=True)
    shift = _rng(32).standard_normal(c["k"].shape[-1])
    o1, _ = _fwd(orc, c)
    dq1, dk1, dv1, _ = _bwd(orc, c)
    c2 = dict(c, k=c["k"] + shift)
    o2, _ = _fwd(orc, c2)
    dq2, dk2, dv2, _ = _bwd(orc, c2)
    assert np.abs(o1 - o2).max() <= 1e-10
    assert np.abs(dq1 - dq2).max() <= 1e-10
    assert np.abs(dv1 - dv2).max() <= 1e-10


def check_gradcheck(orc):
    """Every gradient element against central differences of f = sum(O * g), h = 1e-6,
    with an additive mask, causal, GQA, lengths and Dk != Dv."""
    c = _case(41, B=2, Hq=4, Hkv=2, Lq=4, Lk=5, Dk=3, Dv=2, mask=True, causal=True, lens=True)
    c["len_q"] = np.array([4, 3], np.int32)
    c["len_kv"] = np.array([5, 4], np.int32)
    g = c["dO"]
    dq, dk, dv, _ = _bwd(orc, c, scale=0.7)
    h = 1e-6

    def f(**over):
        cc = dict(c, **over)
        o, _ = _fwd(orc, cc, scale=0.7)
        return (o * g).sum()

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            num[idx] = (f(**{name: xp}) - f(**{name: xm})) / (2 * h)
        err = np.abs(num - grad).max() / max(1.0, np.abs(num).max())
        assert err <= 1e-6, (name, err)


def check_key_permutation_equivariance(orc):
    """Permuting keys with their values (and mask columns) leaves O unchanged and permutes
    dK, dV rows (non-causal, no lengths)."""
    c = _case(51, mask=True, causal=False)
    perm = _rng(52).permutation(c["k"].shape[2])
    c2 = dict(c, k=c["k"][:, :, perm], v=c["v"][:, :, perm], mask=c["mask"][..., perm])
    o1, l1 = _fwd(orc, c)
    o2, l2 = _fwd(orc, c2)
    assert np.abs(o1 - o2).max() <= 1e-12
    assert np.abs(np.nan_to_num(l1) - np.nan_to_num(l2)).max() <= 1e-12
    dq1, dk1, dv1, _ = _bwd(orc, c)
    dq2, dk2, dv2, _ = _bwd(orc, c2)
    assert np.abs(dk1[:, :, perm] - dk2).max() <= 1e-12
    assert np.abs(dv1[:, :, perm] - dv2).max() <= 1e-12
    assert np.abs(dq1 - dq2).max() <= 1e-12


def check_query_independence(orc):
    """Rows are independent: permuting queries permutes outputs; the rows API agrees."""
    c = _case(61, mask=False, causal=False)
    perm = _rng(62).permutation(c["q"].shape[2])
    o1, l1 = _fwd(orc, c)
    o2, l2 = _fwd(orc, dict(c, q=c["q"][:, :, perm]))
    assert np.array_equal(o1[:, :, perm], o2)
    rows = [(1, 3, 2), (0, 0, 6), (1, 1, 0)]
    orow, lrow = orc.forward_rows(c["q"], c["k"], c["v"], rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[r], o1[b, h, i]) and lrow[r] == l1[b, h, i]


def check_batched_equals_per_item(orc):
    """[B, H, T, d] equals B*H separate 2-D problems, gradients too (Lq != Lk)."""
    c = _case(71, B=2, Hq=3, Hkv=3, Lq=5, Lk=8, mask=True, causal=False)
    o, lse = _fwd(orc, c)
    dq, dk, dv, _ = _bwd(orc, c)
    for b in range(2):
        for h in range(3):
            sl = lambda a: a[b:b + 1, h:h + 1]
            cc = dict(c, q=sl(c["q"]), k=sl(c["k"]), v=sl(c["v"]), dO=sl(c["dO"]), mask=sl(c["mask"]))
            o1, l1 = _fwd(orc, cc)
            dq1, dk1, dv1, _ = _bwd(orc, cc)
            assert np.array_equal(o1[0, 0], o[b, h])
            assert np.array_equal(dq1[0, 0], dq[b, h])
            assert np.array_equal(dk1[0, 0], dk[b, h]) and np.array_equal(dv1[0, 0], dv[b, h])


def check_masked_keys(orc):
    """A key blocked for every query gets weight exactly 0 and gradients exactly 0;
    its value never influences O; the open weights still sum to 1."""
    c = _case(81, mask=True, causal=False)
    m = c["mask"].copy()
    m[..., 2] = -np.inf
    c = dict(c, mask=m)
    eye = np.broadcast_to(np.eye(9), (2, 2, 9, 9)).copy()
    w, lse = orc.forward(c["q"], c["k"], eye, mask=m)
    assert np.all(w[..., 2] == 0.0)
    fin = np.isfinite(lse)
    assert np.abs(w.sum(-1)[fin] - 1.0).max() <= 1e-12
    dq, dk, dv, _ = _bwd(orc, c)
    assert np.all(dk[:, :, 2] == 0.0) and np.all(dv[:, :, 2] == 0.0)
    v2 = c["v"].copy()
    v2[:, :, 2] = 1e30
    o1, _ = _fwd(orc, c)
    o2, _ = _fwd(orc, dict(c, v=v2))
    assert np.array_equal(o1, o2)


def check_fully_masked_row(orc):
    """A fully blocked row gives O = 0, dQ = 0, LSE = -inf, and no NaN anywhere."""
    c = _case(91, mask=True, causal=False)
    m = c["mask"].copy()
    m[1, 0, 3, :] = -np.inf
    c = dict(c, mask=m)
    o, lse = _fwd(orc, c)
    dq, dk, dv, D = _bwd(orc, c)
    assert np.all(o[1, 0, 3] == 0.0) and lse[1, 0, 3] == -np.inf
    assert np.all(dq[1, 0, 3] == 0.0) and D[1, 0, 3] == 0.0
    for a in (o, dq, dk, dv, D):
        assert not np.isnan(a).any()


def check_large_scores(orc):
    """Scores of order 1e4 give a clean one-hot (the row max is subtracted)."""
    q = np.zeros((1, 1, 1, 2)); q[..., 0] = 100.0
    k = np.zeros((1, 1, 3, 2)); k[0, 0, :, 0] = [100.0, 99.0, 101.0]
    v = np.arange(6, dtype=float).reshape(1, 1, 3, 2)
    o, lse = orc.forward(q, k, v, scale=1.0)
    assert np.array_equal(o.reshape(-1), v[0, 0, 2]), o
    assert lse.item() == 10100.0


def check_default_scale(orc):
    """The default scale equals an explicit 1/sqrt(Dk), bit for bit (Dk != Dv)."""
    c = _case(101, Dk=6, Dv=3, mask=True)
    o1, l1 = _fwd(orc, c)
    o2, l2 = _fwd(orc, c, scale=1.0 / math.sqrt(6))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    g1 = _bwd(orc, c)
    g2 = _bwd(orc, c, scale=1.0 / math.sqrt(6))
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


def check_causal_is_tril(orc):
    """is_causal equals an explicit additive mask built from tril (diagonal kept), also
    for Lq != Lk (top-left alignment)."""
    for Lq, Lk in ((6, 6), (4, 7), (7, 4)):
        c = _case(111 + Lq, Lq=Lq, Lk=Lk, mask=False)
        tril = np.tril(np.ones((Lq, Lk), bool))
        m = np.where(tril, 0.0, -np.inf).reshape(1, 1, Lq, Lk)
        o1, l1 = _fwd(orc, c, is_causal=True)
        o2, l2 = _fwd(orc, c, mask=m)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        g1 = _bwd(orc, c, is_causal=True)
        g2 = _bwd(orc, c, mask=m)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)


def check_gqa_is_repeat_interleave(orc):
    """GQA equals MHA on K/V expanded in repeat_interleave order (kv0,kv0,..,kv1,..);
    a shared head's dK/dV is the sum of the expanded heads' gradients."""
    c = _case(121, B=2, Hq=6, Hkv=2, mask=True, causal=True)
    G = 3
    ke = np.repeat(c["k"], G, axis=1)
    ve = np.repeat(c["v"], G, axis=1)
    o1, l1 = _fwd(orc, c)
    o2, l2 = _fwd(orc, dict(c, k=ke, v=ve))
    assert np.abs(o1 - o2).max() <= 1e-12 and np.array_equal(np.isinf(l1), np.isinf(l2))
    dq1, dk1, dv1, _ = _bwd(orc, c)
    dq2, dk2, dv2, _ = _bwd(orc, dict(c, k=ke, v=ve))
    assert np.abs(dq1 - dq2).max() <= 1e-12
    assert np.abs(dk1 - dk2.reshape(2, 2, G, *dk2.shape[2:]).sum(2)).max() <= 1e-12
    assert np.abs(dv1 - dv2.reshape(2, 2, G, *dv2.shape[2:]).sum(2)).max() <= 1e-12


def check_score_variance(orc):
    """With q, k ~ N(0,1) and the default scale, the difference of two scores has
    variance 2 at d = 4 and d = 64 (read back from two-key weights through V = I)."""
    for d in (4, 64):
        rng = _rng(131 + d)
        n = 4000
        q = rng.standard_normal((1, n, 1, d))
        k = rng.standard_normal((1, n, 2, d))
        o, _ = orc.forward(q, k, np.broadcast_to(np.eye(2), (1, n, 2, 2)).copy())
        diff = np.log(o[0, :, 0, 0] / o[0, :, 0, 1])
        var = diff.var()
        # sample variance of n draws with variance 2 has sd about 2*sqrt(2/n) (Gaussian-ish)
        assert abs(var - 2.0) < 5 * 2 * math.sqrt(2 / n) * 1.5, (d, var)


def check_single_key(orc):
    """Lk = 1: P = 1, O = v_0, dQ = dK = 0, dV = sum_i dO_i (closed forms)."""
    c = _case(141, Lk=1, mask=False)
    o, lse = _fwd(orc, c)
    G = c["q"].shape[1] // c["k"].shape[1]
    assert np.array_equal(o, np.repeat(c["v"], G, axis=1).repeat(c["q"].shape[2], axis=2))
    dq, dk, dv, _ = _bwd(orc, c)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    ref = c["dO"].reshape(2, 2, G, -1, c["dO"].shape[-1]).sum(axis=(2, 3))
    assert np.abs(dv[:, :, 0] - ref).max() <= 1e-12


def check_identical_keys(orc):
    """All keys equal: uniform weights, O = mean of the values."""
    c = _case(151, mask=False)
    k = np.broadcast_to(c["k"][:, :, :1], c["k"].shape).copy()
    o, _ = orc.forward(c["q"], k, c["v"])
    mean = np.repeat(c["v"].mean(axis=2, keepdims=True), 2, axis=1)
    assert np.abs(o - mean).max() <= 1e-12


def check_mask_at_bf16_min(orc):
    """A mask value at the most negative finite bf16 (what masks built from a dtype's
    minimum carry) is a finite number, not a block: a row holding it for every key has
    equal weights, O = mean of the values, and LSE equal to that value (ln n is below
    its spacing); a row holding it for some keys gives those keys weight 0 and matches the
    same row with -inf there."""
    lo = -3.3895313892515355e38  # -(2 - 2**-7) * 2**127, the most negative finite bf16
    c = _case(157, mask=False, Lq=4, Lk=6)
    B, H, Lq, Lk = c["q"].shape[0], c["q"].shape[1], c["q"].shape[2], c["k"].shape[2]
    m = np.zeros((B, 1, Lq, Lk))
    m[:, :, 0, :] = lo
    m[:, :, 1, ::2] = lo
    o, lse = orc.forward(c["q"], c["k"], c["v"], mask=m)
    mean = np.repeat(c["v"].mean(axis=2), 2, axis=1)  # (B, Hq, Dv), Hq = 2 Hkv
    assert np.abs(o[:, :, 0] - mean).max() <= 1e-12
    assert np.all(lse[:, :, 0] == lo)
    m_inf = m.copy()
    m_inf[:, :, 1, ::2] = -np.inf
    o2, lse2 = orc.forward(c["q"], c["k"], c["v"], mask=m_inf)
    assert np.abs(o[:, :, 1] - o2[:, :, 1]).max() <= 1e-12
    assert np.abs(lse[:, :, 1] - lse2[:, :, 1]).max() <= 1e-12


def check_lengths_are_masks(orc):
    """Per-batch lengths equal an additive mask with -inf at padded keys, with padded query
    rows empty (O = 0, LSE = -inf, no gradient); padded K/V contents are never read
    (NaN poison there changes nothing); a length of 0 empties the batch."""
    c = _case(161, B=3, mask=True, causal=False)
    lq = np.array([7, 4, 0], np.int32)
    lk = np.array([9, 5, 0], np.int32)
    B, H, Lq, Lk = 3, 4, 7, 9
    pad = np.zeros((B, 1, Lq, Lk))
    for b in range(B):
        pad[b, :, lq[b]:, :] = -np.inf
        pad[b, :, :, lk[b]:] = -np.inf
    o1, l1 = _fwd(orc, c, len_q=lq, len_kv=lk)
    o2, l2 = _fwd(orc, c, mask=c["mask"] + pad)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for b in range(B):
        assert np.all(o1[b, :, lq[b]:] == 0.0) and np.all(l1[b, :, lq[b]:] == -np.inf)
    kp, vp = c["k"].copy(), c["v"].copy()
    for b in range(B):
        kp[b, :, lk[b]:] = np.nan
        vp[b, :, lk[b]:] = np.nan
    o3, l3 = _fwd(orc, dict(c, k=kp, v=vp), len_q=lq, len_kv=lk)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
    g1 = _bwd(orc, c, len_q=lq, len_kv=lk)
    g3 = _bwd(orc, dict(c, k=kp, v=vp), len_q=lq, len_kv=lk)
    for a, b in zip(g1, g3):
        assert np.array_equal(np.nan_to_num(a, nan=7.0), a)  # no NaN leaked
        assert np.array_equal(a, b)
    dq, dk, dv, _ = g1
    assert np.all(dq[2] == 0.0) and np.all(dk[2] == 0.0) and np.all(dv[2] == 0.0)
    assert np.all(dk[1, :, 5:] == 0.0) and np.all(dq[1, :, 4:] == 0.0)


def check_torch_library(orc):
    """Library pin: torch's CPU fp64 scaled_dot_product_attention (+ autograd) on random
    inputs with a float mask, causal, and GQA (rows with a finite LSE only)."""
    import torch
    import torch.nn.functional as F

    for seed, causal, use_mask, Hq, Hkv in ((171, False, True, 4, 2), (172, True, False, 4, 1),
                                            (173, False, False, 2, 2)):
        c = _case(seed, Hq=Hq, Hkv=Hkv, Dk=5, Dv=4, mask=use_mask, causal=causal)
        if use_mask:
            c["mask"][:, :, :, 0] = 0.0  # keep every row non-empty for the library
        tq = torch.tensor(c["q"], requires_grad=True)
        tk = torch.tensor(c["k"], requires_grad=True)
        tv = torch.tensor(c["v"], requires_grad=True)
        tm = torch.tensor(c["mask"]) if use_mask else None
        out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, is_causal=causal,
                                             scale=0.6, enable_gqa=Hq != Hkv)
        out.backward(torch.tensor(c["dO"]))
        o, _ = _fwd(orc, c, scale=0.6)
        dq, dk, dv, _ = _bwd(orc, c, scale=0.6)
        assert np.abs(out.detach().numpy() - o).max() <= 1e-10
        assert np.abs(tq.grad.numpy() - dq).max() <= 1e-10
        assert np.abs(tk.grad.numpy() - dk).max() <= 1e-10
        assert np.abs(tv.grad.numpy() - dv).max() <= 1e-10


# ---------------------------------------------------------------------------------
# Bottom-right causal alignment (cuDNN "Attention", forward Configurable Options,
# diagonal masking: BOTTOM_RIGHT with right bound 0)
# ---------------------------------------------------------------------------------
def check_bottom_right_chunked_prefill(orc):
    """The last c queries of a top-left causal problem over n tokens equal the
    bottom-right causal problem of those c queries against all n keys (a prefill chunk
    against its KV cache): same O, LSE and dQ, and the same dK, dV when the other rows
    carry no output gradient.  Per batch, with lengths: the chunk is the last len_q rows
    of the batch's len_kv tokens."""
    rng = _rng(401)
    B, Hq, Hkv, n, c, Dk, Dv = 3, 4, 2, 11, 4, 5, 3
    q = _randn(rng, B, Hq, n, Dk)
    k = _randn(rng, B, Hkv, n, Dk)
    v = _randn(rng, B, Hkv, n, Dv)
    dO = _randn(rng, B, Hq, n, Dv)
    # full sequences: the last c rows
    o_full, l_full = orc.forward(q, k, v, is_causal=True)
    dO_c = np.zeros_like(dO)
    dO_c[:, :, n - c:] = dO[:, :, n - c:]
    gq_f, gk_f, gv_f, _ = orc.backward(q, k, v, dO_c, is_causal=True)
    o, l = orc.forward(q[:, :, n - c:], k, v, is_causal=2)
    gq, gk, gv, _ = orc.backward(q[:, :, n - c:], k, v, dO[:, :, n - c:], is_causal=2)
    assert np.abs(o - o_full[:, :, n - c:]).max() <= 1e-12
    assert np.abs(l - l_full[:, :, n - c:]).max() <= 1e-12
    assert np.abs(gq - gq_f[:, :, n - c:]).max() <= 1e-12
    assert np.abs(gk - gk_f).max() <= 1e-12 and np.abs(gv - gv_f).max() <= 1e-12
    # per-batch lengths: batch b has len_kv tokens and its chunk is the last len_q of them
    lk = np.array([11, 7, 3], np.int32)
    lq = np.array([4, 2, 3], np.int32)
    qc = np.zeros((B, Hq, c, Dk))
    for b in range(B):
        qc[b, :, :lq[b]] = q[b, :, lk[b] - lq[b]:lk[b]]
    o, l = orc.forward(qc, k, v, is_causal=2, len_q=lq, len_kv=lk)
    for b in range(B):
        ob, lb = orc.forward(q[b:b + 1, :, :lk[b]], k[b:b + 1, :, :lk[b]], v[b:b + 1, :, :lk[b]],
                             is_causal=True)
        assert np.abs(o[b, :, :lq[b]] - ob[0, :, lk[b] - lq[b]:]).max() <= 1e-12
        assert np.abs(l[b, :, :lq[b]] - lb[0, :, lk[b] - lq[b]:]).max() <= 1e-12
        assert np.all(o[b, :, lq[b]:] == 0) and np.all(np.isneginf(l[b, :, lq[b]:]))


def check_bottom_right_is_shifted_tril(orc):
    """Bottom-right causal equals an additive mask from numpy's tril with the diagonal
    offset Lk - Lq (the diagonal ends in the bottom-right corner), bit for bit, for Lq < Lk,
    Lq = Lk (where it equals top-left) and Lq > Lk (whose first Lq - Lk rows see no key)."""
    for Lq, Lk in ((4, 7), (6, 6), (7, 4)):
        c = _case(411 + Lq, Lq=Lq, Lk=Lk, mask=False)
        tril = np.tril(np.ones((Lq, Lk), bool), k=Lk - Lq)
        m = np.where(tril, 0.0, -np.inf).reshape(1, 1, Lq, Lk)
        o1, l1 = _fwd(orc, c, is_causal=2)
        o2, l2 = _fwd(orc, c, mask=m)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        g1 = _bwd(orc, c, is_causal=2)
        g2 = _bwd(orc, c, mask=m)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)
        if Lq == Lk:
            o3, l3 = _fwd(orc, c, is_causal=True)
            assert np.array_equal(o1, o3) and np.array_equal(l1, l3)
        if Lq > Lk:
            assert np.all(o1[:, :, :Lq - Lk] == 0) and np.all(np.isneginf(l1[:, :, :Lq - Lk]))
    # one query row against its whole cache: every key is visible (decode)
    c = _case(419, Lq=1, Lk=9, mask=False)
    o1, l1 = _fwd(orc, c, is_causal=2)
    o2, l2 = _fwd(orc, c, is_causal=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def check_window_is_band_mask(orc):
    """A sliding window of W keys (with either diagonal) equals an explicit additive band
    mask built with numpy (tril at the diagonal offset minus tril W further down), bit for
    bit in the forward and the backward, with Lq < Lk, Lq = Lk and Lq > Lk."""
    for Lq, Lk, W, mode in ((7, 9, 3, 1), (7, 9, 3, 2), (6, 6, 2, 1), (8, 5, 4, 2), (5, 11, 1, 2)):
        c = _case(431 + Lq + W, Lq=Lq, Lk=Lk, mask=False)
        off = Lk - Lq if mode == 2 else 0
        band = np.tril(np.ones((Lq, Lk), bool), k=off) & ~np.tril(np.ones((Lq, Lk), bool), k=off - W)
        m = np.where(band, 0.0, -np.inf).reshape(1, 1, Lq, Lk)
        o1, l1 = _fwd(orc, c, is_causal=mode, window=W)
        o2, l2 = _fwd(orc, c, mask=m, is_causal=False)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        g1 = _bwd(orc, c, is_causal=mode, window=W)
        g2 = _bwd(orc, c, mask=m, is_causal=False)
        for a, b in zip(g1, g2):
            assert np.array_equal(a, b)
        # every row sees at most W keys
        assert band.sum(axis=1).max() <= W


def check_window_limits(orc):
    """A window at least as long as the key range is plain causal attention (bit for bit);
    a window of one key leaves each row its diagonal key alone: O_i = v_i, LSE_i = the
    score of that pair, and (P = 1 is constant) dQ = dK = 0 while dV_i = dO_i summed over
    the query heads of the group."""
    c = _case(441, Lq=9, Lk=9, mask=False, lens=True)
    for mode in (1, 2):
        o1, l1 = _fwd(orc, c, is_causal=mode, window=9)
        o2, l2 = _fwd(orc, c, is_causal=mode)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        for a, b in zip(_bwd(orc, c, is_causal=mode, window=40), _bwd(orc, c, is_causal=mode)):
            assert np.array_equal(a, b)
    c = _case(442, Lq=6, Lk=6, mask=False)
    q, k, v, dO = c["q"], c["k"], c["v"], c["dO"]
    B, Hq, L, _ = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(q.shape[-1])
    o, lse = _fwd(orc, c, is_causal=1, window=1)
    dq, dk, dv, _ = _bwd(orc, c, is_causal=1, window=1)
    for h in range(Hq):
        g = h // G
        assert np.array_equal(o[:, h], v[:, g])
        s = scale * np.einsum("bid,bid->bi", q[:, h], k[:, g])
        assert np.abs(lse[:, h] - s).max() <= 1e-12
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    want = dO.reshape(B, k.shape[1], G, L, -1).sum(axis=2)
    assert np.abs(dv - want).max() <= 1e-12


def check_bottom_right_torch(orc):
    """Library pin: torch's CPU fp64 scaled_dot_product_attention with its lower-right
    causal bias (torch.nn.attention.bias.causal_lower_right) and autograd, Lq < Lk, GQA."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention.bias import causal_lower_right

    for seed, Lq, Lk, Hq, Hkv in ((431, 5, 9, 4, 2), (432, 3, 3, 2, 2)):
        c = _case(seed, Lq=Lq, Lk=Lk, Hq=Hq, Hkv=Hkv, mask=False)
        tq = torch.tensor(c["q"], requires_grad=True)
        tk = torch.tensor(c["k"], requires_grad=True)
        tv = torch.tensor(c["v"], requires_grad=True)
        bias = causal_lower_right(Lq, Lk)._materialize()
        tm = torch.zeros(Lq, Lk, dtype=torch.float64).masked_fill(~bias, float("-inf"))
        G = Hq // Hkv
        out = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1),
                                             attn_mask=tm, scale=0.7)
        out.backward(torch.tensor(c["dO"]))
        o, _ = _fwd(orc, c, is_causal=2, scale=0.7)
        dq, dk, dv, _ = _bwd(orc, c, is_causal=2, scale=0.7)
        assert np.abs(out.detach().numpy() - o).max() <= 1e-10
        assert np.abs(tq.grad.numpy() - dq).max() <= 1e-10
        assert np.abs(tk.grad.numpy() - dk).max() <= 1e-10
        assert np.abs(tv.grad.numpy() - dv).max() <= 1e-10


ALL_CHECKS = [
    check_hand_forward, check_hand_lse, check_hand_backward, check_rowsum_identity,
    check_rows_sum_to_one, check_key_shift_invariance, check_gradcheck,
    check_key_permutation_equivariance, check_query_independence, check_batched_equals_per_item,
    check_masked_keys, check_fully_masked_row, check_large_scores, check_default_scale,
    check_causal_is_tril, check_gqa_is_repeat_interleave, check_score_variance,
    check_single_key, check_identical_keys, check_mask_at_bf16_min, check_lengths_are_masks, check_torch_library,
    check_bottom_right_chunked_prefill, check_bottom_right_is_shifted_tril,
    check_bottom_right_torch, check_window_is_band_mask, check_window_limits,
]
