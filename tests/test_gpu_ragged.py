"""Ragged (packed THD) sequences through sdpa_forward_ragged / sdpa_backward_ragged.

Variable-length batches are packed without padding, each batch's rows one after another
(cuDNN "Attention", Support Matrix glossary note 3, Ragged Layout), optionally with gap rows
between batches (the partially packed layout, lengths then given separately), and either
side may be ragged alone.  Each case packs the padded inputs of a seeded workload, runs the
ragged entry points, and checks

  * the valid rows of O, dQ, dK, dV and all of LSE against the padded entry points on the
    same data, bit for bit;
  * the same outputs, unpacked, against the fp64 oracle to the parity tolerances;
  * that rows outside every batch (gaps) are left exactly as they were.
"""

import numpy as np
import pytest
import torch

from gpu_common import (banner, compare_backward, compare_forward, gpu_backward, gpu_forward,
                        oracle_backward, oracle_forward, to_dev)
from scaled_dot_product_sdpa_amd import BackwardCall, ForwardCall
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

W = WORKLOADS
SENTINEL = 7.0

# name -> (workload, q packed?, kv packed?, gap rows after each batch)
CASES = {
    # causal self-attention, GQA, d = 128, fully packed (lengths from the offsets)
    "thd_causal_gqa_d128": (W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=2, Lq=300, Lk=300, lens="qkv",
                                                      len_range=(1, 300), seed=60), True, True, 0),
    # bottom-right diagonal, prefill chunks against their caches, d = 64
    "thd_br_chunk_d64": (W["mha_causal_1k"].scaled(B=4, Hq=3, Hkv=3, Lq=130, Lk=333, causal=2,
                                                   lens="chunk", len_range=(60, 333), seed=61),
                         True, True, 0),
    # partially packed (gaps between batches), padded additive mask, not causal
    "thd_gaps_mask_d128": (W["padded_mask_2k"].scaled(B=3, Hq=2, Hkv=2, Lq=260, Lk=260,
                                                      len_range=(64, 260), seed=62), True, True, 5),
    # only the queries packed; keys padded with lengths
    "q_ragged_only_d64": (W["mha_causal_1k"].scaled(B=2, Hq=2, Hkv=1, Lq=200, Lk=200, lens="qkv",
                                                    len_range=(30, 200), seed=63), True, False, 0),
    # only the keys packed; not causal, Lq != Lk
    "kv_ragged_only_d128": (W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=1, Lq=100, Lk=280, causal=False,
                                                      lens="kv", len_range=(1, 280), seed=64),
                            False, True, 3),
    # sliding window over packed sequences (bottom-right diagonal, GQA, d = 128)
    "thd_window_br_d128": (W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=2, Lq=200, Lk=400, causal=2,
                                                     lens="chunk", len_range=(50, 400), window=90,
                                                     seed=68), True, True, 0),
    # fp32 path
    "thd_fp32_gqa": (W["tiny_fp32"].scaled(B=3, Hq=4, Hkv=2, Lq=70, Lk=70, D=64, lens="qkv",
                                           len_range=(1, 70), seed=65), True, True, 2),
    # decode: one query row per batch (some batches with none), keys packed
    "decode_ragged_d128": (W["gqa_decode_8k"].scaled(B=5, Hq=8, Hkv=2, Lk=900, lens="chunk",
                                                     len_range=(1, 900), seed=66), True, True, 0),
}


def _pack(x, lens, gap, fill):
    """(B, H, L, D) -> packed (T, H, D): batch b's first lens[b] rows at row offs[b], then
    `gap` rows of `fill`."""
    B, H, _, D = x.shape
    offs = [0]
    for b in range(B):
        offs.append(offs[-1] + int(lens[b]) + gap)
    out = torch.full((offs[-1], H, D), fill, dtype=x.dtype)
    for b in range(B):
        n = int(lens[b])
        out[offs[b]:offs[b] + n] = x[b, :, :n].transpose(0, 1)
    return out, torch.tensor(offs, dtype=torch.int32)


def _unpack(t, offs, lens, L):
    """packed (T, H, D) -> padded (B, H, L, D), zeros past each length."""
    B = len(lens)
    out = torch.zeros((B, t.shape[1], L, t.shape[2]), dtype=t.dtype)
    for b in range(B):
        n = int(lens[b])
        out[b, :, :n] = t[offs[b]:offs[b] + n].transpose(0, 1)
    return out


def _gap_rows(offs, lens, T):
    rows = np.ones(T, bool)
    for b in range(len(lens)):
        rows[offs[b]:offs[b] + int(lens[b])] = False
    return rows


@pytest.mark.parametrize("name", list(CASES))
def test_ragged(name, orc):
    w, pq, pkv, gap = CASES[name]
    inp = make_inputs(w)
    if inp["len_q"] is None:
        inp["len_q"] = torch.full((w.B,), w.Lq, dtype=torch.int32)
    if inp["len_kv"] is None:
        inp["len_kv"] = torch.full((w.B,), w.Lk, dtype=torch.int32)
    lq, lk = inp["len_q"].tolist(), inp["len_kv"].tolist()
    banner(f"ragged {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lq={w.Lq} Lk={w.Lk} D={w.D} {w.dtype} "
           f"causal={w.causal} q_packed={pq} kv_packed={pkv} gap={gap} lens_q={lq} lens_kv={lk}")
    nan = float("nan")
    q, oq = _pack(inp["q"], lq, gap, nan) if pq else (inp["q"], None)
    k, okv = _pack(inp["k"], lk, gap, nan) if pkv else (inp["k"], None)
    v, _ = _pack(inp["v"], lk, gap, nan) if pkv else (inp["v"], None)
    # lengths are passed explicitly when there are gaps (or a side is padded); a fully packed
    # side takes them from its offsets
    pass_lens = gap > 0 or not (pq and pkv)
    d = to_dev(inp)
    dev = lambda t: None if t is None else t.cuda()
    ragged_kw = dict(offsets_q=dev(oq), offsets_kv=dev(okv), max_seqlen_q=w.Lq, max_seqlen_kv=w.Lk,
                     seq_lens_q=d["len_q"] if pass_lens else None,
                     seq_lens_kv=d["len_kv"] if pass_lens else None)

    # padded reference run on the GPU
    o_p, lse_p = gpu_forward(d)

    ragged_kw["sliding_window"] = w.window
    fc = ForwardCall(q.cuda(), k.cuda(), v.cuda(), d["mask"], w.scale, w.causal, **ragged_kw)
    fc.o.fill_(SENTINEL)
    fc.launch()
    torch.cuda.synchronize()
    o_r, lse_r = fc.result()
    o_r, lse_r = o_r.cpu(), lse_r.cpu()
    assert torch.equal(lse_r, lse_p.cpu()), "LSE differs from the padded path"
    o_pc = o_p.cpu()
    if pq:
        o_u = _unpack(o_r, oq.tolist(), lq, w.Lq)
        gaps = _gap_rows(oq.tolist(), lq, o_r.shape[0])
        assert torch.all(o_r[torch.from_numpy(gaps)] == SENTINEL), "a gap row of O was written"
        for b in range(w.B):
            assert torch.equal(o_u[b, :, :lq[b]], o_pc[b, :, :lq[b]]), f"O of batch {b} differs"
    else:
        o_u = o_r
        assert torch.equal(o_r, o_pc)
    o_ref, lse_ref = oracle_forward(orc, inp)
    e_o, e_l = compare_forward(inp, o_u, lse_r, o_ref, lse_ref)
    msg = f"O {e_o:.2e} LSE {e_l:.2e}"

    if w.backward:
        g_p = [t.cpu() for t in gpu_backward(d, o_p, lse_p)]
        dO = _pack(inp["dO"], lq, gap, nan)[0] if pq else inp["dO"]
        bc = BackwardCall(q.cuda(), k.cuda(), v.cuda(), fc.o, dO.cuda(), fc.lse, d["mask"], w.scale,
                          w.causal, **ragged_kw)
        for t in (bc.dq, bc.dk, bc.dv):
            t.fill_(SENTINEL)
        bc.launch()
        torch.cuda.synchronize()
        g_r = [t.cpu() for t in bc.result()]
        unpacked = []
        for g, gp, packed, offs, lens, L, nm in ((g_r[0], g_p[0], pq, oq, lq, w.Lq, "dQ"),
                                                 (g_r[1], g_p[1], pkv, okv, lk, w.Lk, "dK"),
                                                 (g_r[2], g_p[2], pkv, okv, lk, w.Lk, "dV")):
            if packed:
                gaps = _gap_rows(offs.tolist(), lens, g.shape[0])
                assert torch.all(g[torch.from_numpy(gaps)] == SENTINEL), f"a gap row of {nm} was written"
                gu = _unpack(g, offs.tolist(), lens, L)
                for b in range(w.B):
                    assert torch.equal(gu[b, :, :lens[b]], gp[b, :, :lens[b]]), f"{nm} of batch {b} differs"
            else:
                gu = g
                assert torch.equal(g, gp), f"{nm} differs from the padded path"
            unpacked.append(gu)
        dq, dk, dv, _ = oracle_backward(orc, inp)
        errs = compare_backward(inp, unpacked, (dq, dk, dv), lse_ref)
        msg += " dQ {:.2e} dK {:.2e} dV {:.2e}".format(*errs)
    banner(f"ragged {name}: {msg}")


def test_ragged_head_major_packing():
    """A packed tensor stored head-major ((H, T, D) memory viewed as (T, H, D)) gives the
    same result as the token-major one: only the strides differ."""
    w = W["mha_causal_1k"].scaled(B=3, Hq=2, Hkv=2, Lq=150, Lk=150, lens="qkv", len_range=(10, 150),
                                  seed=67, backward=False)
    inp = make_inputs(w)
    lens = inp["len_q"].tolist()
    lens_kv = inp["len_kv"].tolist()
    q, oq = _pack(inp["q"], lens, 0, 0.0)
    k, ok = _pack(inp["k"], lens_kv, 0, 0.0)
    v, _ = _pack(inp["v"], lens_kv, 0, 0.0)
    hm = lambda t: t.transpose(0, 1).contiguous().cuda().transpose(0, 1)
    banner(f"ragged head-major packing: lens {lens} / {lens_kv}")
    kw = dict(is_causal=True, offsets_q=oq.cuda(), offsets_kv=ok.cuda())
    a = ForwardCall(q.cuda(), k.cuda(), v.cuda(), None, w.scale, **kw)
    b = ForwardCall(hm(q), hm(k), hm(v), None, w.scale, **kw)
    a.launch()
    b.launch()
    torch.cuda.synchronize()
    assert torch.equal(a.o.cpu(), b.o.cpu()) and torch.equal(a.lse.cpu(), b.lse.cpu())
