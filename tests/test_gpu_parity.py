"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element,
on seeded inputs at sizes the oracle finishes in seconds.  Shapes span several tiles and end
in ragged tails; every feature path (causal, additive mask, lengths, GQA, decode, fp32) is
covered.  Tolerances are in ``gpu_common``.
"""

import json
import os

import numpy as np
import pytest
import torch

from gpu_common import (banner, compare_backward, compare_forward, gpu_backward, gpu_forward,
                        oracle_backward, oracle_forward, to_dev)
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

W = WORKLOADS
CASES = {
    # the tiny fp32 workload at its full size, without and with the causal mask
    "tiny_fp32": W["tiny_fp32"],
    "tiny_fp32_causal": W["tiny_fp32"].scaled(causal=True),
    # fp32 path with GQA, lengths and an additive mask (several 64-row blocks, ragged)
    "fp32_gqa_mask_lens": W["padded_mask_2k"].scaled(dtype="f32", B=2, Hq=4, Hkv=2, Lq=70, Lk=70,
                                                     D=64, len_range=(20, 70), seed=11),
    # bf16 causal MHA, d = 64, ragged tail (300 = 2*128 + 44 query rows, 4*64 + 44 keys)
    "mha_causal_d64": W["mha_causal_1k"].scaled(B=2, Hq=3, Hkv=3, Lq=300, Lk=300, seed=12),
    # bf16 non-causal with Lq != Lk
    "mha_cross_d64": W["mha_causal_1k"].scaled(B=1, Hq=2, Hkv=2, Lq=200, Lk=333, causal=False, seed=13),
    # bf16 causal GQA, d = 128, 4 query heads per KV head
    "gqa_causal_d128": W["gqa_causal_4k"].scaled(B=1, Hq=8, Hkv=2, Lq=333, Lk=333, seed=14),
    # causal with per-batch lengths (q and kv)
    "causal_lens_d128": W["gqa_causal_4k"].scaled(B=2, Hq=2, Hkv=1, Lq=260, Lk=260, lens="qkv",
                                                  len_range=(1, 260), seed=15),
    # padded batch with an additive mask, extra random -inf keys and a fully masked row
    "padded_mask_d128": W["padded_mask_2k"].scaled(B=3, Hq=2, Hkv=2, Lq=260, Lk=260,
                                                   len_range=(64, 260), seed=16),
    # the mask at d = 64 (mask tiles copied with the Q/dO tiles, two tiles in flight)
    "padded_mask_d64": W["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=1, Lq=333, Lk=333, D=64,
                                                  len_range=(100, 333), seed=23),
    # the same inputs, mask only (no length arrays)
    "padded_mask_only_d128": W["padded_mask_2k"].scaled(B=3, Hq=2, Hkv=2, Lq=260, Lk=260,
                                                        len_range=(64, 260), seed=16, lens="none_keep"),
    # bottom-right causal diagonal (a chunk of queries against its KV cache): Lq < Lk,
    # per-batch query and key lengths, Lq > Lk (leading rows see no key), with a mask, fp32
    "chunk_br_d64": W["mha_causal_1k"].scaled(B=2, Hq=3, Hkv=3, Lq=200, Lk=333, causal=2, seed=40),
    "chunk_br_gqa_lens_d128": W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=2, Lq=150, Lk=400, causal=2,
                                                        lens="chunk", len_range=(100, 400), seed=41),
    "br_lq_gt_lk_d128": W["gqa_causal_4k"].scaled(B=1, Hq=2, Hkv=1, Lq=300, Lk=200, causal=2, seed=42),
    "br_mask_lens_d128": W["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=2, Lq=200, Lk=260, causal=2,
                                                    lens="chunk", len_range=(64, 260), seed=43),
    "fp32_br_gqa": W["tiny_fp32"].scaled(B=2, Hq=4, Hkv=2, Lq=40, Lk=70, D=64, causal=2,
                                         lens="chunk", len_range=(30, 70), seed=44),
    # decode (Lq = 1) against a KV cache with lengths and NaN-poisoned padding
    "decode_gqa_d128": W["gqa_decode_8k"].scaled(B=4, Hq=8, Hkv=2, Lk=1100, len_range=(1, 1100), seed=17),
    "decode_mha_d64": W["gqa_decode_8k"].scaled(B=3, Hq=4, Hkv=4, Lk=700, D=64, len_range=(30, 700), seed=18),
    # the widest query-head group the decode kernel takes (16), one not a power of two (6,
    # several key splits), and a wider one (32) that the engine sends down the prefill path
    "decode_g16_d64": W["gqa_decode_8k"].scaled(B=2, Hq=16, Hkv=1, Lk=600, D=64, len_range=(1, 600), seed=19),
    "decode_g6_d128": W["gqa_decode_8k"].scaled(B=2, Hq=12, Hkv=2, Lk=2100, len_range=(500, 2100), seed=20),
    "decode_g32_d128": W["gqa_decode_8k"].scaled(B=2, Hq=32, Hkv=1, Lk=300, len_range=(1, 300), seed=21),
    # sliding window of W keys up to the diagonal: whole key tiles before the window are
    # skipped and the window's first tile is cut per element; d = 64 without a mask runs the
    # one-launch backward, W = 1 leaves only the diagonal key, the decode skips leading splits
    "window_d64": W["mha_causal_1k"].scaled(B=2, Hq=3, Hkv=3, Lq=700, Lk=700, window=100, seed=50),
    "window_br_gqa_lens_d128": W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=2, Lq=300, Lk=700, causal=2,
                                                         lens="chunk", len_range=(100, 700),
                                                         window=150, seed=51),
    "window_1_d128": W["gqa_causal_4k"].scaled(B=1, Hq=2, Hkv=1, Lq=200, Lk=200, window=1, seed=52),
    "window_mask_d128": W["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=2, Lq=400, Lk=400, causal=True,
                                                   len_range=(64, 400), window=130, seed=53),
    "window_mask_br_d64": W["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=1, Lq=300, Lk=450, D=64, causal=2,
                                                     lens="chunk", len_range=(100, 450), window=77,
                                                     seed=54),
    "window_fp32": W["tiny_fp32"].scaled(B=2, Hq=4, Hkv=2, Lq=150, Lk=150, D=64, causal=True,
                                         window=70, seed=55),
    "window_fp32_br_lens": W["tiny_fp32"].scaled(B=2, Hq=2, Hkv=1, Lq=100, Lk=200, causal=2,
                                                 lens="chunk", len_range=(50, 200), window=45, seed=56),
    "decode_window_d128": W["gqa_decode_8k"].scaled(B=4, Hq=8, Hkv=2, Lk=3000, causal=2,
                                                    len_range=(1, 3000), window=1000, seed=57),
    "decode_window_d64": W["gqa_decode_8k"].scaled(B=3, Hq=4, Hkv=4, Lk=900, D=64, causal=2,
                                                   len_range=(30, 900), window=50, seed=58),
    # long enough that the forward without a mask runs key tiles that every wave sees whole
    # as its straight-line loop (groups of six 64-key tiles) before the per-block tested
    # rest: causal with lengths, a long cross-attention, and a window on the bottom-right
    # diagonal (the straight-line loop then starts at the window's first tile)
    "long_causal_lens_d128": W["gqa_causal_4k"].scaled(B=2, Hq=4, Hkv=2, Lq=900, Lk=900, lens="qkv",
                                                       len_range=(500, 900), seed=60),
    "long_cross_d64": W["mha_causal_1k"].scaled(B=1, Hq=2, Hkv=2, Lq=150, Lk=1000, causal=False,
                                                seed=61),
    "long_window_br_d128": W["gqa_causal_4k"].scaled(B=2, Hq=4, Hkv=2, Lq=600, Lk=1300, causal=2,
                                                     window=900, seed=62),
    # d = 128 without a diagonal or a mask (the dK/dV kernel that splits each key slice over
    # two waves): GQA cross-attention with ragged tails, then with per-batch key lengths
    "cross_gqa_d128": W["gqa_causal_4k"].scaled(B=2, Hq=4, Hkv=2, Lq=333, Lk=200, causal=False, seed=63),
    "cross_gqa_lens_d128": W["gqa_causal_4k"].scaled(B=3, Hq=4, Hkv=1, Lq=150, Lk=460, causal=False,
                                                     lens="kv", len_range=(1, 460), poison=True, seed=64),
    # the paired dK/dV loop's first and last phases with nothing between: one query tile
    # (40 rows, MHA), two (65 rows: a tile and a one-row tail) and, causal, a key range
    # whose last workgroup has keys for only some of its wave pairs (300 = 2*128 + 44)
    "one_q_tile_d128": W["gqa_causal_4k"].scaled(B=2, Hq=2, Hkv=2, Lq=40, Lk=300, causal=False, seed=65),
    "two_q_tiles_d128": W["gqa_causal_4k"].scaled(B=1, Hq=4, Hkv=2, Lq=65, Lk=300, causal=False, seed=66),
    "causal_pair_tail_d128": W["gqa_causal_4k"].scaled(B=1, Hq=2, Hkv=1, Lq=300, Lk=300, seed=67),
    "window_cross_d128": W["gqa_causal_4k"].scaled(B=2, Hq=4, Hkv=2, Lq=260, Lk=700, causal=2,
                                                   window=100, seed=68),
    # masks whose rows allow 16-byte copies (key count a multiple of 8), which the paired
    # dK/dV kernel stages per 32-row block: padded with lengths, the same mask only, a GQA
    # causal mask with Lq != Lk and a single query tile
    "padded_mask_vec_d128": W["padded_mask_2k"].scaled(B=3, Hq=2, Hkv=2, Lq=264, Lk=264,
                                                       len_range=(40, 264), seed=69),
    "padded_mask_vec_only_d128": W["padded_mask_2k"].scaled(B=3, Hq=2, Hkv=2, Lq=264, Lk=264,
                                                            len_range=(40, 264), seed=69, lens="none_keep"),
    "causal_mask_gqa_d128": W["padded_mask_2k"].scaled(B=2, Hq=4, Hkv=2, Lq=200, Lk=328, causal=2,
                                                       lens="chunk", len_range=(150, 328), seed=70),
    "mask_one_q_tile_d128": W["padded_mask_2k"].scaled(B=2, Hq=2, Hkv=2, Lq=40, Lk=40,
                                                       len_range=(1, 40), seed=71),
}


def _inputs(name):
    w = CASES[name]
    if w.lens == "none_keep":
        inp = make_inputs(w.scaled(lens="qkv"))
        inp["len_q"] = inp["len_kv"] = None
        return w, inp
    return w, make_inputs(w)


@pytest.mark.parametrize("name", list(CASES))
def test_parity(name, orc):
    w, inp = _inputs(name)
    banner(f"parity {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lq={w.Lq} Lk={w.Lk} D={w.D} {w.dtype} "
           f"causal={w.causal} window={w.window} mask={inp['mask'] is not None} "
           f"lens={inp['len_kv'] is not None}")
    d = to_dev(inp)
    o, lse = gpu_forward(d)
    o_ref, lse_ref = oracle_forward(orc, inp)
    e_o, e_l = compare_forward(inp, o, lse, o_ref, lse_ref)
    msg = f"O {e_o:.2e} LSE {e_l:.2e}"
    if w.backward:
        grads = gpu_backward(d, o, lse)
        dq, dk, dv, _ = oracle_backward(orc, inp)
        errs = compare_backward(inp, grads, (dq, dk, dv), lse_ref)
        msg += " dQ {:.2e} dK {:.2e} dV {:.2e}".format(*errs)
    banner(f"parity {name}: {msg}")


def _hand_padded(D=64):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_example.json")
    with open(path) as f:
        g = json.load(f)
    q = torch.zeros(1, 1, 1, D)
    k = torch.zeros(1, 1, 3, D)
    v = torch.zeros(1, 1, 3, D)
    dO = torch.zeros(1, 1, 1, D)
    q[0, 0, :, :4] = torch.tensor(g["q"], dtype=torch.float32)
    k[0, 0, :, :4] = torch.tensor(g["k"], dtype=torch.float32)
    v[0, 0, :, :2] = torch.tensor(g["v"], dtype=torch.float32)
    dO[0, 0, :, :2] = torch.tensor(g["dO"], dtype=torch.float32)
    return g, q, k, v, dO


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_hand_example_padded(path):
    """The worked example, zero-padded to d = 64 (all inputs exact in bf16), scale 0.5,
    against the page's printed values.  "decode" takes the Lq = 1 split-KV path; a zero
    additive mask routes the same problem through the prefill kernels."""
    from scaled_dot_product_sdpa_amd import sdpa_backward, sdpa_forward
    g, q, k, v, dO = _hand_padded()
    e = g["expected"]
    bf = lambda t: t.to(torch.bfloat16).cuda()
    mask = torch.zeros(1, 1, 1, 3, dtype=torch.bfloat16, device="cuda") if path == "prefill" else None
    banner(f"hand example via {path}")
    o, lse = sdpa_forward(bf(q), bf(k), bf(v), mask=mask, scale=g["scale"])
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().reshape(-1)
    assert np.abs(o[:2] - e["O"]).max() <= 4e-3 and np.all(o[2:] == 0)
    assert abs(lse.item() - np.log(1 + np.e + np.e ** 2)) <= 1e-3
    dq, dk, dv = sdpa_backward(bf(q), bf(k), bf(v), torch.tensor(o).reshape(1, 1, 1, -1).to(torch.bfloat16).cuda(),
                               bf(dO), lse, mask=mask, scale=g["scale"])
    torch.cuda.synchronize()
    dq = dq.float().cpu().numpy().reshape(-1)
    dk = dk.float().cpu().numpy().reshape(3, -1)
    dv = dv.float().cpu().numpy().reshape(3, -1)
    assert np.abs(dq[:4] - e["dQ"]).max() <= 2e-3 and np.all(dq[4:] == 0)
    assert np.abs(dk[:, :4] - np.array(e["dK"])).max() <= 2e-3 and np.all(dk[:, 4:] == 0)
    assert np.abs(dv[:, :2] - np.array(e["dV"])).max() <= 4e-3 and np.all(dv[:, 2:] == 0)
