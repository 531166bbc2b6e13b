"""Paged-KV decode (sdpa_decode_paged) on the GPU: the same result, bit for bit, as the
contiguous decode over the same cache, and the fp64 oracle's within the bf16 tolerances.
The cache is scattered into pages in a random order; pages no sequence uses are filled
with NaN, so a stray read would show."""

import pytest
import torch

from gpu_common import banner, compare_forward, gpu_forward, oracle_forward, to_dev
from scaled_dot_product_sdpa_amd import sdpa_decode_paged
from scaled_dot_product_sdpa_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _paged(inp, page_size, seed, token_major=False):
    """Scatter the contiguous (B, Hkv, Lk, D) cache into pages in a random order."""
    k, v, lens = inp["k"], inp["v"], inp["len_kv"]
    B, Hkv, Lk, D = k.shape
    max_pages = (Lk + page_size - 1) // page_size
    num_pages = B * max_pages + 3
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g)[: B * max_pages].view(B, max_pages)
    shape = (num_pages, page_size, Hkv, D) if token_major else (num_pages, Hkv, page_size, D)
    kp = torch.full(shape, float("nan"), dtype=k.dtype)
    vp = torch.full(shape, float("nan"), dtype=v.dtype)
    if token_major:  # (page, s, h, d) storage viewed as (page, h, s, d)
        kp, vp = kp.transpose(1, 2), vp.transpose(1, 2)
    for b in range(B):
        n = int(lens[b])
        for pg in range((n + page_size - 1) // page_size):
            s0, s1 = pg * page_size, min(n, (pg + 1) * page_size)
            kp[perm[b, pg], :, : s1 - s0] = k[b, :, s0:s1]
            vp[perm[b, pg], :, : s1 - s0] = v[b, :, s0:s1]
    return kp, vp, perm.to(torch.int32)


CASES = [
    # (B, Hq, Hkv, Lk, D, page_size, length range, token-major pages, sliding window)
    (4, 8, 2, 1100, 128, 64, (1, 1100), False, 0),
    (3, 16, 1, 700, 64, 32, (30, 700), True, 0),
    (2, 12, 2, 2100, 128, 256, (500, 2100), False, 0),
    (5, 32, 8, 1500, 128, 128, (0, 1500), True, 0),
    # the last W keys only: the window starts inside a page and inside a 32-key tile, and
    # skips whole key splits
    (4, 8, 2, 2100, 128, 64, (1, 2100), False, 700),
    (3, 4, 4, 900, 64, 32, (30, 900), True, 45),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_G{c[1] // c[2]}_D{c[4]}_ps{c[5]}_W{c[8]}")
def test_paged_decode_matches_contiguous_and_oracle(orc, case):
    B, Hq, Hkv, Lk, D, ps, lr, token_major, win = case
    w = WORKLOADS["gqa_decode_8k"].scaled(B=B, Hq=Hq, Hkv=Hkv, Lk=Lk, D=D, len_range=lr, seed=60 + ps,
                                          causal=2 if win else 0, window=win)
    inp = make_inputs(w)
    if lr[0] == 0:
        inp["len_kv"][1] = 0  # an empty cache: O = 0, LSE = -inf
    if win:
        # keys before the window (an evicted part of the cache) hold NaN, in the contiguous
        # cache and in the pages alike: the window's first 32-key tile starts below its first
        # key, and none of those rows may reach O (0 * NaN)
        for b, n in enumerate(inp["len_kv"].tolist()):
            inp["k"][b, :, : max(n - win, 0)] = float("nan")
            inp["v"][b, :, : max(n - win, 0)] = float("nan")
    banner(f"paged decode B={B} Hq={Hq} Hkv={Hkv} Lk={Lk} D={D} page={ps} token_major={token_major} "
           f"window={win}")
    kp, vp, table = _paged(inp, ps, seed=70 + ps, token_major=token_major)
    d = to_dev(inp)
    o_c, l_c = gpu_forward(d)
    o_p, l_p = sdpa_decode_paged(d["q"][:, :, 0], kp.cuda(), vp.cuda(), table.cuda(), d["len_kv"],
                                 scale=inp["scale"], sliding_window=win)
    torch.cuda.synchronize()
    assert torch.isfinite(o_p).all() and torch.isfinite(o_c).all()
    assert torch.equal(o_p, o_c[:, :, 0]) and torch.equal(l_p, l_c[:, :, 0])
    o_ref, lse_ref = oracle_forward(orc, inp)
    compare_forward(inp, o_p.unsqueeze(2), l_p.unsqueeze(2), o_ref, lse_ref)
