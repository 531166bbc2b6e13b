"""Seeded synthetic inputs for the attention workloads (shared by tests, smoke and bench).

This module only draws numbers: it holds none of the attention arithmetic.  Every
workload is a dict of CPU tensors; bf16 workloads are drawn in fp32 and rounded to bf16
(round-to-nearest-even), so the fp64 oracle can read exactly the values the GPU gets.

Draw order per workload (one ``torch.Generator`` seeded with the workload's seed):
q, k, v, dO ~ N(0, 1) in (B, H, L, D) order, then the per-batch lengths, then the
Bernoulli draws of the random mask.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lk: int
    D: int
    dtype: str                 # "f32" or "bf16"
    causal: int                # 0 none, 1 (True) top-left, 2 bottom-right diagonal
    scale: float
    seed: int
    lens: str = "none"         # "none" | "qkv" (same length for q and kv) | "kv" | "chunk"
                               # (kv lengths, then query lengths <= min(Lq, len_kv): a chunk
                               # of queries at the end of each sequence)
    len_range: tuple = (0, 0)  # inclusive range of the uniform length draw
    mask: str = "none"         # "none" | "padded_random" (B,1,Lq,Lk) additive mask
    mask_drop: float = 0.0     # Bernoulli rate of extra -inf entries inside the lengths
    poison: bool = False       # fill K/V rows at or past len_kv with NaN
    window: int = 0            # sliding window of this many keys up to the diagonal (0: none)
    backward: bool = True
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, Hq=2, Hkv=2, Lq=64, Lk=64, D=32, dtype="f32",
                          causal=False, scale=1 / math.sqrt(32), seed=1,
                          note="fp32, no mask; run again with causal=True"),
    "mha_causal_1k": Workload("mha_causal_1k", B=4, Hq=16, Hkv=16, Lq=1024, Lk=1024, D=64,
                              dtype="bf16", causal=True, scale=1 / 8, seed=2),
    "gqa_causal_4k": Workload("gqa_causal_4k", B=2, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128,
                              dtype="bf16", causal=True, scale=1 / math.sqrt(128), seed=3),
    "padded_mask_2k": Workload("padded_mask_2k", B=8, Hq=16, Hkv=16, Lq=2048, Lk=2048, D=128,
                               dtype="bf16", causal=False, scale=1 / math.sqrt(128), seed=4,
                               lens="qkv", len_range=(256, 2048), mask="padded_random",
                               mask_drop=0.1),
    # measured beside the configurations above: a sliding window of 1024 keys over the GQA
    # 4k prefill, and a 512-query prefill chunk against a 4096-key cache (bottom-right)
    "gqa_swa_4k": Workload("gqa_swa_4k", B=2, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128,
                           dtype="bf16", causal=True, scale=1 / math.sqrt(128), seed=6,
                           window=1024),
    "gqa_chunk_4k": Workload("gqa_chunk_4k", B=2, Hq=32, Hkv=8, Lq=512, Lk=4096, D=128,
                             dtype="bf16", causal=2, scale=1 / math.sqrt(128), seed=7),
    "gqa_decode_8k": Workload("gqa_decode_8k", B=64, Hq=32, Hkv=8, Lq=1, Lk=8192, D=128,
                              dtype="bf16", causal=False, scale=1 / math.sqrt(128), seed=5,
                              lens="kv", len_range=(1024, 8192), poison=True, backward=False),
}


def make_inputs(w: Workload, device="cpu") -> dict:
    """Draw the workload's inputs in the workload's dtype.

    ``device="cpu"`` uses torch's CPU generator; another device draws with that device's
    generator (same seed and draw order, different stream of numbers), which is how the
    full-size workloads are made without a host round trip.  Either way every consumer,
    the oracle included, reads the very tensors drawn here."""
    g = torch.Generator(device=device).manual_seed(w.seed)
    dt = w.torch_dtype
    kw = dict(generator=g, device=device)
    q = torch.randn(w.B, w.Hq, w.Lq, w.D, **kw).to(dt)
    k = torch.randn(w.B, w.Hkv, w.Lk, w.D, **kw).to(dt)
    v = torch.randn(w.B, w.Hkv, w.Lk, w.D, **kw).to(dt)
    dO = torch.randn(w.B, w.Hq, w.Lq, w.D, **kw).to(dt) if w.backward else None

    len_q = len_kv = None
    if w.lens != "none":
        lo, hi = w.len_range
        lens = torch.randint(lo, hi + 1, (w.B,), dtype=torch.int32, **kw)
        len_kv = lens.clone()
        if w.lens == "qkv":
            len_q = lens.clone()
        elif w.lens == "chunk":
            u = torch.rand(w.B, **kw)
            cap = torch.clamp(lens, max=w.Lq).to(torch.float32)
            len_q = torch.minimum(torch.floor(u * (cap + 1)), cap).to(torch.int32)

    mask = None
    if w.mask == "padded_random":
        # -inf outside each batch's length (rows and columns), plus independent
        # Bernoulli(mask_drop) -inf entries inside it, plus one fully masked in-length row.
        L, S = w.Lq, w.Lk
        lens_b = len_kv if len_kv is not None else torch.full((w.B,), S, dtype=torch.int32, device=device)
        ii = torch.arange(L, device=device).view(1, L, 1)
        jj = torch.arange(S, device=device).view(1, 1, S)
        lb = lens_b.view(-1, 1, 1).long()
        blocked = (ii >= lb) | (jj >= lb)
        drop = torch.rand(w.B, L, S, **kw) < w.mask_drop
        blocked = blocked | drop
        row = int(lens_b[0]) // 2
        blocked[0, row, :] = True
        mask = torch.zeros(w.B, 1, L, S, dtype=torch.float32, device=device)
        mask.masked_fill_(blocked.view(w.B, 1, L, S), float("-inf"))
        mask = mask.to(dt)

    if w.poison and len_kv is not None:
        for b, n in enumerate(len_kv.tolist()):
            k[b, :, n:, :] = float("nan")
            v[b, :, n:, :] = float("nan")

    return dict(q=q, k=k, v=v, dO=dO, mask=mask, len_q=len_q, len_kv=len_kv,
                scale=w.scale, is_causal=w.causal, window=w.window)


def fully_masked_rows(inputs: dict) -> list:
    """(b, i) pairs whose every key is blocked by the additive mask (all heads)."""
    m = inputs["mask"]
    if m is None:
        return []
    allneg = torch.isinf(m.float()).all(dim=-1)  # (B, 1 or H, Lq)
    out = []
    for b, h, i in allneg.nonzero().tolist():
        out.append((b, i))
    return sorted(set(out))
