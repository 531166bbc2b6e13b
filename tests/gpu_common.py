"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI binding, run
the fp64 oracle on the same (bf16-rounded) inputs, and compare to the stated tolerances.

Tolerances (fp64 oracle as the reference):
  fp32 path:  max-abs 1e-5 on O, LSE, dQ, dK, dV.
  bf16 path:  O max-abs <= 1e-2, LSE max-abs <= 1e-3 (over finite entries; -inf must match
              exactly), dQ/dK/dV relative Frobenius error <= 2e-2.
  Rows with no visible key: O, dQ exactly 0 and LSE exactly -inf on both sides.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-5
TOL_BF16_O = 1e-2
TOL_BF16_LSE = 1e-3
TOL_BF16_GRAD_REL = 2e-2


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inp: dict, device="cuda") -> dict:
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device) if torch.is_tensor(val) else val
    return out


def f64(t):
    return None if t is None else t.detach().double().cpu().numpy()


def i32(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.int32)


def gpu_forward(inp):
    from scaled_dot_product_sdpa_amd import sdpa_forward
    o, lse = sdpa_forward(inp["q"], inp["k"], inp["v"], mask=inp.get("mask"), scale=inp["scale"],
                          is_causal=inp["is_causal"], seq_lens_q=inp.get("len_q"),
                          seq_lens_kv=inp.get("len_kv"), sliding_window=inp.get("window", 0))
    torch.cuda.synchronize()
    return o, lse


def gpu_backward(inp, o, lse):
    from scaled_dot_product_sdpa_amd import sdpa_backward
    g = sdpa_backward(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, mask=inp.get("mask"),
                      scale=inp["scale"], is_causal=inp["is_causal"], seq_lens_q=inp.get("len_q"),
                      seq_lens_kv=inp.get("len_kv"), sliding_window=inp.get("window", 0))
    torch.cuda.synchronize()
    return g


def oracle_args(inp):
    return dict(mask=f64(inp.get("mask")), scale=inp["scale"], is_causal=inp["is_causal"],
                len_q=i32(inp.get("len_q")), len_kv=i32(inp.get("len_kv")), window=inp.get("window", 0))


def oracle_forward(orc, inp):
    return orc.forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), **oracle_args(inp))


def oracle_backward(orc, inp):
    return orc.backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dO"]), **oracle_args(inp))


def check_lse(lse_gpu, lse_ref, tol, what="LSE"):
    lg = np.asarray(lse_gpu, dtype=np.float64)
    lr = np.asarray(lse_ref, dtype=np.float64)
    ninf_ref = np.isneginf(lr)
    ninf_gpu = np.isneginf(lg)
    assert np.array_equal(ninf_ref, ninf_gpu), f"{what}: -inf pattern differs ({ninf_ref.sum()} vs {ninf_gpu.sum()})"
    fin = ~ninf_ref
    assert np.isfinite(lg[fin]).all(), f"{what}: non-finite values"
    err = np.abs(lg[fin] - lr[fin]).max() if fin.any() else 0.0
    assert err <= tol, f"{what}: max-abs {err:.3e} > {tol:.1e}"
    return err


def check_out(o_gpu, o_ref, lse_ref, tol, what="O"):
    og = np.asarray(o_gpu, dtype=np.float64)
    orf = np.asarray(o_ref, dtype=np.float64)
    assert np.isfinite(og).all(), f"{what}: non-finite values"
    diff = np.abs(og - orf)
    err = diff.max() if diff.size else 0.0
    if err > tol:
        idx = np.unravel_index(np.argmax(diff), diff.shape)
        raise AssertionError(f"{what}: max-abs {err:.3e} > {tol:.1e} at {idx} (gpu {og[idx]}, ref {orf[idx]})")
    empty = np.isneginf(np.asarray(lse_ref))
    if empty.any():
        assert np.all(og[empty] == 0.0), f"{what}: rows with no visible key are not exactly 0"
    return err


def rel_fro(g, ref):
    g = np.asarray(g, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(g - ref)
    return num / den if den > 0 else num


def check_grad(g_gpu, g_ref, dtype, what):
    g = np.asarray(g_gpu, dtype=np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    if dtype == torch.float32:
        err = np.abs(g - g_ref).max() if g.size else 0.0
        assert err <= TOL_F32, f"{what}: max-abs {err:.3e} > {TOL_F32:.1e}"
    else:
        err = rel_fro(g, g_ref)
        assert err <= TOL_BF16_GRAD_REL, f"{what}: rel Frobenius {err:.3e} > {TOL_BF16_GRAD_REL:.1e}"
    return err


def compare_forward(inp, o, lse, o_ref, lse_ref):
    f32 = inp["q"].dtype == torch.float32
    e_o = check_out(f64(o), o_ref, lse_ref, TOL_F32 if f32 else TOL_BF16_O)
    e_l = check_lse(f64(lse), lse_ref, TOL_F32 if f32 else TOL_BF16_LSE)
    return e_o, e_l


def compare_backward(inp, grads, refs, lse_ref=None):
    dt = inp["q"].dtype
    errs = []
    for g, r, n in zip(grads, refs, ("dQ", "dK", "dV")):
        errs.append(check_grad(f64(g), r, dt, n))
    if lse_ref is not None:
        empty = np.isneginf(lse_ref)
        if empty.any():
            assert np.all(f64(grads[0])[empty] == 0.0), "dQ of rows with no visible key is not exactly 0"
    return errs
