#!/usr/bin/env python3
"""Benchmark of the scaled dot-product attention hot path on one MI355X.

One step = the whole hot path over one batch of the headline workload (causal GQA
prefill, B=2, Hq=32, Hkv=8, L=4096, d=128, bf16, the largest workload): forward (O, LSE)
then backward (D prep, dK/dV, dQ).  The step is captured once into a HIP graph and
replayed; inputs are resident in HBM before the timed region starts.  Prints ONE JSON line.

Also reported (same line, "workloads"): the other workloads' forward / backward TFLOP/s
and the GQA decode's HBM GB/s, each with the roofline of its dominant kernel, the
per-kernel durations (HIP events around graph replays of that kernel alone), and the fp64
CPU oracle timed on the host cores as a baseline.

FLOP convention: pairs (i, j) a query may attend to (causal and lengths applied, the
random mask entries not subtracted); forward 2 (Dqk + Dv) flops per pair, backward
2 (3 Dqk + 2 Dv).  Decode GB/s counts the K/V rows read (valid lengths), q, o and lse.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "SDPA fwd / fwd+bwd TFLOP/s (+% bf16 MFMA peak); decode GB/s (+% HBM)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
HEADLINE = "gqa_causal_4k"
EXTRA = ["mha_causal_1k", "padded_mask_2k", "gqa_decode_8k", "tiny_fp32", "gqa_swa_4k", "gqa_chunk_4k"]

# kernel-name fragments (as rocprofv3 reports them) of each launch stage
KERNEL_NAMES = {
    "fwd": "fwd_bf16_kernel", "prep": "bwd_prep_kernel", "dkdv": "bwd_dkdv_",
    "dq": "bwd_dq_", "main": "bwd_fused_kernel", "decode_split": "decode_split_kernel",
    "decode_combine": "decode_combine_kernel",
}
# source file of each kernel (traffic counters are dropped once the source changes)
KERNEL_SOURCES = {
    "fwd": "fwd_bf16.hip", "prep": "bwd_bf16.hip", "dkdv": "bwd_bf16.hip", "dq": "bwd_bf16.hip",
    "main": "bwd_bf16.hip",
    "decode_split": "decode_bf16.hip", "decode_combine": "decode_bf16.hip",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(stage: str) -> str:
    src = ROOT / "scaled_dot_product_sdpa_amd" / "csrc" / KERNEL_SOURCES[stage]
    h = hashlib.sha256(src.read_bytes())
    h.update((ROOT / "scaled_dot_product_sdpa_amd" / "csrc" / "kern_common.h").read_bytes())
    return h.hexdigest()[:16]


def visible_pairs(w, len_q=None, len_kv=None) -> int:
    """Number of (b, h, i, j) a query may attend to under the causal diagonal (top-left or
    bottom-right), the sliding window and the lengths."""
    import numpy as np
    lq = np.full(w.B, w.Lq) if len_q is None else np.asarray(len_q.cpu()).astype(np.int64)
    lk = np.full(w.B, w.Lk) if len_kv is None else np.asarray(len_kv.cpu()).astype(np.int64)
    total = 0
    for b in range(w.B):
        i = np.arange(int(lq[b]))
        if w.causal:
            off = int(lk[b] - lq[b]) if w.causal == 2 else 0
            hi = np.clip(i + 1 + off, 0, lk[b])
            lo = np.maximum(i + off - w.window + 1, 0) if w.window > 0 else 0
            n = np.maximum(hi - lo, 0)
        else:
            n = np.full(i.shape, lk[b])
        total += int(n.sum())
    return total * w.Hq


def flops(w, pairs):
    fwd = 2 * (w.D + w.D) * pairs
    bwd = 2 * (3 * w.D + 2 * w.D) * pairs
    # per-kernel algorithmic shares of the backward: dK/dV does S, dP, dV, dK; dQ adds dQ
    # (the one-launch dK/dV + dQ kernel does all of the backward's matrix products)
    return {"fwd": fwd, "bwd": bwd, "dkdv": 2 * (2 * w.D + 2 * w.D) * pairs, "dq": 2 * w.D * pairs,
            "main": bwd}


def fused_backward(w, has_mask) -> bool:
    """Whether the library runs dK/dV and dQ in one launch for this workload (d = 64, bf16,
    no mask), as sdpa_backward_main documents."""
    return w.dtype == "bf16" and w.D == 64 and not has_mask


class Timer:
    """Graph-replay timing on the current stream with HIP events."""

    def __init__(self, torch):
        self.torch = torch

    def capture(self, fn, reps=1):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()  # warm the launch path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, iters, warmup=2):
        torch = self.torch
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters  # ms per replay


def kernel_ms(timer, fn, reps=20, iters=5):
    """Average duration of one launch of fn: a graph of `reps` back-to-back launches."""
    g = timer.capture(fn, reps=reps)
    return timer.time_graph(g, iters) / reps


def run_workload(torch, timer, name, w, iters, want_bwd=True):
    """Per-stage kernel times and throughput of one workload."""
    from scaled_dot_product_sdpa_amd import BackwardCall, ForwardCall
    from scaled_dot_product_sdpa_amd.workloads import make_inputs
    inp = make_inputs(w, device="cuda")
    fc = ForwardCall(inp["q"], inp["k"], inp["v"], inp["mask"], inp["scale"], inp["is_causal"],
                     inp["len_q"], inp["len_kv"], sliding_window=w.window)
    fc.launch()
    torch.cuda.synchronize()
    res = {"config": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq, "Lk": w.Lk, "D": w.D,
                      "causal": w.causal, "window": w.window, "mask": inp["mask"] is not None,
                      "lens": inp["len_kv"] is not None, "dtype": w.dtype}}
    t = {"fwd": kernel_ms(timer, fc.launch, reps=10, iters=iters)}
    if w.Lq == 1:
        # decode: algorithmic bytes = K/V rows within the lengths + q + o + lse
        lk = inp["len_kv"].to(torch.int64).sum().item() if inp["len_kv"] is not None else w.B * w.Lk
        nbytes = lk * w.Hkv * 2 * w.D * 2 + w.B * w.Hq * (2 * w.D * 2 + 4)
        gbs = nbytes / (t["fwd"] * 1e-3) / 1e9
        res.update(ms={"fwd": t["fwd"]}, bytes=nbytes, GBps=gbs, hbm_frac=gbs / PEAK_HBM_GBS)
        if inp["len_kv"] is not None and w.dtype == "bf16":
            # the same cache stored in 64-key pages in a random page order (paged decode)
            from scaled_dot_product_sdpa_amd import PagedDecodeCall
            ps = 64
            max_pages = (w.Lk + ps - 1) // ps
            g = torch.Generator(device="cuda").manual_seed(w.seed)
            table = torch.randperm(w.B * max_pages, generator=g, device="cuda").view(w.B, max_pages)
            pages = lambda t: t.new_empty(w.B * max_pages, w.Hkv, ps, w.D).index_copy_(
                0, table.reshape(-1),
                t.view(w.B, w.Hkv, max_pages, ps, w.D).transpose(1, 2).reshape(-1, w.Hkv, ps, w.D))
            pc = PagedDecodeCall(inp["q"][:, :, 0], pages(inp["k"]), pages(inp["v"]),
                                 table.to(torch.int32), inp["len_kv"], inp["scale"])
            pc.launch()
            torch.cuda.synchronize()
            assert torch.equal(pc.o, fc.o[:, :, 0]), "paged decode differs from the contiguous one"
            t_p = kernel_ms(timer, pc.launch, reps=10, iters=iters)
            res["ms"]["paged_fwd"] = t_p
            res["GBps_paged"] = nbytes / (t_p * 1e-3) / 1e9
            res["paged"] = {"page_size": ps, "page_order": "random permutation"}
        return res, inp, fc, None
    pairs = visible_pairs(w, inp["len_q"], inp["len_kv"])
    fl = flops(w, pairs)
    bc = None
    if want_bwd and w.backward:
        o, lse = fc.result()
        bc = BackwardCall(inp["q"], inp["k"], inp["v"], o, inp["dO"], lse, inp["mask"],
                          inp["scale"], inp["is_causal"], inp["len_q"], inp["len_kv"],
                          sliding_window=w.window)
        bc.launch()
        torch.cuda.synchronize()
        # prep and the two main passes as the library runs them ("main": one launch at
        # d = 64 without a mask), and the two passes as separate launches for reference
        for st in ("prep", "main", "dkdv", "dq"):
            t[st] = kernel_ms(timer, lambda st=st: bc.launch(st), reps=10, iters=iters)
        t["bwd"] = t["prep"] + t["main"]
        res["fused_backward"] = fused_backward(w, inp["mask"] is not None)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    tf = {"fwd": fl["fwd"] / (t["fwd"] * 1e-3) / 1e12}
    if "bwd" in t:
        tf["bwd"] = fl["bwd"] / (t["bwd"] * 1e-3) / 1e12
        tf["fwd+bwd"] = (fl["fwd"] + fl["bwd"]) / ((t["fwd"] + t["bwd"]) * 1e-3) / 1e12
    res.update(pairs=pairs, gflop={k: v / 1e9 for k, v in fl.items()}, ms=t, TFLOPs=tf,
               peak_frac={k: v / peak for k, v in tf.items()})
    return res, inp, fc, bc


def cpu_baseline(w, inp):
    """The fp64 oracle (as it stands) on the host cores, on one whole step of the headline
    workload (forward over every row, backward over every (batch, KV head) group); the
    backward runs one group per thread, so one step takes about 30 s on 16 threads."""
    from oracle import load_oracle
    orc = load_oracle()
    f = lambda t: None if t is None else t.detach().double().cpu().numpy()
    q, k, v, dO = f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["dO"])
    t0 = time.perf_counter()
    orc.forward(q, k, v, scale=w.scale, is_causal=w.causal)
    t1 = time.perf_counter()
    orc.backward(q, k, v, dO, scale=w.scale, is_causal=w.causal)
    t2 = time.perf_counter()
    fl = flops(w, visible_pairs(w))
    return {"value": (fl["fwd"] + fl["bwd"]) / (t2 - t0) / 1e12, "unit": "TFLOP/s",
            "cores": orc.num_threads, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"one whole {HEADLINE} step (fwd over all {w.B}x{w.Hq} heads' rows, bwd over all "
                      f"{w.B}x{w.Hkv} (batch, KV head) groups), fp64, {t2 - t0:.1f} s",
            "seconds": {"fwd": t1 - t0, "bwd": t2 - t1}}


def traffic_for(workload, stage):
    """HBM bytes per launch of one kernel of a workload from the committed rocprofv3
    counter summary, if it was taken on the current source of that kernel (else None)."""
    path = ROOT / "profiles" / "traffic.json"
    if not path.exists():
        return None
    try:
        data = json.loads(path.read_text())
    except ValueError:
        return None
    ent = data.get(workload, {}).get(stage) if isinstance(data.get(workload), dict) else None
    if not ent or ent.get("source_hash") != source_hash(stage):
        return None
    return ent.get("bytes_per_launch")


def roofline(name, w, res):
    """Roofline of a workload's dominant kernel: algorithmic flops (or bytes) of one launch
    over its measured average duration, against the published peak."""
    t = res["ms"]
    if w.Lq == 1:
        # decode: the split kernel streams the cache; the call's time (split + combine) is
        # the duration, the algorithmic bytes those of the whole call
        return {"bound": "hbm", "achieved": res["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": res["GBps"] / PEAK_HBM_GBS, "traffic": traffic_for(name, "decode_split"),
                "kernel": "decode_split_kernel + decode_combine_kernel", "kernel_ms": t["fwd"]}
    stages = ("fwd", "prep", "main") if res.get("fused_backward") else ("fwd", "prep", "dkdv", "dq")
    kt = {k: t[k] for k in stages if k in t}
    dom = max(kt, key=kt.get)
    if dom == "prep":
        nbytes = w.B * w.Hq * w.Lq * (2 * w.D * 2 + 4 + 2 * 4)
        roof = {"bound": "hbm", "achieved": nbytes / (kt[dom] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        roof = {"bound": "mfma" if w.dtype == "bf16" else "alu",
                "achieved": res["gflop"][dom] * 1e9 / (kt[dom] * 1e-3) / 1e12,
                "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic_for(name, dom)
    kname = KERNEL_NAMES[dom]
    if dom == "dq":  # at d = 128 dQ is formed from the dS blocks the dK/dV pass stored
        kname = "bwd_dq_ds_kernel" if w.D == 128 else "bwd_dq_kernel"
    if dom == "dkdv":  # at d = 128 each key slice is split over two waves (the workloads' masks
        kname = "bwd_dkdv_pair_kernel" if w.D == 128 else "bwd_dkdv_kernel"  # allow 16-byte copies)
    if w.dtype == "f32":  # the fp32 path's kernels (main: its dK/dV and dQ kernels)
        kname = {"fwd": "fwd_f32_kernel", "prep": "bwd_prep_f32_kernel", "dkdv": "bwd_dkdv_f32_kernel",
                 "dq": "bwd_dq_f32_kernel"}.get(dom, kname)
    roof["kernel"] = kname
    roof["kernel_ms"] = kt[dom]
    return roof


def cpu_model() -> str:
    try:
        for ln in Path("/proc/cpuinfo").read_text().splitlines():
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---- profile helpers (no GPU): turn rocprofv3 output into the committed summaries ----

COPY_KERNELS = ("__amd_rocclr_copyBuffer", "copy_kernel")
# The decode kernels read the KV cache with non-temporal buffer loads, which the counters
# see differently from the copy's loads; their counters are scaled by what the same counter
# reads for the HBM streaming probe (ceilings.hip) in that load form over a known size.
STREAM_CAL_KERNEL = "ceil_stream"
STREAM_CAL_BYTES = 2 * (256 << 20)  # two 256 MiB streams
STREAM_CAL_STAGES = ("decode_split",)
CALIBRATION_BYTES = 1 << 30  # the --calibrate device copy: 1 GiB read and 1 GiB written


def _pmc_rows(directory, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(fetch_dir, write_dir, command, workload, l2_dir=None):
    """profiles/traffic.json, entry `workload`: HBM bytes per launch of each of its kernels,
    from a FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch) of a bench command that
    runs that workload alone, each counter scaled by what it reads for the --calibrate copy
    of known size; with l2_dir (a TCC_HIT_sum, TCC_MISS_sum run of the same command) also
    each kernel's L2 hit rate, hits / (hits + misses) over its dispatches."""
    path = ROOT / "profiles" / "traffic.json"
    data = {}
    if path.exists():
        try:
            data = json.loads(path.read_text())
        except ValueError:
            data = {}
    data = {k: v for k, v in data.items() if isinstance(v, dict) and k != workload}
    out = {"command": command}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        cal = [v for n, v in rows if any(c in n for c in COPY_KERNELS)]
        if not cal:
            raise SystemExit(f"no calibration copy kernel in {d}")
        scale = CALIBRATION_BYTES / (max(cal) * 1024.0)
        out[counter.lower() + "_scale"] = round(scale, 4)
        cal_nt = [v for n, v in rows if STREAM_CAL_KERNEL in n]
        scale_nt = None
        if cal_nt and counter == "FETCH_SIZE":
            scale_nt = STREAM_CAL_BYTES / (max(cal_nt) * 1024.0)
            out["fetch_size_scale_nontemporal"] = round(scale_nt, 4)
        for stage, frag in KERNEL_NAMES.items():
            vals = [v for n, v in rows if frag in n and "sdpa::" in n]
            if vals:
                sc = scale_nt if (scale_nt and stage in STREAM_CAL_STAGES) else scale
                per.setdefault(stage, {})[counter] = (sum(vals) / len(vals), len(vals), sc, scale)
    for stage, c in per.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        (fk, fn, fs, fcopy), (wk, wn, ws, _) = c["FETCH_SIZE"], c["WRITE_SIZE"]
        out[stage] = {"kernel": KERNEL_NAMES[stage], "source_hash": source_hash(stage),
                      "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                      "dispatches": min(fn, wn),
                      "bytes_per_launch": int(fk * 1024 * fs + wk * 1024 * ws)}
        if fs != fcopy:
            out[stage]["bytes_per_launch_copy_scale"] = int(fk * 1024 * fcopy + wk * 1024 * ws)
    if l2_dir:
        # the FETCH_SIZE run's command with the L2 counters and their output folder
        out["l2_command"] = (command.split(" ; ")[0].replace("--pmc FETCH_SIZE", "--pmc TCC_HIT_sum TCC_MISS_sum")
                             .replace("pmc_FETCH_SIZE_", "pmc_L2_"))
        hits, misses = _pmc_rows(l2_dir, "TCC_HIT_sum"), _pmc_rows(l2_dir, "TCC_MISS_sum")
        for stage, frag in KERNEL_NAMES.items():
            h = sum(v for n, v in hits if frag in n and "sdpa::" in n)
            m = sum(v for n, v in misses if frag in n and "sdpa::" in n)
            if stage in out and h + m > 0:
                out[stage]["l2_hit_pct"] = round(100.0 * h / (h + m), 1)
    data[workload] = out
    data["note"] = {"text": "per workload: HBM bytes per launch = counter KiB * 1024 * scale, scale = "
                            "known bytes of the calibration copy / its counter bytes; the decode split "
                            "kernel's FETCH_SIZE takes the scale of the streaming probe in its load form "
                            "(non-temporal buffer loads) instead"}
    path.write_text(json.dumps(data, indent=1) + "\n")
    print(json.dumps(out, indent=1))


def summarize_trace(stats_csv, out_md, command):
    """Short markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv."""
    import csv
    rows = []
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e6))
    lines = ["# rocprofv3 kernel trace summary", "",
             "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | total ms |",
             "|---|---:|---:|---:|---:|---:|"]
    for n, c, a, mn, mx, tot in sorted(rows, key=lambda r: -r[5]):
        if "sdpa::" not in n:
            continue
        n = n.replace("void sdpa::(anonymous namespace)::", "")
        n = re.sub(r"\(sdpa::\w+(, int)?\)$", "", n)  # the argument list
        lines.append(f"| `{n}` | {c} | {a:.2f} | {mn:.2f} | {mx:.2f} | {tot:.3f} |")
    Path(out_md).write_text("\n".join(lines) + "\n")
    print(Path(out_md).read_text())


# Derived per-kernel figures from SQ/GRBM counters, with rocprofv3's own definitions
# (256 CUs, 1024 SIMDs on the MI355X): MFMA busy = MFMA busy cycles over all SIMDs'
# active cycles; VALU busy = VALU-active cycles per CU over active cycles; LDS bank
# conflict = conflict-stall cycles per CU over active cycles; mean waves per CU from the
# wave-cycle count (sampled every 4 cycles).  The csv gives GRBM_GUI_ACTIVE summed over
# the 8 XCDs (8x the dispatch's cycles); the definitions take one XCD's, hence the / 8.
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8
COUNTER_COLUMNS = [
    ("clock GHz", lambda c: c["GRBM_GUI_ACTIVE"] / XCD_NUM / c["ns"]),
    ("MFMA busy %", lambda c: 100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCD_NUM * SIMD_NUM)),
    ("VALU busy %", lambda c: 100 * c["SQ_ACTIVE_INST_VALU"] / CU_NUM / (c["GRBM_GUI_ACTIVE"] / XCD_NUM)),
    ("LDS bank-conflict %", lambda c: 100 * c["SQ_LDS_BANK_CONFLICT"] / CU_NUM / (c["GRBM_GUI_ACTIVE"] / XCD_NUM)),
    ("waves / CU", lambda c: 4 * c["SQ_WAVE_CYCLES"] / CU_NUM / (c["GRBM_GUI_ACTIVE"] / XCD_NUM)),
    ("MFMA instr (M)", lambda c: c["SQ_INSTS_MFMA"] / 1e6),
    ("VALU instr / MFMA instr", lambda c: c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"] if c["SQ_INSTS_MFMA"] else None),
    ("LDS instr / MFMA instr", lambda c: c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"] if c["SQ_INSTS_MFMA"] else None),
]
COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT",
            "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]


def summarize_counters(pmc_dir, out_md, command):
    """Markdown table of per-kernel averages of the COUNTERS pass and the figures derived
    from them (COUNTER_COLUMNS)."""
    import csv
    import glob
    per = {}  # kernel -> dispatch -> counter -> value
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                n = r["Kernel_Name"]
                if "sdpa::" not in n:
                    continue
                d = per.setdefault(n, {}).setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    lines = ["# rocprofv3 counters per kernel", "",
             "Command (from the repository root, one MI355X):", "", "```", command, "```", "",
             "Per-kernel means over its dispatches. " + "; ".join(
                 ["A = GRBM_GUI_ACTIVE / 8 (the csv sums it over the 8 XCDs)",
                  "clock = A / dispatch duration",
                  "MFMA busy = 100·SQ_VALU_MFMA_BUSY_CYCLES / (A·1024 SIMDs)",
                  "VALU busy = 100·SQ_ACTIVE_INST_VALU / 256 CUs / A",
                  "LDS bank-conflict = 100·SQ_LDS_BANK_CONFLICT / 256 / A",
                  "waves / CU = 4·SQ_WAVE_CYCLES / 256 / A",
                  "MFMA instr = SQ_INSTS_MFMA per dispatch (millions)"]) + ". For dispatches "
             "of a few tens of microseconds GRBM_GUI_ACTIVE also counts cycles around the kernel "
             "(the clock column then reads above the real ~2 GHz), so their busy and wave figures "
             "are low by that factor.", "",
             "| kernel | dispatches | " + " | ".join(c for c, _ in COUNTER_COLUMNS) + " |",
             "|---|---:|" + "---:|" * len(COUNTER_COLUMNS)]
    table = []
    for n, disp in per.items():
        full = [d for d in disp.values() if all(k in d for k in COUNTERS)]
        if not full:
            continue
        mean = {k: sum(d[k] for d in full) / len(full) for k in COUNTERS + ["ns"]}
        name = n.replace("void sdpa::(anonymous namespace)::", "")
        name = re.sub(r"\(sdpa::\w+(, int)?\)$", "", name)
        table.append((mean["GRBM_GUI_ACTIVE"] * len(full), f"| `{name}` | {len(full)} | " +
                      " | ".join("–" if fn(mean) is None else f"{fn(mean):.2f}"
                                 for _, fn in COUNTER_COLUMNS) + " |"))
    lines += [t for _, t in sorted(table, key=lambda t: -t[0])]
    Path(out_md).write_text("\n".join(lines) + "\n")
    print(Path(out_md).read_text())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the live MFMA / HBM ceiling probes (libceilings.so)")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline step (with --only: profile other workloads alone)")
    ap.add_argument("--only", default=None, help="comma list of extra workloads to run")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run one 1 GiB device copy (the reference for HBM counters)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COMMAND", "WORKLOAD"),
                    help="add WORKLOAD to profiles/traffic.json from two rocprofv3 --pmc runs (no GPU)")
    ap.add_argument("--l2-dir", default=None,
                    help="with --write-traffic: a TCC_HIT_sum TCC_MISS_sum --pmc run of the same command")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "OUT_MD", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 kernel_stats.csv (no GPU)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("PMC_DIR", "OUT_MD", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 --pmc run of COUNTERS (no GPU)")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic, l2_dir=args.l2_dir)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    from scaled_dot_product_sdpa_amd import load_library
    from scaled_dot_product_sdpa_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    load_library()
    timer = Timer(torch)
    w = WORKLOADS[HEADLINE]
    if args.calibrate:
        src = torch.empty(CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        # reads of a known size in the decode kernel's load form (see STREAM_CAL_KERNEL)
        import ctypes
        from scaled_dot_product_sdpa_amd.build import CEIL_LIB
        if CEIL_LIB.exists():
            lib = ctypes.CDLL(str(CEIL_LIB))
            lib.ceil_stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            lib.ceil_stream_probe.restype = ctypes.c_int
            half = STREAM_CAL_BYTES // 2
            buf = torch.zeros(STREAM_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
            chunk = 256 << 10
            res = torch.empty(half // chunk * 64, dtype=torch.float32, device="cuda")
            rc = lib.ceil_stream_probe(2, 1, ctypes.c_void_p(buf.data_ptr()), half, chunk,
                                       ctypes.c_void_p(res.data_ptr()),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise SystemExit(f"bench.py: streaming calibration probe failed ({rc})")
            torch.cuda.synchronize()
            del buf, res
        torch.cuda.empty_cache()

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    inp = None
    if not args.no_headline:
        # ---- headline: the whole step, graph-replayed
        log(f"headline {HEADLINE}: building inputs")
        head, inp, fc, bc = run_workload(torch, timer, HEADLINE, w, iters=5)

        def step():
            fc.launch()
            bc.launch()  # the whole backward: prep, then dK/dV and dQ

        g = timer.capture(step)
        # the replayed graph must reproduce the eager step bit for bit
        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (fc.o, fc.lse, bc.dq, bc.dk, bc.dv)]
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (fc.o, fc.lse, bc.dq, bc.dk, bc.dv)):
            if not torch.equal(a, b):
                raise SystemExit("bench.py: graph replay differs from the eager step")

        log(f"headline: {args.warmup} warmup + {args.steps} timed steps")
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        gpu_ms_per_step = e0.elapsed_time(e1) / args.steps
        gfl = head["gflop"]
        value = (gfl["fwd"] + gfl["bwd"]) * 1e9 / (ms_per_step * 1e-3) / 1e12
        stages = ("fwd", "prep", "main") if head["fused_backward"] else ("fwd", "prep", "dkdv", "dq")
        out.update({
            "value": round(value, 3), "unit": "TFLOP/s", "ms_per_step": round(ms_per_step, 5),
            "gpu_ms_per_step": round(gpu_ms_per_step, 5),
            "config": {"workload": HEADLINE, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.Lq, "D": w.D,
                       "causal": True,
                       "step": "fwd + bwd (prep, then dK/dV and dQ"
                               + (" in one launch)" if head["fused_backward"] else ")")},
            "peak_frac": round(value / PEAK_BF16_TFLOPS, 4),
            # forward and backward apart (kernel time of each, graph-replayed launches)
            "peak_frac_fwd": round(head["peak_frac"]["fwd"], 4),
            "peak_frac_bwd": round(head["peak_frac"]["bwd"], 4),
            "roofline": roofline(HEADLINE, w, head),
            "kernels_ms": {k: head["ms"][k] for k in stages},
        })

    # ---- other workloads
    if not args.no_extra:
        names = list(EXTRA)
        if args.only:
            names = [n for n in names + [HEADLINE] if n in args.only.split(",")]
        extra = {}
        for name in names:
            log(f"workload {name}")
            res, _, fc2, bc2 = run_workload(torch, timer, name, WORKLOADS[name], iters=3)
            res["roofline"] = roofline(name, WORKLOADS[name], res)
            extra[name] = res
            del fc2, bc2
            torch.cuda.empty_cache()
        out["workloads"] = extra

    # ---- the chip's ceilings measured now (clock under MFMA load, a bf16 MFMA stream, a
    # MALL-busting HBM read), and each roofline's fraction of them beside that of the spec
    # (the default run only: the per-workload profiling runs keep their traces to the kernels)
    if not (args.no_ceilings or args.only or args.no_headline):
        log("measured ceilings: MFMA stream, HBM read, clock")
        from scaled_dot_product_sdpa_amd.ceilings import measured
        ceil = measured()
        out["measured_ceilings"] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in ceil.items()}

        def add_frac(roof):
            if not roof:
                return
            c = (ceil["hbm_read_tbs"] * 1e3 if roof["unit"] == "GB/s"
                 else ceil["mfma_bf16_tflops"] if roof["bound"] == "mfma" else None)
            roof["frac_of_measured"] = round(roof["achieved"] / c, 4) if c else None

        add_frac(out.get("roofline"))
        for res in out.get("workloads", {}).values():
            add_frac(res.get("roofline"))
        if "peak_frac_fwd" in out:
            r = PEAK_BF16_TFLOPS / ceil["mfma_bf16_tflops"]
            out["measured_frac_fwd"] = round(out["peak_frac_fwd"] * r, 4)
            out["measured_frac_bwd"] = round(out["peak_frac_bwd"] * r, 4)

    # ---- CPU baseline (rank 0, N = 1 only)
    if not args.no_cpu and inp is not None:
        log("cpu baseline: fp64 oracle on the headline step")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
