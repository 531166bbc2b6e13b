"""Ceilings of the gfx950 resources the attention kernels use, measured on the GPU.

``python -m scaled_dot_product_sdpa_amd.ceilings`` runs the probes of ``csrc/ceilings.hip``
(libceilings.so, built with the library) and prints one markdown table: the bf16 MFMA
rate, LDS read rates in the two operand patterns of the kernels, the forward's matrix
skeleton (S and PV products with their LDS operand reads, no softmax) at 32 and 64 query
rows per wave, with the MFMA accumulators in VGPRs or AGPRs, and MFMA next to independent
vector arithmetic.  Each probe fills every SIMD with 1 or 2 waves and is timed with HIP
events around five back-to-back launches (after a warm-up launch); the shader clock under
MFMA load is read with s_memtime against the 100 MHz constant-rate counter.
"""

from __future__ import annotations

import ctypes
import sys

from .build import CEIL_LIB

PEAK_BF16_TFLOPS = 2500.0
CUS = 256
REPS = 5

# id: (name, MFMAs per wave per iteration, LDS bytes per wave per iteration)
PROBES = {
    0: ("MFMA 32x32x16 bf16, one accumulation chain", 1, 0),
    1: ("MFMA 32x32x16 bf16, four independent chains", 4, 0),
    2: ("LDS 16-byte row reads (K operand pattern)", 0, 16 * 1024),
    3: ("LDS ds_read_b64_tr_b16 pairs (V^T operand pattern)", 0, 16 * 1024),
    6: ("forward skeleton, 32 rows per wave, operands in registers", 32, 0),
    7: ("forward skeleton, 64 rows per wave, operands in registers", 64, 0),
    4: ("forward skeleton, 32 rows per wave, LDS operands, VGPR accumulators", 32, 32 * 1024),
    15: ("forward skeleton, 32 rows per wave, LDS operands, AGPR accumulators", 32, 32 * 1024),
    5: ("forward skeleton, 64 rows per wave, LDS operands, VGPR accumulators", 64, 32 * 1024),
    16: ("forward skeleton, 64 rows per wave, LDS operands, AGPR accumulators", 64, 32 * 1024),
    8: ("MFMA + 4 v_fma_f32 per MFMA", 8, 0),
    9: ("MFMA + 6 v_fma_f32 per MFMA", 8, 0),
    10: ("MFMA + 8 v_fma_f32 per MFMA", 8, 0),
    11: ("MFMA + 2 (v_exp_f32, v_sub_f32) per MFMA", 8, 0),
    12: ("MFMA + 4 (v_exp_f32, v_sub_f32) per MFMA", 8, 0),
    13: ("MFMA + 4 v_fma_f32 + (v_exp_f32, v_sub_f32) per MFMA", 8, 0),
    14: ("MFMA + 5 v_fma_f32 + (v_exp_f32, v_sub_f32) per MFMA", 8, 0),
    18: ("probe 13's work per 16 MFMAs in their second half only: 8 + 0, then 8 x (8 v_fma_f32 + 2 (v_exp_f32, v_sub_f32))", 16, 0),
    19: ("the same as a forward phase spreads it: 8 x 1 v_fma_f32, then 8 x (7 v_fma_f32 + 2 (v_exp_f32, v_sub_f32))", 16, 0),
}
SKELETON = {4, 5, 6, 7, 15, 16}
# probes whose registers do not fit two waves per SIMD
ONE_WAVE_ONLY = {16}
# iterations per launch, per probe kind (a few hundred microseconds each)
ITERS = {"mfma": 4000, "lds": 4000, "skeleton": 1000, "mix": 2000}


def _iters(pid, scale):
    kind = "mfma" if pid in (0, 1) else "lds" if pid in (2, 3) else "skeleton" if pid in SKELETON else "mix"
    return max(1, int(ITERS[kind] * scale))


def run(scale: float = 1.0, ids=None) -> str:
    """The MFMA / LDS / mix table (only the probes in `ids` if given, then without the
    atomics and streaming tables)."""
    import torch
    lib = ctypes.CDLL(str(CEIL_LIB))
    lib.ceil_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_probe.restype = ctypes.c_int
    out = torch.empty(65536 * 2, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(pid, wps, it):
        rc = lib.ceil_probe(pid, wps, ctypes.c_void_p(out.data_ptr()), it, stream)
        if rc != 0:
            raise RuntimeError(f"probe {pid}: status {rc}")

    # shader clock under MFMA load
    it = _iters(0, scale)
    launch(17, 2, it)
    torch.cuda.synchronize()
    cyc, ticks = out[0].item(), out[1].item()
    ghz = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else float("nan")
    rows = [f"Shader clock under MFMA load (s_memtime over s_memrealtime at 100 MHz): {ghz:.2f} GHz; "
            f"the MFMA peak at that clock is {PEAK_BF16_TFLOPS * ghz / 2.4:.0f} TFLOP/s.", "",
            "| probe | waves / SIMD | us per launch | MFMA TFLOP/s | % of bf16 peak | LDS TB/s | LDS B/clk/CU |",
            "|---|---:|---:|---:|---:|---:|---:|"]
    for pid, (name, mf, lds_bytes) in PROBES.items():
        if ids is not None and pid not in ids:
            continue
        for wps in (1, 2):
            if wps == 2 and pid in ONE_WAVE_ONLY:
                continue
            it = _iters(pid, scale)
            launch(pid, wps, it)  # warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(REPS):
                launch(pid, wps, it)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / REPS
            waves = CUS * 4 * wps
            # MFMAs per wave per iteration: the chains (0, 1); 2 blocks x 2 products x 8 per
            # 32-row group (skeleton); 8 (mixes)
            mfmas = (mf // 32) * 2 * 2 * 8 if pid in SKELETON else mf
            tf = waves * it * mfmas * 32768 / (us * 1e-6) / 1e12 if mfmas else None
            lds = waves * it * lds_bytes / (us * 1e-6) / 1e12 if lds_bytes else None
            per_clk = lds * 1e12 / CUS / (ghz * 1e9) if lds else None
            rows.append(f"| {name} | {wps} | {us:.1f} | " + ("–" if tf is None else f"{tf:.0f}") + " | " +
                        ("–" if tf is None else f"{100 * tf / PEAK_BF16_TFLOPS:.1f}") + " | " +
                        ("–" if lds is None else f"{lds:.1f}") + " | " +
                        ("–" if per_clk is None else f"{per_clk:.0f}") + " |")
    if ids is None:
        rows += ["", atomics(scale), "", streaming()]
    return "\n".join(rows)


def streaming() -> str:
    """HBM read rate in the decode kernel's access pattern (csrc/ceilings.hip, probe 7):
    one-wave workgroups each streaming a contiguous chunk of one or two 512 MiB streams (K,
    V) in 8 KB tiles, two tiles per stream in flight, with and without the non-temporal
    cache policy; chunk sizes of a 768-key decode split (192 KiB per stream) and of long
    streams (2 MiB)."""
    import torch
    lib = ctypes.CDLL(str(CEIL_LIB))
    lib.ceil_stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ceil_stream_probe.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sb = 512 << 20
    buf = torch.ones(2 * sb // 4, dtype=torch.float32, device="cuda")
    rows = ["| HBM streaming read | streams | chunk per stream | cache policy | us per launch | TB/s | % of 8 TB/s |",
            "|---|---:|---:|---|---:|---:|---:|"]
    for nstr in (1, 2):
        for chunk in (192 << 10, 2 << 20):
            n = sb // chunk * chunk  # whole chunks per stream
            out = torch.empty(n // chunk * 64, dtype=torch.float32, device="cuda")
            for nt in (1, 0):
                def launch():
                    rc = lib.ceil_stream_probe(nstr, nt, ctypes.c_void_p(buf.data_ptr()), n, chunk,
                                               ctypes.c_void_p(out.data_ptr()), stream)
                    if rc != 0:
                        raise RuntimeError(f"stream probe: status {rc}")

                launch()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(REPS):
                    launch()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / REPS
                tbs = nstr * n / (us * 1e-6) / 1e12
                rows.append(f"| one wave per chunk, 2 x 8 KB tiles in flight per stream | {nstr} | "
                            f"{chunk >> 10} KiB | {'non-temporal' if nt else 'default'} | {us:.1f} | "
                            f"{tbs:.2f} | {100 * tbs / 8.0:.1f} |")
    # at the decode kernel's two workgroups per SIMD: two, then three tiles per stream in
    # flight (non-temporal)
    chunk = 192 << 10
    n = sb // chunk * chunk
    out = torch.empty(n // chunk * 64, dtype=torch.float32, device="cuda")
    for code, tif in ((4, 2), (3, 3)):
        def launch():
            rc = lib.ceil_stream_probe(2, code, ctypes.c_void_p(buf.data_ptr()), n, chunk,
                                       ctypes.c_void_p(out.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"stream probe: status {rc}")

        launch()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPS):
            launch()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / REPS
        tbs = 2 * n / (us * 1e-6) / 1e12
        rows.append(f"| one wave per chunk, {tif} x 8 KB tiles in flight per stream, two workgroups per SIMD "
                    f"| 2 | {chunk >> 10} KiB | non-temporal | {us:.1f} | {tbs:.2f} | {100 * tbs / 8.0:.1f} |")
    del buf
    return "\n".join(rows)


def atomics(scale: float = 1.0) -> str:
    """fp32 accumulation into global memory (csrc/ceilings.hip, probe 6): atomic adds
    without return against plain stores of the same addresses, over a buffer that fits the
    L2 of one XCD (4 MiB) and one that does not (128 MiB)."""
    import torch
    lib = ctypes.CDLL(str(CEIL_LIB))
    lib.ceil_atomic_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.ceil_atomic_probe.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows = ["| fp32 accumulation | buffer | workgroups | us per launch | G updates/s | GB/s |",
            "|---|---:|---:|---:|---:|---:|"]
    for n in (1 << 20, 1 << 25):
        buf = torch.zeros(n, dtype=torch.float32, device="cuda")
        for mode, what in ((0, "atomic add (no return)"), (1, "plain store")):
            for blocks in (512, 2048):
                it = max(1, int(200 * scale))

                def launch():
                    rc = lib.ceil_atomic_probe(mode, ctypes.c_void_p(buf.data_ptr()), n, it, blocks, stream)
                    if rc != 0:
                        raise RuntimeError(f"atomic probe: status {rc}")

                launch()  # warm-up
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(REPS):
                    launch()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / REPS
                ups = blocks * 256 * it / (us * 1e-6)
                rows.append(f"| {what} | {n * 4 >> 20} MiB | {blocks} | {us:.1f} | {ups / 1e9:.0f} | {ups * 4 / 1e9:.0f} |")
        del buf
    return "\n".join(rows)


def measured() -> dict:
    """The ceilings a bench line is read against, measured now: the shader clock under MFMA
    load, the bf16 MFMA rate of a 32x32x16 stream (four independent accumulation chains, two
    waves per SIMD; probe 1) and the HBM read rate of two 512 MiB streams in the decode
    kernel's pattern with the non-temporal policy (probe 7; 1 GiB per launch, four times the
    256 MB last-level cache).  About a second of GPU time."""
    import torch
    lib = ctypes.CDLL(str(CEIL_LIB))
    lib.ceil_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.ceil_probe.restype = ctypes.c_int
    lib.ceil_stream_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ceil_stream_probe.restype = ctypes.c_int
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = torch.empty(65536 * 2, dtype=torch.float32, device="cuda")

    def timed(fn):
        fn()  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(REPS):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / REPS  # us

    def probe(pid, wps, it):
        rc = lib.ceil_probe(pid, wps, ctypes.c_void_p(out.data_ptr()), it, stream)
        if rc != 0:
            raise RuntimeError(f"probe {pid}: status {rc}")

    it = _iters(1, 1.0)
    probe(17, 2, it)
    torch.cuda.synchronize()
    cyc, ticks = out[0].item(), out[1].item()
    ghz = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else float("nan")
    us = timed(lambda: probe(1, 2, it))
    mfma_tf = CUS * 4 * 2 * it * 4 * 32768 / (us * 1e-6) / 1e12
    sb = 512 << 20
    chunk = 192 << 10
    n = sb // chunk * chunk
    buf = torch.ones(2 * sb // 4, dtype=torch.float32, device="cuda")
    sout = torch.empty(n // chunk * 64, dtype=torch.float32, device="cuda")

    def stream_read():
        rc = lib.ceil_stream_probe(2, 1, ctypes.c_void_p(buf.data_ptr()), n, chunk,
                                   ctypes.c_void_p(sout.data_ptr()), stream)
        if rc != 0:
            raise RuntimeError(f"stream probe: status {rc}")

    us = timed(stream_read)
    del buf, sout
    return {"clock_ghz": ghz, "mfma_bf16_tflops": mfma_tf, "hbm_read_tbs": 2 * n / (us * 1e-6) / 1e12,
            "mfma_probe": "v_mfma_f32_32x32x16_bf16, four independent chains, two waves per SIMD",
            "hbm_probe": "two 512 MiB streams, one-wave workgroups, 192 KiB chunks, non-temporal loads"}


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "atomics":
        print(atomics(float(sys.argv[2]) if len(sys.argv) > 2 else 1.0))
    elif len(sys.argv) > 1 and sys.argv[1] == "streaming":
        print(streaming())
    elif len(sys.argv) > 1 and sys.argv[1] == "mix":
        print(run(1.0, ids={8, 9, 10, 11, 12, 13, 14, 18, 19}))
    else:
        print(run(float(sys.argv[1]) if len(sys.argv) > 1 else 1.0))
