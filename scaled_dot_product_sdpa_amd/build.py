"""Build libsdpa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m scaled_dot_product_sdpa_amd.build`` (or ``build()`` from Python).
Each source is compiled to an object file in ``_build/`` in parallel, then linked.
``python -m scaled_dot_product_sdpa_amd.build --resource-usage`` instead prints, as a
markdown table, the registers, LDS and register-limited occupancy the compiler gives each
kernel (its ``kernel-resource-usage`` remarks on a device-only compile).
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libsdpa.so"
SOURCES = ["sdpa_api.cpp", "fwd_bf16.hip", "bwd_bf16.hip", "decode_bf16.hip", "attn_f32.hip"]
# microbenchmarks of the hardware ceilings (not part of libsdpa.so)
CEIL_LIB = PKG / "libceilings.so"
CEIL_SOURCE = "ceilings.hip"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs where they fit: the softmax-style arithmetic on
    # the S / dP accumulators then needs no copies out of AGPRs, and the d = 64 dK/dV kernel
    # fits in 256 registers, so two of its waves share a SIMD (measured 21-31 % faster)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


# the same without the VGPR-form MFMA flag: the compiler then keeps MFMA accumulators in
# AGPRs wherever a kernel's registers exceed 256 or it uses AGPRs anyway
AGPR_FLAGS = [f for f in FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=1")]


def _compile(src: Path, obj: Path, extra=(), flags=None) -> None:
    lang = ["-x", "hip"] if src.suffix == ".cpp" else []
    cmd = [HIPCC, *(FLAGS if flags is None else flags), *extra, *lang, "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src.name}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False, extra=()) -> Path:
    BUILD.mkdir(exist_ok=True)
    objs = []
    jobs = []
    for name in SOURCES:
        src = CSRC / name
        obj = BUILD / (name.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        jobs.append((src, obj))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _compile(j[0], j[1], extra), jobs))
    tmp = LIB.with_name(LIB.name + f".tmp{os.getpid()}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libsdpa.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    # the ceilings library: its AGPR-form probes are a second object of the same source,
    # compiled without the flag that forces VGPR-form MFMAs
    _compile(CSRC / CEIL_SOURCE, BUILD / "ceilings.o", extra)
    _compile(CSRC / CEIL_SOURCE, BUILD / "ceilings_agpr.o", ["-DCEIL_AGPR_FORM", *extra], flags=AGPR_FLAGS)
    tmp = CEIL_LIB.with_name(CEIL_LIB.name + f".tmp{os.getpid()}")
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp),
                        str(BUILD / "ceilings.o"), str(BUILD / "ceilings_agpr.o")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libceilings.so failed")
    os.replace(tmp, CEIL_LIB)
    return LIB


def resource_usage() -> str:
    """Markdown table of every kernel's VGPRs, AGPRs, SGPRs, LDS bytes per workgroup,
    waves per SIMD the registers allow, and spills, from hipcc's resource remarks."""
    rows = []
    for name in SOURCES:
        if not name.endswith(".hip"):
            continue
        cmd = [HIPCC, *FLAGS, "--offload-device-only", "-Rpass-analysis=kernel-resource-usage",
               "-c", str(CSRC / name), "-o", os.devnull]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            raise RuntimeError(f"hipcc failed on {name}")
        cur = None
        for ln in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", ln)
            if m:
                cur = {"sym": m.group(1)}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass", ln)
            if m and cur is not None:
                cur[m.group(1).strip()] = m.group(2)
    dem = subprocess.run(["c++filt"], input="\n".join(r["sym"] for r in rows), capture_output=True,
                         text=True).stdout.splitlines()
    out = ["| kernel | VGPRs | AGPRs | SGPRs | LDS bytes / workgroup | waves / SIMD (registers) | spills V/S |",
           "|---|---:|---:|---:|---:|---:|---|"]
    for r, d in zip(rows, dem):
        d = re.sub(r"\(.*\)$", "", d.replace("sdpa::(anonymous namespace)::", "").replace("sdpa::", ""))
        out.append(f"| `{d}` | {r['VGPRs']} | {r['AGPRs']} | {r['TotalSGPRs']} | "
                   f"{r['LDS Size [bytes/block]']} | {r['Occupancy [waves/SIMD]']} | "
                   f"{r['VGPRs Spill']}/{r['SGPRs Spill']} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv[1:]:
        print(resource_usage())
    else:
        build(verbose=True)
