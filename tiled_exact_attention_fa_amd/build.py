"""Builds libfa.so in-tree with hipcc for gfx950.

    python -m tiled_exact_attention_fa_amd.build [--jobs N] [--verbose]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (see HIPFLAGS); the host-only validator is compiled with
the same driver.  Objects go to _build/ next to this file; the shared library
lands at tiled_exact_attention_fa_amd/libfa.so.  The compiler's per-kernel
resource report (registers, scratch, occupancy) is kept in
_build/kernel_resources.json.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
RESOURCES = os.path.join(BUILD, "kernel_resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["fa_fwd_mfma.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_kv_append.hip", "fa_bwd.hip", "fa_fp8_quant.hip"]
CPP_SOURCES = ["fa_check.cpp", "fa_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
HIPFLAGS = COMMON + [
    "--offload-arch=gfx950",
    "-munsafe-fp-atomics",
    # the kernels never rely on NaN propagation (masked scores are -inf, which
    # stays honoured); without this, every fmaxf gets a canonicalising max
    "-fno-honor-nans",
    # packed fp32 VALU forms are avoided on this hardware: keep the compiler
    # from selecting them for ordinary float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # per-kernel resource usage as compiler remarks (parsed into RESOURCES)
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes",
         "Occupancy [waves/SIMD]": "waves_per_simd", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
         "LDS Size [bytes/block]": "static_lds_bytes"}


def _resources(stderr: str) -> dict:
    """Per-kernel figures from the kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val)
    return out


def _compile(src: str, verbose: bool) -> tuple:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC] + HIPFLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + COMMON + ["-x", "c++", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln and ln.strip()]
    if noise and verbose:
        print("\n".join(noise), file=sys.stderr)
    return obj, (_resources(r.stderr) if src.endswith(".hip") else {})


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CPP_SOURCES
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in done]
    kernels = {}
    for _, res in done:
        kernels.update(res)
    with open(RESOURCES, "w") as f:
        json.dump(kernels, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
