"""Build liblce.so (HIP kernels + C ABI) for gfx950 with hipcc.

Run ``python -m vocabulary_cross_entropy_row_amd.build`` (or call ``build()``).
Objects compile in parallel; the shared library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblce.so")

ARCH = "gfx950"
# (source, extra flags, object name).  ce_rows_inst.hip is compiled once per
# (dtype, rounds in VGPRs, rounds in LDS) family of the resident row kernel.
FAMILIES = [(1, 0), (2, 0), (4, 0), (8, 0), (4, 8), (8, 8), (10, 9), (13, 9), (16, 9)]
# The families also built for rows that need not start on a 16-byte boundary.
UA_FAMILIES = [(1, 0), (2, 0), (4, 0), (8, 0), (4, 8), (8, 8)]
# Short-row kernel families (waves per row, 16-byte vectors per lane), ce_rows_mr.hip.
MR_FAMILIES = [(1, 1), (1, 2), (1, 4), (1, 8), (2, 8), (4, 8), (4, 16)]
# Half-row kernel families (rounds of 960 vectors per half row), ce_rows_half.hip.
HALF_FAMILIES = [5, 6, 7, 8, 9, 10]
UNITS = [("ce_kernels.hip", [], "ce_kernels"), ("flce.hip", [], "flce"), ("ce_split.hip", [], "ce_split"), ("lce_api.cpp", ["-x", "hip"], "lce_api")] + [
    ("ce_rows_inst.hip", [f"-DLCE_BF16={b}", f"-DLCE_KR={kr}", f"-DLCE_KL={kl}", "-DLCE_UA=0"], f"ce_rows_{b}_{kr}_{kl}")
    for b in (1, 0) for kr, kl in FAMILIES] + [
    ("ce_rows_inst.hip", [f"-DLCE_BF16={b}", f"-DLCE_KR={kr}", f"-DLCE_KL={kl}", "-DLCE_UA=1"], f"ce_rows_ua_{b}_{kr}_{kl}")
    for b in (1, 0) for kr, kl in UA_FAMILIES] + [
    ("ce_rows_mr.hip", [f"-DLCE_BF16={b}", f"-DLCE_P={p}", f"-DLCE_KV={kv}"], f"ce_rows_mr_{b}_{p}_{kv}")
    for b in (1, 0) for p, kv in MR_FAMILIES] + [
    ("ce_rows_half.hip", [f"-DLCE_BF16={b}", f"-DLCE_KH={kh}"], f"ce_rows_half_{b}_{kh}")
    for b in (1, 0) for kh in HALF_FAMILIES]

# Packed-fp32 VALU ops are switched off for every device pass: hipcc -O3 would
# otherwise form v_pk_fma/add/mul_f32 on its own.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}",
          f"-I{CSRC}"]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblce.so)")


def _compile(unit, verbose: bool) -> str:
    src, flags, name = unit
    out = os.path.join(OBJ, name + ".o")
    cmd = [_hipcc(), *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = max(1, min(len(UNITS), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
