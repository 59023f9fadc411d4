"""Build libdgfp8.so in-tree with hipcc for gfx950.

    python moe_fp8_gemm_amd/build.py [-v]

(run it as a script: importing the package loads the library being built)

Every HIP source is compiled with packed-fp32 code generation disabled and the
default (correctly rounded) fp32 division; no fast-math flags.

Every kernel's resources (VGPRs, AGPRs, SGPRs, scratch, spills, LDS,
occupancy) are taken from the compiler's kernel-resource-usage remarks and
written to _build/resource_usage.txt; the build fails when any kernel uses
scratch memory or spills VGPRs (a spill in the K loop costs more than the
loop's own memory traffic).  SGPR spills, which go to VGPR lanes, are only
reported.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libdgfp8.so")
SOURCES = ["api.cpp", "gemm_fp8.hip", "cast_fp8.hip", "scratch.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


# Per-source extra flags.  With fp32 scales the GEMM multiplies its MFMA
# accumulators on the VALU between K blocks (the scale mantissa), so the
# accumulators must live in VGPRs: force the VGPR-destination MFMA form (LLVM
# otherwise picks the AGPR form for kernels allowed more than 256 VGPRs, and each
# rescale then needs v_accvgpr_read/write moves).
EXTRA_FLAGS = {"gemm_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


RESOURCE_REPORT = os.path.join(BUILD_DIR, "resource_usage.txt")
_REMARK = "-Rpass-analysis=kernel-resource-usage"
_FIELDS = [("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("TotalSGPRs", "sgpr"), ("ScratchSize", "scratch"),
           ("VGPRs Spill", "vspill"), ("SGPRs Spill", "sspill"), ("LDS Size", "lds"), ("Occupancy", "occ")]


def parse_resource_remarks(text: str):
    """[{name, vgpr, agpr, sgpr, scratch, vspill, sspill, lds, occ}] from the
    compiler's kernel-resource-usage remarks (one block per kernel)."""
    kernels, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\w+) \[" + re.escape(_REMARK), line)
        if m and cur is not None:
            for key, short in _FIELDS:
                if m.group(1).strip() == key:
                    cur[short] = int(m.group(2)) if m.group(2).isdigit() else m.group(2)
    return kernels


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        out = r.stdout.splitlines()
        if len(out) == len(names):
            return [o.replace("dgfp8::(anonymous namespace)::", "").replace("dgfp8::", "") for o in out]
    except (OSError, subprocess.CalledProcessError):
        pass
    return names


def resource_table(kernels) -> str:
    names = _demangle([k["name"] for k in kernels])
    lines = ["%-6s %-6s %-6s %-8s %-7s %-7s %-8s %-4s %s" % ("VGPR", "AGPR", "SGPR", "scratch", "vspill", "sspill",
                                                             "LDS", "occ", "kernel")]
    for k, n in zip(kernels, names):
        lines.append("%-6s %-6s %-6s %-8s %-7s %-7s %-8s %-4s %s" % (
            k.get("vgpr"), k.get("agpr"), k.get("sgpr"), k.get("scratch"), k.get("vspill"), k.get("sspill"),
            k.get("lds"), k.get("occ"), n))
    return "\n".join(lines)


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    remarks = [_REMARK] if src.endswith(".hip") else []
    cmd = ([hipcc()] + _flags() + EXTRA_FLAGS.get(src, []) + remarks +
           ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = (r.stderr or "").splitlines()
    err = "\n".join(l for l in lines if noise not in l and "remark" not in l and _REMARK not in l
                    and not l.strip().startswith(("|", "^")) and not re.match(r"\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if verbose and err.strip():
        print(err)
    return obj, parse_resource_remarks(r.stderr or "")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in results]
    kernels = [k for _, ks in results for k in ks]
    table = resource_table(kernels)
    with open(RESOURCE_REPORT, "w") as f:
        f.write(table + "\n")
    if verbose:
        print(table)
    # SGPR spills go to lanes of VGPRs, not to memory: reported, not fatal.
    bad = [k for k in kernels if k.get("scratch", 0) or k.get("vspill", 0)]
    if bad:
        raise RuntimeError("kernels use scratch memory or spill VGPRs:\n" +
                           resource_table(bad) + f"\n(full table: {RESOURCE_REPORT})")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
