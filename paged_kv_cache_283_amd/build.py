"""Compile the gfx950 HIP library libpagedkv.so in-tree (hipcc, no JIT cache).

    python -m paged_kv_cache_283_amd.build [--jobs N]

Every HIP translation unit is built for gfx950 only, with packed-fp32 VALU
instructions disabled, then linked with the C-ABI layer (csrc/api.cpp) into
paged_kv_cache_283_amd/libpagedkv.so.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"

HIP_SOURCES = ["decode_attn.hip", "prefill_attn.hip", "kv_write.hip", "kv_compact.hip", "kv_swap.hip", "keep_select.hip",
               "probe.hip"]
HOST_SOURCES = ["api.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpagedkv.so)")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    # HIP sources: MFMA accumulators stay in VGPRs (no AGPR copies around the
    # VALU work on them).
    lang = ["-x", "hip", "-mllvm", "-amdgpu-mfma-vgpr-form"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link; `defines` (e.g. ["PKV_ATTN_NT_LOADS=1"]) and `out` serve tuning builds."""
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    srcs = HIP_SOURCES + HOST_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
