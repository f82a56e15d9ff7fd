"""Build librssm.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python -m linear_attention_decode_replayssm_amd.build [-v] [--isa] [--define NAME]...

Each translation unit is compiled to an object in ``_build/`` (in parallel),
then linked into ``librssm.so`` next to this file.  ``--isa`` additionally
keeps the device assembly of every kernel under ``_build/isa/``; ``--define
NAME`` passes -DNAME to every translation unit (RSSM_M2_VERIFY_MFMA selects
the matrix-core variant of the Mamba-2 verify contraction, RSSM_XCD_WHOLE the
whole-sequence XCD order for every kernel; both kept for measurement).

Packed fp32 instructions are disabled for all device code
(``-target-feature -packed-fp32-ops``): the compiler would otherwise form
them from ordinary float code.  The atomic optimizer is off
(``-amdgpu-atomic-optimizer-strategy=None``): every atomic here is issued by
one lane, and the optimizer's lane scan reads the returned value right away,
which makes the issuing wave wait for all of its earlier loads -- the whole
state stream -- before it reaches the workgroup's first barrier.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librssm.so")

SOURCES = ["api.cpp", "m2_kernels.hip", "gdn_kernels.hip", "index_kernels.hip", "prefill_kernels.hip",
           "eager_spec_kernels.hip", "probe_kernels.hip"]
ARCH = "gfx950"


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-Wall", "-Wno-unused-function", "-I", INC, "-I", CSRC]


DEFINES = []


def _compile(src, verbose, isa):
    out_dir = BUILD
    extra = []
    if isa and src.endswith(".hip"):
        out_dir = os.path.join(BUILD, "isa")
        os.makedirs(out_dir, exist_ok=True)
        extra = ["-save-temps=obj"]
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    defs = [f"-D{d}" for d in DEFINES]
    cmd = [_hipcc()] + _flags() + defs + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, flush=True)
    return obj


def build(verbose: bool = False, isa: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, isa), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    args = sys.argv[1:]
    for i, a in enumerate(args):
        if a == "--define" and i + 1 < len(args):
            DEFINES.append(args[i + 1])
    print(build(verbose="-v" in args, isa="--isa" in args))
