"""Build the gfx950 attention library (libfmha.so) in-tree with hipcc.

Usage: python -m fmha_fwd_amd.build [--verbose]
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libfmha.so")
SOURCES = ["api.cpp", "quantize.hip", "nvfp4.hip", "attention.hip"]
# The attention kernel never sees NaN scores (masked keys are -inf, inputs are
# finite), so its max reductions need no NaN quieting.  Host validation code
# keeps full IEEE semantics (it rejects NaN arguments).
EXTRA = {"attention.hip": ["-fno-honor-nans"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay disabled (ordinary float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, verbose, tag="libfmha", defines=()):
    obj = os.path.join(LIBDIR, f"{tag}_{os.path.splitext(src)[0]}.o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + [f"-D{d}" for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def build(verbose=False, out=None, defines=()):
    """Compile every source for gfx950 and link libfmha.so (or `out`, with
    extra -D `defines` for tuning variants); returns the library path."""
    os.makedirs(LIBDIR, exist_ok=True)
    lib = out or LIB
    tag = os.path.basename(lib).replace(".so", "")
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, tag, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    for o in objs:
        os.remove(o)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
