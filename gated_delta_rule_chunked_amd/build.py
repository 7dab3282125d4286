"""Build libkda.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m gated_delta_rule_chunked_amd.build

Each source is compiled to an object under _build/ in parallel, then linked
into gated_delta_rule_chunked_amd/libkda.so with an rpath to the ROCm
runtime.  Always recompiles (cheap; a few seconds per file).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "kda")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_intra.hip", "kda_inter.hip", "kda_decode.hip",
           "kda_epilogue.hip", "kda_backward.hip", "kda_check.hip", "kda_noalloc.hip"]
ARCH = "gfx950"


def _rocm():
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _hipcc():
    p = shutil.which("hipcc") or os.path.join(_rocm(), "bin", "hipcc")
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the KDA library needs ROCm's hipcc")
    return p


# Packed-fp32 instructions stay off: the compiler otherwise forms
# v_pk_{add,mul,fma}_f32 from ordinary float code.
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Wall", "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + HIP_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + [
        f"-Wl,-rpath,{_rocm()}/lib", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
