"""Build libna_attn.so (the C-ABI attention library) for gfx950 with hipcc.

Usage: python -m causal_self_attention_mha_amd.build   (or call build())

Each .hip/.cpp under csrc/ is compiled to an object in _build/ (in parallel),
then linked into causal_self_attention_mha_amd/lib/libna_attn.so.  hipcc
cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libna_attn.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("NA_ATTN_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["api.cpp", "fwd_bf16.hip", "bwd_bf16.hip", "decode_bf16.hip", "attn_f32.hip",
           "prologue_bf16.hip"]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stderr}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link the library.  Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_DIR = os.path.join(BUILD, "asan")
SAN_LIB = os.path.join(SAN_DIR, "libna_attn_asan.so")


def build_sanitized(verbose: bool = False) -> str:
    """A host-sanitized twin of the library for the C-ABI tests: api.cpp (the
    host-side argument checks and launch code) compiled by the host compiler
    with AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular device objects of the last build().  Loading it needs the
    sanitizer runtimes preloaded (LD_PRELOAD); it runs the host checks only,
    never on a GPU."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    os.makedirs(SAN_DIR, exist_ok=True)
    obj = os.path.join(SAN_DIR, "api.o")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), *san, "-c",
           os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed\n{' '.join(cmd)}\n{r.stderr}")
    dev_objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "api.cpp"]
    missing = [o for o in dev_objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"device objects missing (run build() first): {missing}")
    cmd = [gxx, "-shared", *san, obj, *dev_objs, "-L", "/opt/rocm/lib",
           "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
