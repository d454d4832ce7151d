"""Compiles libmoefp8.so for gfx950 in-tree with hipcc (no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoefp8.so")
SOURCES = ["quant.hip", "route.hip", "permute.hip", "gemm.hip", "backward.hip", "validate.hip", "api.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off",                     # no silent a*b+c fusion: rounding is written out explicitly
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",    # MFMA results in VGPRs: the fp32 scale promotion reads them directly
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build (CPU checks of the C ABI's host
# code; the device code is built as usual): each -fsanitize goes to the host compilation only.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
ASAN_LIB = os.path.join(BUILD, "host_sanitize", "libmoefp8.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc (to preload into a non-instrumented python)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str, out_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    out_dir = os.path.dirname(ASAN_LIB) if host_sanitize else BUILD
    lib = ASAN_LIB if host_sanitize else LIB
    extra = tuple(SANITIZE) if host_sanitize else ()
    os.makedirs(out_dir, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, host_sanitize="--host-sanitize" in sys.argv)
