"""Build libhr.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m codebook_decode_amd.build          # writes codebook_decode_amd/libhr.so
    python -m codebook_decode_amd.build --asan   # writes codebook_decode_amd/libhr_asan.so

Objects go to codebook_decode_amd/_build/ (git-ignored); the shared library
sits next to the Python binding that loads it.

--asan: the host code (the C ABI's validation and launch sequencing) built
with AddressSanitizer and UndefinedBehaviorSanitizer; the GPU code is built as
usual (the sanitizers apply to the host pass only).  Load it through the
binding with HR_LIB=<path> and the ASan runtime preloaded (asan_runtime()
gives its path), e.g. to run tests/test_abi.py on the CPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhr.so")
LIB_ASAN = os.path.join(PKG, "libhr_asan.so")
BUILD_ASAN = os.path.join(PKG, "_build_asan")
# host-pass sanitizers (each -fsanitize= right after -Xarch_host: host code only)
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-fno-omit-frame-pointer", "-g", "-shared-libsan"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed-fp32 VALU forms stay disabled: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 dwords of every kernel's arguments preloaded into SGPRs at
    # dispatch (the code keeps the s_load fallback): a kernel starts without
    # waiting on its argument loads (36-layer stack: P = 13 2.404 -> 2.369 ms,
    # P = 512 6.45 -> 6.41 ms, same-box A/B)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources() -> list:
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    return [os.path.join(CSRC, f) for f in names]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


def _compile(src: str, asan: bool = False) -> str:
    obj = os.path.join(BUILD_ASAN if asan else BUILD, os.path.basename(src) + ".o")
    flags = FLAGS + (ASAN_FLAGS if asan else [])
    cmd = [_hipcc(), *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), *flags, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def asan_runtime() -> str:
    """Path of the ASan runtime the sanitizer build links against (to preload)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = True, asan: bool = False) -> str:
    """Compile every source and link libhr.so (or libhr_asan.so); always rebuilds."""
    os.makedirs(BUILD_ASAN if asan else BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, asan), srcs))
    lib = LIB_ASAN if asan else LIB
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if asan:
        cmd += ["-fsanitize=address,undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources", file=sys.stderr)
    return lib


if __name__ == "__main__":
    build(asan="--asan" in sys.argv[1:])
