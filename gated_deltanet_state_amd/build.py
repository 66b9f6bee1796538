"""Build libgdn.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m gated_deltanet_state_amd.build [--asan]  (or build() from Python).
Every HIP translation unit is compiled with packed-fp32 instructions turned
off; the host code of the ABI is compiled by the same driver.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgdn.so")

SOURCES = ["gdn_prep.hip", "gdn_prep_bf16.hip", "gdn_chain.hip", "gdn_chain_bf16.hip", "gdn_compose.hip", "gdn_decode.hip", "gdn_front.hip", "gdn_scalar.hip", "gdn_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in ordinary VGPRs: the kernels post-process every
          # product with vector ALU code, which AGPR accumulators would force
          # through extra register moves
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-munsafe-fp-atomics"]


def _compile(src: str, bdir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on " + src)
    return obj


# Host-side AddressSanitizer build of the library (CPU checks of the C ABI's
# argument handling): the host code of every translation unit is
# instrumented, the device code is built as usual.  Load it with the ASan
# runtime preloaded (asan_runtime()).
LIB_ASAN = os.path.join(HERE, "libgdn_asan.so")
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's host compiler."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang ASan runtime under /opt/rocm/llvm")
    return hits[-1]


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile every translation unit and link libgdn.so (libgdn_asan.so with
    asan=True)."""
    out_lib = LIB_ASAN if asan else LIB
    bdir = os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR
    os.makedirs(bdir, exist_ok=True)
    extra = ASAN_HOST if asan else []
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, bdir, extra), SOURCES))
    tmp = out_lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + extra + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of %s failed" % os.path.basename(out_lib))
    os.replace(tmp, out_lib)
    if verbose:
        print("built", out_lib)
    return out_lib


if __name__ == "__main__":
    build(verbose=True, asan="--asan" in sys.argv)
