"""Build libnbattn.so (HIP kernels + C-ABI) for gfx950, in-tree.

Usage: ``python -m sliding_window_attention_fold_amd.build`` (or ``__graft_entry__.build()``).
Each translation unit is compiled with hipcc into ``_build/`` and linked into
``sliding_window_attention_fold_amd/libnbattn.so`` (atomically replaced).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnbattn.so")
SOURCES = [
    "csrc/segment_build.hip",
    "csrc/attn_fwd.hip",
    "csrc/attn_bwd.hip",
    "csrc/exchange.hip",
    "csrc/ring.hip",
    "csrc/nbattn_host.cpp",
]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the device code on purpose.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(PKG, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build(jobs: int = 4) -> str:
    """Compile every source and link libnbattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # every kernel launch stub must resolve inside the library
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "_ZN2nb" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"link left library symbols undefined: {missing or nm.stderr}")
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(PKG, "libnbattn_asan.so")
# Host-only AddressSanitizer: the sanitizer flags follow -Xarch_host, so the
# device code is the same as in libnbattn.so and only the host side (the C-ABI
# preflight and launch code) is instrumented.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a process must preload to load libnbattn_asan.so."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime under /opt/rocm/lib/llvm")
    return hits[-1]


def build_asan() -> str:
    """libnbattn_asan.so: nbattn_host.cpp rebuilt with host-side AddressSanitizer, linked with the other
    objects of the regular build (run build() first).  A debug build for the CPU tests of the C-ABI."""
    src = os.path.join(PKG, "csrc/nbattn_host.cpp")
    obj = os.path.join(BUILD, "nbattn_host_asan.o")
    r = subprocess.run([HIPCC, *FLAGS, *ASAN_HOST, "-x", "hip", "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (asan) failed:\n{r.stderr}")
    objs = [os.path.join(BUILD, os.path.basename(x) + ".o") for x in SOURCES if not x.endswith("nbattn_host.cpp")]
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_HOST, *objs, obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (asan) failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build())
    if "--asan" in sys.argv:
        print(build_asan())
