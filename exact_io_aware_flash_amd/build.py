"""Builds ``libfa.so`` (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: ``python -m exact_io_aware_flash_amd.build`` or ``build()`` from Python.
Every call recompiles all sources (the object files are kept next to the sources
in ``_build/`` only for the duration of the link).
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]

SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd32.hip", "fa_fp8.hip"]


def _compile(src: str, obj: str, extra=()) -> str:
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{out}")
    return out


# Host-side sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) for the argument
# validation and launch code; device code is compiled as usual. Load the result with
# FA_LIBRARY=<path> and the clang ASan runtime preloaded (see sanitizer_runtime()).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a sanitized build needs preloaded."""
    import glob
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return found[-1]


# The race-check library: every ring step of the kernels also waits for all of its loads
# and passes a full workgroup barrier (FA_SYNC_CHECK in fa_device.h); a GPU test compares
# its results with the normal library's bit for bit.
SYNC_CHECK_LIB = os.path.join(PKG, "libfa_synccheck.so")


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB,
          sync_check: bool = False) -> str:
    """Compile every HIP source for gfx950 and link ``libfa.so`` (or ``out``); returns its
    path. ``sanitize``: host code built with AddressSanitizer and UBSan (SANITIZE).
    ``sync_check``: the race-check variant (FA_SYNC_CHECK=1)."""
    extra = list(SANITIZE if sanitize else [])
    if sync_check:
        extra.append("-DFA_SYNC_CHECK=1")
    bdir = os.path.join(PKG, "_build_san" if sanitize else "_build_sync" if sync_check
                        else "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        futs = [ex.submit(_compile, s, o, extra) for s, o in zip(SOURCES, objs)]
        for s, f in zip(SOURCES, futs):
            msg = f.result()
            if verbose and msg.strip():
                print(f"[{s}]\n{msg}", file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    shutil.rmtree(bdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
