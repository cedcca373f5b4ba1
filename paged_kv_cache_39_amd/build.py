"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_39_amd.build              # build (always recompiles)
    python -m paged_kv_cache_39_amd.build --sanitize   # host-side ASan + UBSan build
    python -m paged_kv_cache_39_amd.build --debug      # device contract reports
    python -m paged_kv_cache_39_amd.build --all        # regular + debug, in parallel

The sanitizer build (libpagedkv_sanitize.so) instruments the host code only
(argument validation, workspace layout, the block manager); its device code
is the regular build's. It is for CPU test runs: load it through the
PAGEDKV_LIBRARY environment variable with clang's ASan runtime preloaded
(see sanitizer_env()).

The debug build (libpagedkv_debug.so) compiles the kernels with
PKV_DEBUG_CHECKS=1: where a kernel clamps a block id, length, cu_seqlens
entry, slot or copy pair that breaks the caller's contract, it also records
the kind in a device word (pkv_debug_take_errors reads it). Same arguments
and results as the regular build; slower only where it reports.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedkv.so")
SANITIZE_LIB = os.path.join(PKG, "libpagedkv_sanitize.so")
DEBUG_LIB = os.path.join(PKG, "libpagedkv_debug.so")
SOURCES = ["api.hip", "kv_write.hip", "decode.hip", "varlen.hip", "block_manager.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # keep the compiler from forming packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
    ]


# host-only instrumentation: every sanitizer flag goes to the host pass
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                  "-fno-omit-frame-pointer", "-shared-libasan", "-g"]


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime that the sanitizer build links."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found")
    return path


def sanitizer_env() -> dict:
    """Environment for a Python process that loads the sanitizer build."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["PAGEDKV_LIBRARY"] = SANITIZE_LIB
    # the interpreter itself is not instrumented: its own allocations are
    # not leak-checked; UBSan findings abort with a report
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _command(lib: str, sanitize: bool, debug: bool) -> list[str]:
    return [hipcc(), *compile_flags(), *(SANITIZE_FLAGS if sanitize else []),
            *(["-DPKV_DEBUG_CHECKS=1"] if debug else []), "-shared", "-o", lib + ".tmp",
            *[os.path.join(CSRC, s) for s in SOURCES]]


def _finish(lib: str, res_code: int, out: str, verbose: bool) -> str:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in out.splitlines() if noise not in ln]
    if res_code != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(lib)}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(lib + ".tmp", lib)
    return lib


def build(verbose: bool = False, sanitize: bool = False, debug: bool = False) -> str:
    """Compile every source into libpagedkv.so, or with `sanitize` into the
    host-instrumented libpagedkv_sanitize.so, or with `debug` into
    libpagedkv_debug.so (always recompiles)."""
    lib = SANITIZE_LIB if sanitize else DEBUG_LIB if debug else LIB
    cmd = _command(lib, sanitize, debug)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return _finish(lib, res.returncode, res.stdout + res.stderr, verbose)


def build_all(verbose: bool = False) -> list[str]:
    """The regular and the debug build, compiled side by side."""
    jobs = []
    for lib, debug in ((LIB, False), (DEBUG_LIB, True)):
        cmd = _command(lib, False, debug)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                           stderr=subprocess.STDOUT, text=True)))
    done = []
    for lib, proc in jobs:
        out, _ = proc.communicate()
        done.append((lib, proc.returncode, out))
    return [_finish(lib, code, out, verbose) for lib, code, out in done]


if __name__ == "__main__":
    quiet = "-q" in sys.argv
    if "--all" in sys.argv:
        print("\n".join(build_all(verbose=not quiet)))
    else:
        print(build(verbose=not quiet, sanitize="--sanitize" in sys.argv,
                    debug="--debug" in sys.argv))
