"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no GPU): argument validation,
workspace and grid sizing in the C entry points, and the block manager
(free-block scans, reference counts, copy-on-write bookkeeping, pending
copies). The ATB PagedAttention page names reference-count leaks and
copy-on-write races among the pitfalls of a paged cache, and these are the
host-memory bugs the sanitizers catch.

The instrumented build (build.py --sanitize) is loaded in a child process
with clang's ASan runtime preloaded, and runs the ABI validation tests and
the block manager's random-script parity against the oracle there."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_block_manager_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from paged_kv_cache_39_amd import build as b
    try:
        b.hipcc()
        b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build(sanitize=True)
    assert os.path.exists(lib)
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi.py"),
         os.path.join(ROOT, "tests", "test_block_manager_lib.py")],
        cwd=ROOT, env=b.sanitizer_env(), capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
