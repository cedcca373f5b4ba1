"""GPU parity of the plain packed call's narrow path against the CPU oracle:
sequences whose query rows fit one 16-row matrix-core tile (Lq x group <= 16:
decode rows, multi-token decode) are taken per (sequence, kv head) by four
waves walking their own 32-key tiles, the other sequences by the query-tile
path in the same launch. Cases sit on both sides of the 16-row limit for
each group size, with ragged key tails, empty contexts, rows with no visible
key (Lq > Lk, causal), long rows, every block size and both head dims;
and the split call, whose chunks of narrow sequences take the same path."""

import numpy as np
import pytest

from paged_kv_cache_39_amd import workloads as wl
from tests.test_gpu_varlen import check_varlen
from tests.test_gpu_varlen_split import check_split

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (32, 8), (6, 2), (16, 2), (16, 1), (64, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_narrow_limit_per_group(dtype, hq, hkv, causal):
    """Lq = 1, the largest narrow Lq (16 // group) and one more, next to a
    prefill-sized sequence, over keys spanning several 32-key tiles."""
    group = hq // hkv
    top = max(1, 16 // group)
    ql = [1, top, top + 1, 2, 150]
    kl = [333, 97, 160, 31, 150]
    case = wl.varlen_case(1300 + hq + hkv, ql, kl, hq, hkv, 128, 16, dtype, causal=causal)
    check_varlen(case)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_narrow_block_sizes(d, bs):
    ql = [1, 4, 3, 1, 64]
    kl = [bs - 1, bs + 1, 3 * bs + 5, 1, 200]
    case = wl.varlen_case(1320 + d + bs, ql, kl, 32, 8, d, bs, "bf16", causal=True)
    check_varlen(case)


def test_narrow_empty_and_masked_rows():
    """Lk = 0 (zero output), Lq > Lk under the causal mask (the first rows see
    no key: zero), Lk = 1, and a key count that is a multiple of the tile."""
    ql = [1, 4, 3, 4, 2, 1]
    kl = [0, 2, 1, 0, 64, 128]
    case = wl.varlen_case(1340, ql, kl, 32, 8, 128, 16, "f16", causal=True)
    check_varlen(case)


def test_narrow_long_rows():
    """Rows over thousands of keys (many tiles per wave), Lq 1 and 4."""
    ql = [1, 4, 1, 2]
    kl = [5003, 4096, 2049, 777]
    case = wl.varlen_case(1350, ql, kl, 32, 8, 128, 32, "bf16", causal=True)
    check_varlen(case)


def test_narrow_many_sequences():
    """200 sequences: mostly narrow rows of varied lengths, some wide ones
    (the tile lookup's later wave-wide chunks skip the narrow ones)."""
    rng = np.random.default_rng(21)
    ql = np.where(rng.random(200) < 0.8, rng.integers(1, 5, size=200),
                  rng.integers(5, 40, size=200))
    kl = ql + rng.integers(0, 400, size=200)
    case = wl.varlen_case(1360, ql.tolist(), kl.tolist(), 32, 8, 64, 16, "bf16", causal=True)
    check_varlen(case)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (6, 2, 64), (4, 4, 128)])
def test_narrow_split_call(causal, hq, hkv, d):
    """The split call: narrow sequences over long keys are cut into chunks
    that take the narrow path and leave their triples to the merge kernel;
    short ones are not cut; a row of only masked chunks (Lq > Lk under the
    causal mask) and an empty context merge to zero."""
    group = hq // hkv
    top = max(1, 16 // group)
    ql = [1, top, 2, top, 1, 3, 40]
    kl = [4100, 2049, 1, 0, 700, 5000, 1500]
    case = wl.varlen_case(1370 + hq + d, ql, kl, hq, hkv, d, 16, "bf16", causal=causal)
    check_split(case)
