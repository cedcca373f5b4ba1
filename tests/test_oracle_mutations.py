"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that at least one pin catches each. This shows the pins would notice a
dropped term, a wrong index or sign, or a misread of the masking rules."""

import numpy as np
import pytest

import oracle.paged_attention as pa
import tests.test_oracle_pins as pins


def _gather_off_by_one(cache, row, n, bs):
    nb, _, hkv, d = cache.shape
    flat = cache.reshape(nb * bs, hkv, d)
    idx = [int(row[j // bs]) * bs + (j + 1) % bs for j in range(n)]
    return flat[np.array(idx, dtype=np.int64)]


def _gather_wrong_block(cache, row, n, bs):
    nb, _, hkv, d = cache.shape
    flat = cache.reshape(nb * bs, hkv, d)
    idx = [int(row[min(j // bs + 0, len(row) - 1)]) * bs + j % bs if j % bs else
           int(row[max(j // bs - 1, 0)]) * bs for j in range(n)]
    return flat[np.array(idx, dtype=np.int64)]


def _softmax_no_scale(q_vec, keys, values, scale):
    return _real_softmax(q_vec, keys, values, 1.0)


def _softmax_unnormalised(q_vec, keys, values, scale):
    n = keys.shape[0]
    if n == 0:
        return np.zeros(q_vec.shape[0]), np.zeros(0)
    s = scale * (keys @ q_vec)
    p = np.exp(s - s.max())
    return p @ values, p


def _softmax_transposed(q_vec, keys, values, scale):
    # values used where keys belong
    return _real_softmax(q_vec, values, keys, scale)


def _causal_top_left(i, lq, lk):
    return max(0, min(lk, i + 1))


def _causal_off_by_one(i, lq, lk):
    return max(0, min(lk, i + lk - lq))


def _merge_no_rescale(parts):
    live = [p for p in parts if not np.isneginf(p[0])]
    return sum(p[2] for p in live) / sum(p[1] for p in live)


_real_softmax = pa.softmax_attention

MUTATIONS = [
    ("gather_kv", _gather_off_by_one, [pins.test_decode_brute_force]),
    ("gather_kv", _gather_wrong_block, [pins.test_decode_brute_force]),
    ("softmax_attention", _softmax_no_scale, [pins.test_decode_brute_force]),
    ("softmax_attention", _softmax_unnormalised, [pins.test_softmax_weights_sum_to_one_and_are_positive]),
    ("softmax_attention", _softmax_transposed, [pins.test_decode_matches_torch_sdpa_gqa]),
    ("causal_allowed", _causal_top_left, [pins.test_decode_equals_varlen_with_one_query]),
    ("causal_allowed", _causal_off_by_one, [pins.test_causal_prefill_row_equals_decode_prefix]),
    ("lse_merge", _merge_no_rescale, [pins.test_lse_merge_equals_full_softmax]),
]


def _run_pin(fn):
    import inspect
    import os
    params = inspect.signature(fn).parameters
    kwargs = {}
    defaults = {"dtype": "f16", "hq": 4, "hkv": 2, "causal": True, "seed": 0, "which": 0,
                "golden_dir": os.path.join(os.path.dirname(__file__), "golden")}
    for name in params:
        kwargs[name] = defaults[name]
    fn(**kwargs)


def test_pins_pass_unmutated():
    for _, _, tests in MUTATIONS:
        for t in tests:
            _run_pin(t)


@pytest.mark.parametrize("idx", range(len(MUTATIONS)))
def test_mutation_is_caught(monkeypatch, idx):
    name, bad, tests = MUTATIONS[idx]
    monkeypatch.setattr(pa, name, bad)
    monkeypatch.setattr(pins.oracle, name, bad, raising=False)
    caught = False
    for t in tests:
        try:
            _run_pin(t)
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught, f"mutation {bad.__name__} of {name} slipped past {[t.__name__ for t in tests]}"


def test_gqa_map_mistake_is_caught(monkeypatch):
    """Query head h read against kv head h % Hkv instead of h // (Hq/Hkv)."""
    real = pa.decode

    def decode_mod_map(q, k_cache, v_cache, block_table, context_lens, block_size, scale, dtype,
                       compute=np.float64, pairs=None, return_weights=False):
        bsz, hq, d = q.shape
        hkv = k_cache.shape[2]
        out = np.empty((bsz, hq, d))
        for r in range(hq // hkv):
            # heads r*hkv + k (k < hkv) all have h % hkv == k: run them with one
            # query head per kv head so that head k reads kv head k
            heads = [r * hkv + k for k in range(hkv)]
            out[:, heads] = real(q[:, heads], k_cache, v_cache, block_table, context_lens,
                                 block_size, scale, dtype, compute)
        return out

    monkeypatch.setattr(pins.oracle, "decode", decode_mod_map)
    with pytest.raises(AssertionError):
        pins.test_decode_matches_torch_sdpa_gqa()
