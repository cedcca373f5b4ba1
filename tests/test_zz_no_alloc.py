"""GPU check of paged_kv_write_decode_noalloc (the decode step with the
split-KV partials in the library's own scratch) against paged_kv_write_decode
(the same step with a caller workspace), through the C ABI.

Two calls in a row share the scratch; the second has a smaller input, so
anything it read from the first call's partials would show. Each call runs
on a copy of the same pre-written pool for both entry points: the pools must
match each other and the oracle's write bit for bit, and the outputs must
agree with each other and with the oracle within the attention tolerance
(bf16 1.5e-2, fp16 2e-3; the two calls may differ in summation order)."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_39_amd import binding
from paged_kv_cache_39_amd import workloads as wl
from tests.gpu_util import ATOL, DeviceCase, ints, max_abs_err, to_device, to_host, widen_host

pytestmark = pytest.mark.gpu


def bits(a):
    return a.view(np.uint16)


def step_both(case):
    """Pre-write every context token but each sequence's last, then run the
    step through both entry points on copies of that pool. Returns host
    (out, k, v) of the workspace call, of the no-allocation call, and the
    oracle's pool after the step."""
    dc = DeviceCase(case, write=False)
    rows = case.new_token_rows
    pre = case.slot_mapping.copy()
    pre[rows] = -1
    binding.paged_kv_write(dc.k_cache, dc.v_cache, dc.key, dc.value, ints(pre))
    nk = to_device(case.key[rows], case.dtype)
    nv = to_device(case.value[rows], case.dtype)
    sm = ints(case.slot_mapping[rows])
    res = []
    for fn in (binding.paged_kv_write_decode, binding.paged_kv_write_decode_noalloc):
        k, v = dc.k_cache.clone(), dc.v_cache.clone()
        out = torch.full_like(dc.q, float("nan"))
        fn(out, dc.q, k, v, nk, nv, sm, dc.block_table, dc.seq_lens, case.block_size,
           case.scale)
        torch.cuda.synchronize()
        res.append((to_host(out, case.dtype), to_host(k, case.dtype), to_host(v, case.dtype)))
    k_ref, v_ref = oracle.write_kv(case.empty_pool(), case.empty_pool(), case.key, case.value,
                                   case.slot_mapping, case.block_size)
    return res[0], res[1], k_ref, v_ref


def check(case):
    print(f"no-alloc step: {case.name} dtype={case.dtype} ctx={case.seq_lens.tolist()} "
          f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} bs={case.block_size}", flush=True)
    need = binding.paged_attention_decode_workspace_size(
        case.num_seqs, case.num_q_heads, case.head_dim, case.max_blocks_per_seq, case.block_size)
    assert 0 < need <= binding.NOALLOC_SCRATCH_BYTES   # the split plan, inside the scratch
    (out_a, k_a, v_a), (out_b, k_b, v_b), k_ref, v_ref = step_both(case)
    assert np.array_equal(bits(k_b), bits(k_a)) and np.array_equal(bits(v_b), bits(v_a))
    assert np.array_equal(bits(k_b), bits(k_ref)) and np.array_equal(bits(v_b), bits(v_ref))
    tol = ATOL[case.dtype]
    assert max_abs_err(out_b, widen_host(out_a, case.dtype), case.dtype) <= tol
    want = oracle.decode(case.q, k_ref, v_ref, case.block_table, case.seq_lens,
                         case.block_size, case.scale, case.dtype)
    assert max_abs_err(out_b, want, case.dtype) <= tol
    assert max_abs_err(out_a, want, case.dtype) <= tol


def test_noalloc_two_calls_second_smaller():
    # 1: 16/2 heads over contexts up to 9000 tokens (512-token partitions +
    #    the reduce); 2: fewer, shorter sequences of another shape, fp16
    big = wl.decode_case(730, [9000, 2049, 8191, 5000], 16, 2, 128, 32, "bf16")
    small = wl.decode_case(731, [3000, 700], 8, 2, 64, 16, "f16")
    check(big)
    check(small)
