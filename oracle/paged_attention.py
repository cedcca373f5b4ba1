"""CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library
and its Python binding) never calls it, and this module shares no code with
that path.

What it computes, and where the pages define it:

* ``slot_of`` / ``write_kv`` -- logical -> physical address translation and
  the KV write scatter. The pages ("model-infer-kvcache" skill page,
  section 3.1 "physical memory layout and logical mapping") give the mapping
  ``logical block = pos // block_size``, ``offset = pos % block_size``,
  ``physical block = block_table[b, logical block]``,
  ``slot = physical block * block_size + offset``; section 3.3 says the write
  op is addressed by ``slot_mapping`` and the attention read by
  ``block_table`` with the same addressing.
* ``gather_kv`` -- reads a sequence's first ``n`` tokens back through its
  block_table row into a contiguous array (the vLLM-on-CANN page,
  ``read_kv`` in its ``PagedKVCache`` listing, describes the same read).
* ``decode`` / ``varlen`` -- textbook softmax attention over the gathered
  keys: scores ``scale * <q, k_j>``, max-subtracted softmax over the allowed
  keys, weighted sum of values. Decode lets a single query see every one of
  ``context_lens[b]`` keys (sparse_mode 0 in the skill page's Appendix C);
  varlen prefill applies a causal mask per packed sequence (sparse_mode 3;
  "Paged KV infra" page section 3.1 on cu_seqlens: each sequence gets its own
  tril(len_i), no padding).
* ``lse_merge`` -- exact merge of per-partition (max, sum, unnormalised
  output) triples into the softmax over the union (the vLLM-on-CANN page:
  scattered blocks force block-by-block online merging).

Readings taken where the pages are silent:
GQA maps query head h to kv head h // (Hq // Hkv); causal alignment is
bottom-right (query i of a sequence with Lq queries and Lk keys sees keys
j <= i + Lk - Lq); a query with no allowed key outputs exactly 0; a context
length of 0 outputs exactly 0; negative slots are skipped by the write.

Storage conventions: fp32 data is numpy.float32, fp16 is numpy.float16 and
bf16 is numpy.uint16 holding the bf16 bit pattern (numpy has no bf16). The
oracle widens every stored value exactly to float64 (or float32 on request)
before any arithmetic.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage <-> real numbers (exact widening only)
# ---------------------------------------------------------------------------

_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def widen(arr: np.ndarray, dtype: str, compute=np.float64) -> np.ndarray:
    """Exactly widen stored values to ``compute`` (float64 by default).

    bf16 bit patterns become float32 by placing the 16 stored bits in the
    high half of a 32-bit word; that float32 is exact, and so is its float64.
    """
    if dtype == "bf16":
        if arr.dtype != np.uint16:
            raise TypeError("bf16 storage must be uint16 bit patterns")
        f32 = (arr.astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(compute)
    if dtype == "f64":   # already real numbers (e.g. a dequantised int8 pool)
        if arr.dtype != np.float64:
            raise TypeError(f"f64 data must be float64, got {arr.dtype}")
        return arr.astype(compute)
    want = _STORAGE[dtype]
    if arr.dtype != want:
        raise TypeError(f"{dtype} storage must be {want}, got {arr.dtype}")
    return arr.astype(compute)


# ---------------------------------------------------------------------------
# address translation and the KV write
# ---------------------------------------------------------------------------


def slot_of(block_table: np.ndarray, b: int, pos: int, block_size: int) -> int:
    """Physical slot of token ``pos`` of sequence ``b``.

    Skill page, section 3.1: logical block pos // bs, offset pos % bs,
    physical block block_table[b, logical block], slot = physical * bs + offset.
    """
    logical_block = pos // block_size
    offset = pos % block_size
    physical_block = int(block_table[b, logical_block])
    return physical_block * block_size + offset


def write_kv(k_cache, v_cache, key, value, slot_mapping, block_size):
    """Scatter new tokens into the pool; returns new (k_cache, v_cache).

    For each token t in order with s = slot_mapping[t] >= 0, row
    ``cache[s // block_size, s % block_size]`` (all kv heads, all dims) is
    replaced by ``key[t]`` / ``value[t]``. Pure bit copy in the storage dtype.
    Inputs are not modified. Duplicate non-negative slots are a caller error
    and raise here, because which token wins is then undefined.
    """
    k_out = k_cache.copy()
    v_out = v_cache.copy()
    num_blocks = k_cache.shape[0]
    slots = [int(s) for s in slot_mapping]
    live = [s for s in slots if s >= 0]
    if len(set(live)) != len(live):
        raise ValueError("duplicate slots in slot_mapping")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if blk >= num_blocks:
            raise IndexError(f"slot {s} is outside the pool")
        k_out[blk, off] = key[t]
        v_out[blk, off] = value[t]
    return k_out, v_out


def gather_kv(cache, block_table_row, n, block_size):
    """Return the first ``n`` tokens of one sequence as ``[n, Hkv, D]``
    storage, read through its block_table row (skill page, section 3.1)."""
    num_blocks, bs, hkv, d = cache.shape
    assert bs == block_size
    flat = cache.reshape(num_blocks * block_size, hkv, d)
    idx = np.empty(n, dtype=np.int64)
    for j in range(n):
        blk = int(block_table_row[j // block_size])
        if not 0 <= blk < num_blocks:
            raise IndexError(f"token {j}: block id {blk} outside the pool")
        idx[j] = blk * block_size + j % block_size
    return flat[idx]


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def softmax_attention(q_vec, keys, values, scale):
    """Textbook attention of one query over ``keys``/``values``.

    Returns (output vector, weights). No allowed key -> (zeros, empty).
    """
    n = keys.shape[0]
    d = values.shape[1] if values.ndim == 2 else q_vec.shape[0]
    if n == 0:
        return np.zeros(d, dtype=q_vec.dtype), np.zeros(0, dtype=q_vec.dtype)
    s = scale * (keys @ q_vec)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ values, p


def decode(q, k_cache, v_cache, block_table, context_lens, block_size, scale,
           dtype, compute=np.float64, pairs=None, return_weights=False, kv_dtype=None):
    """Single-token paged decode.

    q: [B, Hq, D]; caches [NB, bs, Hkv, D] in ``dtype`` storage.
    For each sequence b and query head h (kv head h // (Hq // Hkv)), the
    query attends over the ``context_lens[b]`` tokens read through
    ``block_table[b]``. ``pairs`` optionally restricts the work to a list of
    (b, h); the other rows of the result are left as NaN. ``kv_dtype``
    (default ``dtype``) is the storage of the caches when it differs from q's.
    Returns out [B, Hq, D] in ``compute`` (and weights per (b, h) if asked).
    """
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    bsz, hq, d = q.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    qf = widen(q, dtype, compute)
    out = np.full((bsz, hq, d), np.nan, dtype=compute)
    weights = {}
    if pairs is None:
        pairs = [(b, h) for b in range(bsz) for h in range(hq)]
    by_seq = {}
    for b, h in pairs:
        by_seq.setdefault(b, []).append(h)
    for b, heads in by_seq.items():
        n = int(context_lens[b])
        kv_needed = sorted({h // group for h in heads})
        if n > 0:
            k_seq = gather_kv(k_cache, block_table[b], n, block_size)
            v_seq = gather_kv(v_cache, block_table[b], n, block_size)
        for kvh in kv_needed:
            if n > 0:
                keys = widen(np.ascontiguousarray(k_seq[:, kvh, :]), kv_dtype, compute)
                vals = widen(np.ascontiguousarray(v_seq[:, kvh, :]), kv_dtype, compute)
            else:
                keys = np.zeros((0, d), dtype=compute)
                vals = np.zeros((0, d), dtype=compute)
            for h in heads:
                if h // group != kvh:
                    continue
                o, p = softmax_attention(qf[b, h], keys, vals, compute(scale))
                out[b, h] = o
                weights[(b, h)] = p
    if return_weights:
        return out, weights
    return out


def causal_allowed(i, lq, lk):
    """Number of keys query i (0-based, local) may see under the
    bottom-right causal reading: keys j with j <= i + lk - lq, and j < lk."""
    return max(0, min(lk, i + lk - lq + 1))


def varlen(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, causal,
           block_size, dtype, compute=np.float64, scale=None, rows=None):
    """Packed variable-length prefill over the paged cache.

    q: [total_q, Hq, D]; sequence b owns query rows
    [cu_seqlens_q[b], cu_seqlens_q[b+1]) and keys 0 .. seq_lens[b]-1 read
    through block_table[b]. With ``causal``, local query i sees keys
    j <= i + Lk - Lq (bottom-right alignment). Scale defaults to 1/sqrt(D).
    ``rows`` optionally restricts the work to a list of (global row, head);
    the other outputs stay NaN.
    """
    total_q, hq, d = q.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    cu = [int(x) for x in cu_seqlens_q]
    if cu[0] != 0 or cu[-1] != total_q or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens_q must start at 0, end at total_q, and not decrease")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qf = widen(q, dtype, compute)
    out = np.full((total_q, hq, d), np.nan, dtype=compute)
    want = None
    if rows is not None:
        want = {}
        for r, h in rows:
            want.setdefault(r, set()).add(h)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        lq, lk = hi - lo, int(seq_lens[b])
        if lq == 0:
            continue
        if want is not None and not any(r in want for r in range(lo, hi)):
            continue
        if lk > 0:
            k_seq = gather_kv(k_cache, block_table[b], lk, block_size)
            v_seq = gather_kv(v_cache, block_table[b], lk, block_size)
        for h in range(hq):
            kvh = h // group
            if lk > 0:
                keys = widen(np.ascontiguousarray(k_seq[:, kvh, :]), dtype, compute)
                vals = widen(np.ascontiguousarray(v_seq[:, kvh, :]), dtype, compute)
            for i in range(lq):
                r = lo + i
                if want is not None and h not in want.get(r, ()):
                    continue
                n_allowed = causal_allowed(i, lq, lk) if causal else lk
                if n_allowed == 0:
                    out[r, h] = 0.0
                    continue
                o, _ = softmax_attention(qf[r, h], keys[:n_allowed], vals[:n_allowed],
                                         compute(scale))
                out[r, h] = o
    return out


# ---------------------------------------------------------------------------
# split-KV algebra
# ---------------------------------------------------------------------------


def partial_softmax(q_vec, keys, values, scale):
    """(m, l, o) for one partition: m = max score, l = sum exp(s - m),
    o = sum exp(s - m) * v (unnormalised). Empty partition -> (-inf, 0, 0)."""
    if keys.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(values.shape[1] if values.ndim == 2 else q_vec.shape[0])
    s = scale * (keys @ q_vec)
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ values


def lse_merge(parts):
    """Merge partition triples into the normalised output over their union:
    M = max m_p, L = sum l_p exp(m_p - M), out = sum exp(m_p - M) o_p / L.
    All partitions empty -> zeros."""
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    if len(parts) == 0 or np.all(np.isneginf(ms)):
        d = parts[0][2].shape[0] if parts else 0
        return np.zeros(d)
    big_m = ms.max()
    total_l = 0.0
    acc = np.zeros_like(parts[0][2], dtype=np.float64)
    for m, l, o in parts:
        if np.isneginf(m):
            continue
        w = np.exp(m - big_m)
        total_l += l * w
        acc = acc + w * o
    return acc / total_l
