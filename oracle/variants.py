"""CPU oracle for the attention variants: a sliding window (band) and ALiBi
position biases, for decode and packed varlen.

TEST INFRASTRUCTURE, like the rest of ``oracle/``.

The skill page lists a "Band" (sliding-window) mask mode for prefill and
decode that needs a count of preceding tokens (``pre_tokens``), and the FA
call on the cann-recipes-infer page takes ``alibi_slopes`` for ALiBi
positional encoding. Neither is spelled out; the readings taken:

* positions are aligned to the last key, as for the causal mask: local query
  i of a sequence with Lq queries and Lk keys sits at p = i + Lk - Lq (a
  decode query at p = Lk - 1);
* window ``window_left`` >= 0: the query sees keys j >= p - window_left (the
  query itself and window_left keys before it); with causal also j <= p;
  with causal off, keys after p stay visible. A negative value: no window;
* ALiBi: query head h adds ``alibi_slopes[h] * (j - p)`` to the scaled
  score of key j (a penalty growing with distance for the keys before the
  query);
* a query with no allowed key outputs 0.

Everything else is ``paged_attention.decode`` / ``varlen``: textbook softmax
over the allowed keys in float64.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import gather_kv, widen


def attend(q_vec, keys, values, scale, positions, p, slope, window_left, causal=True,
           lk=None):
    """One query at position p over keys at ``positions`` (ascending ints):
    allowed keys by the window / causal rule, ALiBi bias slope * (j - p)."""
    pos = np.asarray(positions, dtype=np.int64)
    allowed = np.ones(pos.shape, dtype=bool)
    if causal:
        allowed &= pos <= p
    if window_left is not None and window_left >= 0:
        allowed &= pos >= p - window_left
    if not allowed.any():
        return np.zeros(values.shape[1], dtype=np.float64)
    k, v, j = keys[allowed], values[allowed], pos[allowed].astype(np.float64)
    s = scale * (k @ q_vec) + slope * (j - p)
    s = s - s.max()
    w = np.exp(s)
    w = w / w.sum()
    return w @ v


def decode_ext(q, k_cache, v_cache, block_table, context_lens, block_size, scale, dtype,
               alibi_slopes=None, window_left=-1, pairs=None, kv_dtype=None):
    """Single-token paged decode with optional ALiBi slopes [Hq] and window."""
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    bsz, hq, d = q.shape
    group = hq // k_cache.shape[2]
    qf = widen(q, dtype)
    slopes = np.zeros(hq) if alibi_slopes is None else np.asarray(alibi_slopes, np.float64)
    out = np.full((bsz, hq, d), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(bsz) for h in range(hq)]
    for b, h in pairs:
        n = int(context_lens[b])
        if n == 0:
            out[b, h] = 0.0
            continue
        kv = h // group
        keys = widen(np.ascontiguousarray(gather_kv(k_cache, block_table[b], n, block_size)[:, kv]),
                     kv_dtype)
        vals = widen(np.ascontiguousarray(gather_kv(v_cache, block_table[b], n, block_size)[:, kv]),
                     kv_dtype)
        out[b, h] = attend(qf[b, h], keys, vals, scale, range(n), n - 1, slopes[h], window_left)
    return out


def varlen_ext(q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, causal, block_size,
               dtype, alibi_slopes=None, window_left=-1, rows=None, scale=None):
    """Packed varlen with optional ALiBi slopes [Hq] and window."""
    total_q, hq, d = q.shape
    group = hq // k_cache.shape[2]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qf = widen(q, dtype)
    slopes = np.zeros(hq) if alibi_slopes is None else np.asarray(alibi_slopes, np.float64)
    out = np.full((total_q, hq, d), np.nan)
    cu = [int(x) for x in cu_seqlens_q]
    want = None
    if rows is not None:
        want = {}
        for r, h in rows:
            want.setdefault(r, set()).add(h)
    for b in range(len(cu) - 1):
        lo, hi = cu[b], cu[b + 1]
        lq, lk = hi - lo, int(seq_lens[b])
        if lq == 0 or (want is not None and not any(r in want for r in range(lo, hi))):
            continue
        if lk > 0:
            k_seq = gather_kv(k_cache, block_table[b], lk, block_size)
            v_seq = gather_kv(v_cache, block_table[b], lk, block_size)
        for h in range(hq):
            kv = h // group
            if lk > 0:
                keys = widen(np.ascontiguousarray(k_seq[:, kv]), dtype)
                vals = widen(np.ascontiguousarray(v_seq[:, kv]), dtype)
            for i in range(lq):
                r = lo + i
                if want is not None and h not in want.get(r, ()):
                    continue
                if lk == 0:
                    out[r, h] = 0.0
                    continue
                out[r, h] = attend(qf[r, h], keys, vals, scale, range(lk), i + lk - lq, slopes[h],
                                   window_left, causal)
    return out

