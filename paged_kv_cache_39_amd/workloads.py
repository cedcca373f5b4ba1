"""Seeded synthetic workloads for paged KV-cache attention.

Pure data generation (NumPy only): sequence lengths, a random assignment of
physical blocks, query/key/value values drawn N(0, 1) in float32 and rounded
to the storage dtype, and the per-token slot of every written token. Both
the HIP path and the CPU oracle consume the arrays produced here; this module
contains no attention arithmetic.

Storage conventions: "f32" -> numpy.float32, "f16" -> numpy.float16,
"bf16" -> numpy.uint16 bit patterns (round-to-nearest-even from float32).

The named workloads follow the shapes of the pages' LLaMA-7B-class runs
(32 heads x head_dim 128, batch 8 at 2048 tokens), plus GQA, ragged,
packed-prefill and long-context variants. Draw order per workload:
lengths -> block permutation -> q -> K -> V, from numpy.random.default_rng.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage dtype with round-to-nearest-even (inputs finite)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def nan_fill_value(dtype: str):
    """A quiet-NaN element in storage form, used for never-written pool cells."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return STORAGE[dtype](np.nan)


def normal(rng, shape, dtype):
    return round_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclass
class PagedCase:
    """One synthetic paged-attention workload (host arrays)."""

    name: str
    dtype: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_table: np.ndarray          # int32 [B, max_blocks_per_seq], -1 = unused
    seq_lens: np.ndarray             # int32 [B]   (KV length per sequence)
    q: np.ndarray                    # decode: [B, Hq, D]; varlen: [total_q, Hq, D]
    key: np.ndarray                  # [T, Hkv, D] tokens to write
    value: np.ndarray                # [T, Hkv, D]
    slot_mapping: np.ndarray         # int32 [T]
    scale: float
    cu_seqlens_q: np.ndarray | None = None   # varlen only, int32 [B+1]
    causal: bool = True
    new_token_rows: np.ndarray | None = None  # rows of key/value written per decode step
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)

    def empty_pool(self) -> np.ndarray:
        """A pool with every cell set to NaN (sentinel for unwritten slots)."""
        return np.full(self.pool_shape(), nan_fill_value(self.dtype), dtype=STORAGE[self.dtype])

    def kv_bytes_read(self) -> int:
        """Algorithmic KV bytes one decode call reads: every context token's
        K and V rows of every kv head, once."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * \
            self.head_dim * ELEM_BYTES[self.dtype]

    def decode_bytes(self) -> int:
        """KV bytes + q + out + the live part of block_table + context_lens."""
        e = ELEM_BYTES[self.dtype]
        qo = 2 * self.num_seqs * self.num_q_heads * self.head_dim * e
        nblk = int(sum(-(-int(n) // self.block_size) for n in self.seq_lens))
        return self.kv_bytes_read() + qo + 4 * nblk + 4 * self.num_seqs

    def prefill_flops(self) -> int:
        """4 * D * Hq * (number of (query, key) pairs the mask allows)."""
        pairs = 0
        cu = self.cu_seqlens_q
        for b in range(self.num_seqs):
            lq = int(cu[b + 1] - cu[b])
            lk = int(self.seq_lens[b])
            if self.causal:
                i = np.arange(lq, dtype=np.int64)
                pairs += int(np.clip(i + lk - lq + 1, 0, lk).sum())
            else:
                pairs += lq * lk
        return 4 * self.head_dim * self.num_q_heads * pairs


def _assign_blocks(rng, lens, block_size, num_blocks, max_blocks=None, perm=None):
    need = [-(-int(n) // block_size) for n in lens]
    if perm is None:
        perm = rng.permutation(num_blocks)
    if sum(need) > num_blocks:
        raise ValueError("pool too small")
    width = max(max(need) if need else 1, 1) if max_blocks is None else max_blocks
    table = np.full((len(lens), width), -1, dtype=np.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    return table


def _token_slots(table, lens, block_size):
    """Slot of every token of every sequence, in sequence order."""
    out = []
    for b, n in enumerate(lens):
        pos = np.arange(int(n), dtype=np.int64)
        out.append(table[b, pos // block_size].astype(np.int64) * block_size + pos % block_size)
    if not out:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(out).astype(np.int32)


def decode_case(seed, context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                dtype, num_blocks=None, spare=0.1, max_blocks=None, name="decode",
                perm_blocks=None, values=True):
    """A decode workload: every context token written, then one query per
    sequence. ``context_lens`` may be an int list or a callable(rng).
    ``values=False`` stops after the metadata draws (q/key/value are None)."""
    rng = np.random.default_rng(seed)
    lens = context_lens(rng) if callable(context_lens) else list(context_lens)
    lens = [int(x) for x in lens]
    need = sum(-(-n // block_size) for n in lens)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(need * (1.0 + spare)))
    perm = rng.permutation(num_blocks) if perm_blocks is None else perm_blocks(rng, num_blocks)
    table = _assign_blocks(rng, lens, block_size, num_blocks, max_blocks, perm)
    bsz = len(lens)
    total = sum(lens)
    q = key = value = None
    if values:
        q = normal(rng, (bsz, num_q_heads, head_dim), dtype)
        key = normal(rng, (total, num_kv_heads, head_dim), dtype)
        value = normal(rng, (total, num_kv_heads, head_dim), dtype)
    slots = _token_slots(table, lens, block_size)
    # the last token of each non-empty sequence is the one a decode step writes
    ends = np.cumsum(lens)
    new_rows = np.array([e - 1 for e, n in zip(ends, lens) if n > 0], dtype=np.int64)
    return PagedCase(name=name, dtype=dtype, block_size=block_size, num_blocks=num_blocks,
                     num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                     block_table=table, seq_lens=np.array(lens, dtype=np.int32), q=q,
                     key=key, value=value, slot_mapping=slots,
                     scale=1.0 / math.sqrt(head_dim), new_token_rows=new_rows)


def varlen_case(seed, q_lens, kv_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                dtype, causal=True, spare=0.1, num_blocks=None, name="varlen", values=True):
    """A packed prefill workload: ``kv_lens[b]`` tokens of sequence b are
    written to the pool; its last ``q_lens[b]`` positions are the queries.
    Either list may be a callable(rng) (kv_lens may then use q_lens).
    ``values=False`` stops after the metadata draws (q/key/value are None)."""
    rng = np.random.default_rng(seed)
    ql = q_lens(rng) if callable(q_lens) else list(q_lens)
    ql = [int(x) for x in ql]
    kl = kv_lens(rng, ql) if callable(kv_lens) else list(kv_lens)
    kl = [int(x) for x in kl]
    need = sum(-(-n // block_size) for n in kl)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(need * (1.0 + spare)))
    perm = rng.permutation(num_blocks)
    table = _assign_blocks(rng, kl, block_size, num_blocks, None, perm)
    total_q = sum(ql)
    total = sum(kl)
    q = key = value = None
    if values:
        q = normal(rng, (total_q, num_q_heads, head_dim), dtype)
        key = normal(rng, (total, num_kv_heads, head_dim), dtype)
        value = normal(rng, (total, num_kv_heads, head_dim), dtype)
    slots = _token_slots(table, kl, block_size)
    cu = np.zeros(len(ql) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    return PagedCase(name=name, dtype=dtype, block_size=block_size, num_blocks=num_blocks,
                     num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                     block_table=table, seq_lens=np.array(kl, dtype=np.int32), q=q,
                     key=key, value=value, slot_mapping=slots,
                     scale=1.0 / math.sqrt(head_dim), cu_seqlens_q=cu, causal=causal)


def int8_scales(num_kv_heads):
    """Per-kv-head int8 dequantisation scales for the synthetic N(0,1) data:
    fixed, distinct per head, clipping the tails beyond about 3 sigma."""
    h = np.arange(num_kv_heads, dtype=np.float64)
    k_scale = ((3.0 + 0.25 * (h % 4)) / 127.0).astype(np.float32)
    v_scale = ((3.25 + 0.125 * (h % 5)) / 127.0).astype(np.float32)
    return k_scale, v_scale


def alibi_slopes(num_heads):
    """ALiBi slopes for the synthetic runs: 2^(-8 (h + 1) / H), the geometric
    sequence of the ALiBi paper for a power-of-two head count."""
    return np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)],
                    dtype=np.float32)


def log_uniform_lengths(rng, n, lo, hi):
    """round(exp(U(ln lo, ln hi))) clipped to [lo, hi]."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return [int(v) for v in np.clip(np.rint(x), lo, hi)]


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: "tiny paged decode: ctx [37, 100], 4/4 heads, D 64, bs 16, pool 16, fp32",
    2: "LLaMA-7B-shaped decode: batch 8 x ctx 2048, 32/32 heads, D 128, bs 16, pool 4096, fp16",
    3: "ragged GQA decode: batch 32, ctx U{50..2000}, 32/8 heads, D 128, bs 32, bf16",
    4: "packed varlen causal prefill: 16 seqs, len log-U[64, 2048], 32/8 heads, D 128, bs 128, bf16",
    5: "long-context split-KV decode: batch 4 x ctx 131072, 64/8 heads, D 128, bs 128, pool 4096, bf16",
    6: "mixed varlen batch: 24 decode (Lq 1) + 6 multi-token decode (Lq 4), ctx U{512..4096}, "
       "+ 2 chunked prefills (Lq 512 over Lk 2048); 32/8 heads, D 128, bs 16, bf16",
}


def _mixed_lengths(rng):
    """Query / KV lengths of the mixed batch: 24 single-token decodes and 6
    four-token decodes over contexts U{512..4096}, then two 512-token chunks
    continuing 1536 cached tokens."""
    ctx = rng.integers(512, 4097, size=30).tolist()
    ql = [1] * 24 + [4] * 6 + [512, 512]
    kl = ctx + [2048, 2048]
    return ql, kl


def workload(c: int, values: bool = True) -> PagedCase:
    """Named workload ``c`` (1..6), seeded with 1000 + c. ``values=False``
    returns only the metadata (lengths, block table, slots)."""
    seed = 1000 + c
    if c == 1:
        return decode_case(seed, [37, 100], 4, 4, 64, 16, "f32", num_blocks=16,
                           name="tiny_decode_fp32", values=values)
    if c == 2:
        return decode_case(seed, [2048] * 8, 32, 32, 128, 16, "f16", num_blocks=4096,
                           name="llama7b_decode_fp16_b8_ctx2048", values=values)
    if c == 3:
        return decode_case(seed, lambda rng: rng.integers(50, 2001, size=32).tolist(),
                           32, 8, 128, 32, "bf16", spare=0.1,
                           name="ragged_gqa_decode_bf16_b32", values=values)
    if c == 4:
        return varlen_case(seed, lambda rng: log_uniform_lengths(rng, 16, 64, 2048),
                           lambda rng, ql: ql, 32, 8, 128, 128, "bf16", causal=True,
                           spare=0.1, name="packed_varlen_causal_prefill_bf16_16seq",
                           values=values)
    if c == 5:
        return decode_case(seed, [131072] * 4, 64, 8, 128, 128, "bf16", num_blocks=4096,
                           name="long_ctx_splitkv_decode_bf16_b4_ctx131072", values=values)
    if c == 6:
        box = {}

        def qlens(rng):
            box["ql"], box["kl"] = _mixed_lengths(rng)
            return box["ql"]

        return varlen_case(seed, qlens, lambda rng, ql: box["kl"], 32, 8, 128, 16, "bf16",
                           causal=True, spare=0.1, name="mixed_decode_chunked_prefill_bf16",
                           values=values)
    raise ValueError(f"no workload {c}")
