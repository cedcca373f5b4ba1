// Paged decode attention: one query token per sequence attends over its
// context, read block by block through the block table.
//
// Definition: out[b,h] = sum_j softmax_j(scale * <q[b,h], K_j>) V_j over the
// context_lens[b] tokens of sequence b ("model-infer-kvcache" skill page,
// Appendix C: decode uses no mask and the KV length bounds the keys; the
// "ATB PagedAttention" page computes it page by page with an online softmax).
//
// Split-KV: the context is cut into partitions (kDecodePart tokens here; the
// matrix-core kernel's launch plan takes 512 to 4096). One workgroup handles
// one (partition, group of query heads sharing a kv head, sequence) and
// produces, per query head, the partial triple
//   m = max score (log2 units), l = sum 2^(s - m), o = sum 2^(s - m) V.
// A sequence with a single partition is normalised in place; otherwise the
// reduce kernel merges the triples exactly (the vLLM-on-CANN page: physically
// scattered blocks are combined with a block-by-block online softmax).
//
// Lane mapping (wave64): a wave is 4 rows of 16 lanes. A row works on one
// token at a time; each of its 16 lanes owns D/16 consecutive elements of the
// token's K and V rows (16 bytes for 16-bit types at D=128), so one wave-wide
// load instruction fetches 4 whole 256-byte rows. q.k is a 16-lane DPP
// reduction inside the row; the running max/sum live per row, and the 4 rows
// and the 4 waves are merged once at the end. The partition's block ids are
// staged in LDS once per workgroup and broadcast to scalar registers.

#include "debug_checks.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kMaxPartTokens = kDecodeMaxPart;   // longest partition a workgroup takes
constexpr int kQuadsPerIter = 8;                  // each row handles 8 tokens per iteration
constexpr int kTokPerIter = 4 * kQuadsPerIter;    // 32 tokens per wave iteration
// compile-time item kind of the decode kernel's item body (false: the
// workgroup's own row, true: the partner's tail)
template <bool V>
struct item_kind {
  static constexpr bool value = V;
};
// shortest tail a paired row hands over (a second item costs its workgroup
// about one more round trip to memory)
constexpr int kPairMinTail = 256;
// K/V bytes by which the longer row's piece exceeds the shorter row's
// workgroup's share: that workgroup also pays a second item's start (table,
// queries, first tile) and the hand-over, ~3-4 us of streaming (measured
// best among 64, 96, 128 and 160 KB on the ragged GQA batch)
constexpr int kPairBiasBytes = 96 * 1024;

template <class Ty, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_partition_kernel(
    typename Ty::storage* __restrict__ out, const typename Ty::storage* __restrict__ q,
    const typename Ty::storage* __restrict__ k_cache,
    const typename Ty::storage* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, float scale_log2, int num_q_heads, int num_kv_heads, int group,
    int log2_bs, int max_blocks_per_seq, int64_t num_blocks, int num_parts) {
  constexpr int EPL = D / 16;
  const int p = blockIdx.x;
  const int h0 = blockIdx.y * G;  // first query head of this workgroup
  const int kvh = h0 / group;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, row = lane >> 4, c = lane & 15;
  const int bs = 1 << log2_bs;

  int ctx = context_lens[b];
  PKV_DBG_REPORT(tid == 0 && (ctx < 0 || ctx > (max_blocks_per_seq << log2_bs)), kDbgLength);
  ctx = max(0, min(ctx, max_blocks_per_seq << log2_bs));
  const int part_start = p * kDecodePart;
  if (part_start >= ctx) {
    if (p == 0) {  // empty context: the output row is zero
      for (int i = tid; i < G * D; i += kDecThreads)
        out[((size_t)b * num_q_heads + h0 + i / D) * D + i % D] = from_f32<Ty>(0.f);
    }
    return;
  }
  const int ntok = min(kDecodePart, ctx - part_start);
  const int nparts_b = (ctx + kDecodePart - 1) / kDecodePart;

  __shared__ int s_blk[kDecodePart / 16];
  __shared__ float s_m[kDecWaves][G];
  __shared__ float s_l[kDecWaves][G];
  __shared__ float s_o[kDecWaves][G][D];

  const int nblk = (ntok + bs - 1) >> log2_bs;
  if (tid < nblk) {
    const int id = block_table[(size_t)b * max_blocks_per_seq + (part_start >> log2_bs) + tid];
    PKV_DBG_REPORT(!(id >= 0 && id < num_blocks), kDbgBlockId);
    s_blk[tid] = (id >= 0 && id < num_blocks) ? id : -1;
  }

  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const auto qc = load_chunk<Ty, EPL>(q + ((size_t)b * num_q_heads + h0 + g) * D + c * EPL);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[g][e] = qc.get(e) * scale_log2;
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  __syncthreads();

  const int row_stride = num_kv_heads * D;  // elements between consecutive slots
  const int lane_off = kvh * D + c * EPL;
  const int nchunks = (ntok + kTokPerIter - 1) / kTokPerIter;
  const int last_quad = (ntok - 1) & ~3;

  for (int ci = wave; ci < nchunks; ci += kDecWaves) {
    Chunk<Ty, EPL> kr[kQuadsPerIter], vr[kQuadsPerIter];
    bool valid[kQuadsPerIter];
#pragma unroll
    for (int u = 0; u < kQuadsPerIter; ++u) {
      const int tq = ci * kTokPerIter + 4 * u;     // first token of this quad (wave-uniform)
      const int tql = min(tq, last_quad);          // quads past the end re-read the last one
      const int tok = min(tql + row, ntok - 1);    // stays inside tql's block
      int blk = __builtin_amdgcn_readfirstlane(s_blk[tql >> log2_bs]);
      valid[u] = (tq + row < ntok) && (blk >= 0);
      blk = max(blk, 0);
      const typename Ty::storage* kb = k_cache + (size_t)blk * bs * row_stride;
      const typename Ty::storage* vb = v_cache + (size_t)blk * bs * row_stride;
      const int off = (tok & (bs - 1)) * row_stride + lane_off;
      kr[u] = load_chunk<Ty, EPL, true>(kb + off);
      vr[u] = load_chunk<Ty, EPL, true>(vb + off);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[kQuadsPerIter];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kQuadsPerIter; ++u) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[g][e], kr[u].get(e), acc);
        acc = row16_sum(acc);
        s[u] = valid[u] ? acc : -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      const float mnew = fmaxf(m[g], mx);
      const float mref = safe_max_ref(mnew);
      const float alpha = fast_exp2(m[g] - mref);
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
#pragma unroll
      for (int u = 0; u < kQuadsPerIter; ++u) {
        const float pu = fast_exp2(s[u] - mref);
        l[g] += pu;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pu, vr[u].get(e), o[g][e]);
      }
      m[g] = mnew;
    }
  }

  // merge the 4 rows of each wave (lanes c, c+16, c+32, c+48)
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {
      const float mo = shfl_xor_f(m[g], mask);
      const float lo = shfl_xor_f(l[g], mask);
      const float mn = fmaxf(m[g], mo);
      const float mr = safe_max_ref(mn);
      const float wa = fast_exp2(m[g] - mr), wb = fast_exp2(mo - mr);
      l[g] = l[g] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = o[g][e] * wa + shfl_xor_f(o[g][e], mask) * wb;
      m[g] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][g][c * EPL + e] = o[g][e];
      if (c == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  // merge the waves; one thread per (head, element)
  for (int i = tid; i < G * D; i += kDecThreads) {
    const int g = i / D, d = i % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mm = fmaxf(mm, s_m[w][g]);
    const float mr = safe_max_ref(mm);
    float ll = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float wt = fast_exp2(s_m[w][g] - mr);
      ll += s_l[w][g] * wt;
      acc += s_o[w][g][d] * wt;
    }
    const size_t bh = (size_t)b * num_q_heads + h0 + g;
    if (nparts_b == 1) {
      out[bh * D + d] = from_f32<Ty>(ll > 0.f ? acc / ll : 0.f);
    } else {
      ws_o[(bh * num_parts + p) * D + d] = acc;
      if (d == 0) {
        ws_ml[(bh * num_parts + p) * 2 + 0] = mm;
        ws_ml[(bh * num_parts + p) * 2 + 1] = ll;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core decode (fp16 / bf16). One workgroup per (partition, group of up
// to 16 query heads sharing a kv head, sequence); its WAVES waves walk the
// partition TT tokens (one tile) at a time, taking tiles on demand.
//
// K and V rows are fetched exactly as in the vector kernel (16 lanes x 16 B
// per 256-byte row, non-temporal) into registers, one tile ahead, and parked
// in a wave-private LDS tile. From there
//   S^T = K Q^T     (A: K rows, ds_read_b128; B: the group's queries, held in
//                    registers, heads padded to 16 with zeros; k = 32 MFMA)
//   O^T += V^T P^T  (A: V^T via the LDS transpose read; B: P^T straight from
//                    the S^T accumulators, rounded to the input type)
// so each lane owns one query head's statistics and output rows; the token
// max needs two cross-lane exchanges per tile and nothing else moves. The
// waves are merged through LDS at the end.
//
// Ragged batches: with one workgroup per whole context, the kernel time is
// that of the longest row (a lone compute unit streams ~45 GB/s). Rows are
// therefore paired longest with shortest and the longer row's tail moves to
// the shorter row's workgroup (see the pairing plan in the kernel); the two
// partial triples are merged by the workgroup that finishes second, through
// device-coherent stores and one exchange word per row.
// ---------------------------------------------------------------------------

template <int D, int WAVES, int TT>
struct MfLds {
  static constexpr int rowB = D * 2 + 16;            // padded row pitch (bytes)
  static constexpr int tileB = TT * rowB;             // one K or V tile
  static constexpr int waveB = 2 * tileB;
  static constexpr int totalB = WAVES * waveB;
  static constexpr int oRow = D + 4;                  // merge row pitch (floats): rows of
                                                      // successive heads start 4 banks apart
  static constexpr int mergeB = WAVES * 16 * (2 + oRow) * 4;
  static constexpr int bytes = totalB > mergeB ? totalB : mergeB;
};

// Q8: the cache holds int8 codes with per-kv-head scales (value = code *
// scale). A 16-byte load then carries 16 codes; they are widened exactly to
// Ty on the way into LDS, k_scale folds into the score scale and v_scale
// into the merged output, and everything between is the 16-bit path.
// EXT: the attention variants -- a sliding window (keys j >= ctx-1-window_left
// only, window_left >= 0) and ALiBi (score + alibi[h] * (j - (ctx-1)));
// alibi may be NULL and window_left negative. Positions are those of the
// decode query, the last token of its context.
// APP: the decode step's KV write rides along (one launch instead of two).
// new_k / new_v [B, Hkv, D] hold each sequence's new token, slot_mapping[b]
// its pool slot (skipped when negative or past the pool). In every
// workgroup whose partition holds the last position ctx-1, wave 0 walks the
// partition's last tile first and fetches the new row with it; when
// slot_mapping[b] is the table's slot of ctx-1 that row replaces the pool's
// (the values the write stores there), so no workgroup waits for the store,
// and the workgroup of the kv head's first head group stores it into the
// pool once its walk is done. The result equals the write followed by the
// decode as long as no other sequence of the call reads that slot (a
// sequence's last block is its own). Over an int8 cache (Q8) the new row is quantised with the kv head's
// scales first, to the codes the int8 write would store.
// The pool as the kernel reads it. Only the fused-write instances (APP)
// also store into it (through app_k_cache / app_v_cache, the same buffers),
// so only there may the read pointers not be restrict-qualified.
template <bool APP>
struct PoolRead {
  using type = const void* __restrict__;
};
template <>
struct PoolRead<true> {
  using type = const void*;
};

template <class Ty, int D, int WAVES, int TT, bool Q8, bool EXT, bool APP>
__global__ __launch_bounds__(WAVES * kWave) void decode_mfma_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    typename PoolRead<APP>::type k_cache, typename PoolRead<APP>::type v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ context_lens,
    float* __restrict__ ws_ml, float* __restrict__ ws_o, float scale_log2, int num_q_heads,
    int num_kv_heads, int group, int heads_per_wg, int log2_bs, int max_blocks_per_seq,
    int64_t num_blocks, int num_parts, int part_tokens, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, const float* __restrict__ alibi, int window_left,
    uint8_t* app_k_cache, uint8_t* app_v_cache, const void* __restrict__ new_k,
    const void* __restrict__ new_v, const int32_t* __restrict__ slot_mapping, int xcd_bit,
    unsigned long long* __restrict__ pair_words, unsigned long long epoch, int pair_seqs) {
  using L = MfLds<D, WAVES, TT>;
  constexpr int NT = WAVES * kWave;
  constexpr int EB = Q8 ? 1 : 2;      // bytes per cached element
  constexpr int EPC = 16 / EB;        // elements per 16-byte chunk
  constexpr int CPR = D / EPC;        // 16-byte chunks per cached row
  constexpr int RPI = kWave / CPR;    // rows per load instruction
  constexpr int LPI = TT / RPI;       // load instructions per tile
  constexpr int KS = D / 32;          // k-steps of q.k
  constexpr int ND = D / 16;          // 16-dim tiles of the output
  constexpr int NS = TT / 16;         // 16-token blocks per tile

  __shared__ __attribute__((aligned(16))) uint8_t s_mem[L::bytes];
  __shared__ int s_blk[kMaxPartTokens / 16];
  __shared__ int s_claim;   // next tile to hand out

  // Which (partition, head group, sequence) this workgroup takes. With
  // xcd_bit >= 0 the host found that bit xcd_bit of the head-group index
  // is bit 8 of every kv slice address the group reads; the workgroup then
  // takes an item whose bit 8 differs from its dispatch slot's parity (slot
  // i runs on XCD i mod 8): items 2k and 2k+1 trade slots.
  int p = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  if (xcd_bit >= 0) {
    const int slot = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int item = slot ^ 1, half_y = gridDim.y >> 1;
    int j = item >> 1;
    p = j % (int)gridDim.x;
    j /= (int)gridDim.x;
    const int yh = j % half_y;
    b = j / half_y;
    hg = ((yh >> xcd_bit) << (xcd_bit + 1)) | ((item & 1) << xcd_bit) |
         (yh & ((1 << xcd_bit) - 1));
  }
  const int h0 = hg * heads_per_wg;
  const int kvh = h0 / group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int lrow = lane / CPR, lch = lane % CPR;
  const int bs = 1 << log2_bs;
  static_assert(NT >= kMaxPartTokens / 16, "one block id per thread");
  static_assert(!APP || !EXT, "the fused write is a form of the plain decode");
  const int row_stride = num_kv_heads * D;
  const bool head_ok = l16 < heads_per_wg;

  // Pairing (pair_words set by the host: one workgroup per whole context,
  // at most 64 sequences). The sequences are ranked by context length,
  // longest first (ties by index), and rank k is paired with rank B-1-k.
  // When the longer context exceeds the split point -- the middle of the
  // two lengths moved toward the longer row by half of kPairBiasBytes,
  // rounded down to a multiple of the tile and the block -- by
  // at least kPairMinTail tokens, the longer row's workgroup stops there and
  // the shorter row's workgroup attends the rest after its own row. The two
  // partial triples meet in the workspace; the workgroup that finishes
  // second merges them. Every head group of a sequence pairs alike.
  int cut_own = -1;                             // own row ends here (head piece)
  int tail_seq = -1, tail_beg = 0;              // partner row's tail this workgroup takes
  // One item's attention, inlined once per item kind (each copy is
  // straight-line code with the item kind fixed).
  auto run_item = [&](auto tail_tag) __attribute__((always_inline)) {
    // item 0: the workgroup's own (partition of its) row; item 1: the tail of
    // the partner's row
    constexpr bool is_tail = decltype(tail_tag)::value;
    const int sb = is_tail ? tail_seq : b;
    const int pp = is_tail ? 0 : p;

    // pairing: every sequence's context length (lane s: sequence s),
    // requested in the same round trip as the item's own loads and ahead of
    // them (the plan then waits for it and the block ids, not the queries)
    int pair_raw = 0;
    if (!is_tail && pair_words != nullptr && lane < pair_seqs) pair_raw = context_lens[lane];
    // The context length, the partition's block ids (every entry a full
    // partition would use; those past the context are never read), the
    // queries and (APP) the new token's row and slot depend only on the
    // workgroup's indices: they are fetched in one round trip.
    const int part_start = is_tail ? tail_beg : pp * part_tokens;
    const int first_blk = part_start >> log2_bs;
    const int nblk_max = min(part_tokens >> log2_bs, max_blocks_per_seq - first_blk);
    const int id_raw =
        tid < nblk_max ? block_table[(size_t)sb * max_blocks_per_seq + first_blk + tid] : -1;
    // queries as the B operand: lane holds head h0 + l16, dims 32s + 8*g4 .. +8
    u32x4_t qb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qb[s] = head_ok ? load16<false>(q + ((size_t)sb * num_q_heads + h0 + l16) * D + 32 * s + 8 * g4)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }

    int ctx = context_lens[sb];
    PKV_DBG_REPORT(tid == 0 && (ctx < 0 || ctx > (max_blocks_per_seq << log2_bs)), kDbgLength);
    ctx = max(0, min(ctx, max_blocks_per_seq << log2_bs));
    const int app_slot = APP ? slot_mapping[sb] : -1;
    PKV_DBG_REPORT(APP && tid == 0 && (int64_t)app_slot >= (num_blocks << log2_bs), kDbgSlot);
    // the item's pair slot (0 head, 1 tail), or -1 for a whole partition
    // (item 0 learns whether it is cut only once its first loads are out)
    int pslot = is_tail ? 1 : -1;
    const bool pairing = !is_tail && pair_words != nullptr;
    // The pairing plan of item 0, computed by every wave once its first
    // tile is requested (the lengths came with the item's own loads, and the
    // search hides under that tile's latency), or right away by a workgroup
    // whose own row is empty. A cut row keeps [0, at), which holds the first
    // tile of every wave.
    auto plan = [&]() {
      const int nb = pair_seqs;
      const int maxc = max_blocks_per_seq << log2_bs;   // <= the partition: 4096
      int raw = pair_raw;
      asm volatile("" : "+v"(raw));   // not hoisted above the item's loads
      const int len = lane < nb ? max(0, min(raw, maxc)) : -1;
      // no pair differs by enough: nothing to plan
      if (wave_max_i(len) - (-wave_max_i(lane < nb ? -len : INT32_MIN + 1)) < 2 * kPairMinTail)
        return;
      // a unique key per sequence: the length, then the lower index first
      const int key = len >= 0 ? (len << 6) | (63 - lane) : -1;
      const int kb = lane_value(key, b);
      const int rb = __popcll(__builtin_amdgcn_ballot_w64(key > kb));
      const int rp = nb - 1 - rb;
      if (rp == rb) return;
      // the key of rank rp: the largest k with at least rp + 1 keys >= k
      int k = 0;
      for (int bit = 31 - __builtin_clz((maxc << 6) | 63); bit >= 0; --bit) {
        const int cand = k | (1 << bit);
        if (__popcll(__builtin_amdgcn_ballot_w64(key >= cand)) > rp) k = cand;
      }
      const int lb = kb >> 6, lp = k >> 6;
      const int quant = max(TT, bs);
      const int at = ((lb + lp + kPairBiasBytes / (2 * D * EB)) >> 1) & ~(quant - 1);
      // (a head piece keeps at least the first tile of every wave)
      if (max(lb, lp) - at < kPairMinTail || at < WAVES * TT) return;
      if (rb < rp) {
        cut_own = at;
      } else {
        tail_seq = 63 - (k & 63);
        tail_beg = at;
      }
    };
    // APP: the pool row is stored by the workgroup of the partition holding
    // ctx-1 (partition 0 for an empty context) and of the kv head's first head
    // group, from its wave 0, lanes of rows 0 (K) and 1 (V), chunk lch each
    // element index of the lane's chunk of the new row (new_k / new_v hold Ty)
    const size_t app_src = (size_t)sb * row_stride + kvh * D + lch * EPC;
    const bool holds_last = is_tail || pp == (ctx > 0 ? (ctx - 1) / part_tokens : 0);
    bool app_writer = APP && wave == 0 && h0 == kvh * group && holds_last && app_slot >= 0 &&
                      (int64_t)app_slot < (num_blocks << log2_bs);
    auto app_put = [&](const u32x4_t& kc, const u32x4_t& vc) {
      if (lrow < 2) {
        uint8_t* dst = lrow ? app_v_cache : app_k_cache;
        *reinterpret_cast<u32x4_t*>(
            dst + ((size_t)app_slot * row_stride + kvh * D + lch * EPC) * EB) = lrow ? vc : kc;
      }
    };
    // the lane's chunk of the new K / V row in the cache's form: the 16-bit
    // values, or (int8 cache) their 16 codes under the kv head's scales, the
    // same codes the int8 write stores
    auto app_load = [&](u32x4_t& kc, u32x4_t& vc) {
      using S = typename Ty::storage;
      if constexpr (Q8) {
        const uint4 kq = quantize16<Ty>(static_cast<const S*>(new_k) + app_src, k_scale[kvh]);
        const uint4 vq = quantize16<Ty>(static_cast<const S*>(new_v) + app_src, v_scale[kvh]);
        kc = u32x4_t{kq.x, kq.y, kq.z, kq.w};
        vc = u32x4_t{vq.x, vq.y, vq.z, vq.w};
      } else {
        kc = *reinterpret_cast<const u32x4_t*>(static_cast<const S*>(new_k) + app_src);
        vc = *reinterpret_cast<const u32x4_t*>(static_cast<const S*>(new_v) + app_src);
      }
    };
    auto app_store = [&]() {   // the store when no tile of the workgroup holds the row
      if constexpr (APP) {
        if (app_writer) {
          u32x4_t kc, vc;
          app_load(kc, vc);
          app_put(kc, vc);
        }
      }
    };
    // visible keys [lo, ctx); loads start at lo16 (16-aligned: one block per load)
    const int lo = (EXT && window_left >= 0) ? max(0, ctx - 1 - window_left) : 0;
    const int lo16 = lo & ~15;
    if (part_start >= ctx) {
      if (pairing) plan();   // (an empty row is never cut; it may take a tail)
      app_store();   // an empty context: its new row is still stored
      if (pp == 0) {
        for (int i = tid; i < heads_per_wg * D; i += NT)
          out[((size_t)sb * num_q_heads + h0 + i / D) * D + i % D] = 0;
      }
      return;        // uniform over the workgroup
    }
    if (EXT && part_start + part_tokens <= lo16) return;   // no visible key: the reduce skips it
    int ntok = min(part_tokens, ctx - part_start);
    const int tb = EXT ? max(0, lo16 - part_start) : 0;    // first local token loaded
    const int nparts_b = (ctx + part_tokens - 1) / part_tokens;

    const int nblk = (ntok + bs - 1) >> log2_bs;
    if (tid < nblk) s_blk[tid] = (id_raw >= 0 && id_raw < num_blocks) ? id_raw : -1;
    // (blocks wholly before a window's first loaded token are never read)
    PKV_DBG_REPORT(tid < nblk && ((tid + 1) << log2_bs) > tb && !(id_raw >= 0 && id_raw < num_blocks),
                   kDbgBlockId);
    // APP: wave 0 takes the last tile (the one holding ctx-1) first and the
    // counter hands out the others, so only that first step differs
    if (tid == 0) s_claim = APP ? WAVES - 1 : WAVES;
    __syncthreads();

    // local token whose K/V come from new_k / new_v (-1: none)
    int app_pos = -1;
    if constexpr (APP) {
      const int last = ctx - 1 - part_start;
      if (last >= 0 && last < ntok && app_slot >= 0) {
        const int blk = s_blk[last >> log2_bs];
        if (blk >= 0 && (int64_t)blk * bs + (last & (bs - 1)) == (int64_t)app_slot) app_pos = last;
      }
      if (app_pos < 0) app_store();   // the slot given is not the slot of ctx-1
    }

    const int head_off = kvh * D + lch * EPC;
    const uint8_t* kbytes = static_cast<const uint8_t*>(k_cache);
    const uint8_t* vbytes = static_cast<const uint8_t*>(v_cache);
    const float sl2 = Q8 ? scale_log2 * k_scale[kvh] : scale_log2;   // scores in log2 units
    const float vsc = Q8 ? v_scale[kvh] : 1.f;
    // ALiBi slope of the lane's head, log2 units
    const float al2 = (EXT && alibi != nullptr && head_ok) ? alibi[h0 + l16] * 1.4426950408889634f
                                                           : 0.f;
    const int lo_local = lo - part_start;
    // Tiles g = 0 .. ntiles-1 cover local tokens [tb + g*TT, tb + (g+1)*TT).
    // Wave w starts on tile w and claims each further tile from a counter in
    // LDS as it issues that tile's loads. (With fixed equal shares the second
    // wave of each SIMD, which loses issue arbitration to the first, finished
    // several microseconds after it; on demand the waves end within about a
    // tile of each other.) A wave's set of tiles, and so the rounding of its
    // partial sums, varies from call to call.
    int ntiles = (ntok - tb + TT - 1) / TT;
    int last_grp = (ntok - 1) & ~(RPI - 1);

    uint8_t* s_k = s_mem + wave * L::waveB;
    uint8_t* s_v = s_k + L::tileB;

    // the next tile is fetched into registers while the current one is used
    u32x4_t kr[LPI], vr[LPI];
    auto fetch = [&](int g) {
#pragma unroll
      for (int j = 0; j < LPI; ++j) {
        const int t0 = tb + g * TT + j * RPI;               // first row of this load (uniform)
        const int tg = min(t0, last_grp);                    // groups past the end re-read the last
        const int tok = min(tg + lrow, ntok - 1);
        const int blk = max(__builtin_amdgcn_readfirstlane(s_blk[tg >> log2_bs]), 0);
        const size_t off = (((size_t)blk * bs + (tok & (bs - 1))) * row_stride + head_off) * EB;
        kr[j] = load16<true>(kbytes + off);
        vr[j] = load16<true>(vbytes + off);
      }
    };
    auto claim = [&]() {   // wave-uniform
      int g = 0;
      if (lane == 0) g = atomicAdd(&s_claim, 1);
      return __builtin_amdgcn_readfirstlane(g);
    };

    f32x4_t acc[ND];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[nd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // V^T operand: lane i of a 16-lane group points at token 4*g4 + i/4 (+16n),
    // dims 16nd + 4*(i%4) .. +4, and receives dim 16nd + i of tokens 4*g4 .. +4
    const uint8_t* vt = s_v + (4 * g4 + (l16 >> 2)) * L::rowB + (l16 & 3) * 8;

    auto tile = [&](int g) {
      f32x4_t st[NS];
#pragma unroll
      for (int n = 0; n < NS; ++n) {
        st[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const u32x4_t a =
              *reinterpret_cast<const u32x4_t*>(s_k + (16 * n + l16) * L::rowB + 64 * s + 16 * g4);
          st[n] = Mma<Ty>::mfma(a, qb[s], st[n]);
        }
      }
      // lane holds tokens 16n + 4*g4 + i of this tile for head l16
      const int tbase = tb + g * TT + 4 * g4;
      // distance of the lane's first token to the query (ALiBi)
      const float dj0 = (float)(part_start + tbase - (ctx - 1));
      float sv[NS][4];
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tbase + 16 * n + i;
          bool vis = t < ntok;
          float x = st[n][i] * sl2;
          if constexpr (EXT) {
            vis = vis && t >= lo_local;
            x = fmaf(al2, dj0 + (float)(16 * n + i), x);
          }
          sv[n][i] = vis ? x : -INFINITY;
          mx = fmaxf(mx, sv[n][i]);
        }
      mx = max_xor32(max_xor16(mx));
      const float mnew = fmaxf(m_run, mx);
      const float mref = safe_max_ref(mnew);
      const float alpha = fast_exp2(m_run - mref);
      m_run = mnew;
      float pv[NS][4];
      float psum = 0.f;
#pragma unroll
      for (int n = 0; n < NS; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[n][i] = fast_exp2(sv[n][i] - mref);
          psum += pv[n][i];
        }
      l_run = l_run * alpha + psum;
      if constexpr (NS == 1) {
        const u32x2_t pb = {Mma<Ty>::pack(pv[0][0], pv[0][1]), Mma<Ty>::pack(pv[0][2], pv[0][3])};
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const u32x2_t a = lds_read_tr16(vt + nd * 32);
          acc[nd] *= alpha;
          acc[nd] = Mma<Ty>::mfma16(a, pb, acc[nd]);
        }
      } else {
        const u32x4_t pb = {Mma<Ty>::pack(pv[0][0], pv[0][1]), Mma<Ty>::pack(pv[0][2], pv[0][3]),
                            Mma<Ty>::pack(pv[1][0], pv[1][1]), Mma<Ty>::pack(pv[1][2], pv[1][3])};
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const u32x2_t lo = lds_read_tr16(vt + nd * 32);
          const u32x2_t hi = lds_read_tr16(vt + 16 * L::rowB + nd * 32);
          const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
          acc[nd] *= alpha;
          acc[nd] = Mma<Ty>::mfma(a, pb, acc[nd]);
        }
      }
    };

    // park the fetched tile in the wave's LDS tile (int8 codes widened on the
    // way); later LDS reads of this wave see it
    auto park = [&]() {
#pragma unroll
      for (int j = 0; j < LPI; ++j) {
        uint8_t* dk = s_k + (j * RPI + lrow) * L::rowB + lch * 32 / EB;
        uint8_t* dv = s_v + (j * RPI + lrow) * L::rowB + lch * 32 / EB;
        if constexpr (Q8) {
          u32x4_t lo, hi;
          widen_i8x16<Ty>(kr[j], lo, hi);
          *reinterpret_cast<u32x4_t*>(dk) = lo;
          *reinterpret_cast<u32x4_t*>(dk + 16) = hi;
          widen_i8x16<Ty>(vr[j], lo, hi);
          *reinterpret_cast<u32x4_t*>(dv) = lo;
          *reinterpret_cast<u32x4_t*>(dv + 16) = hi;
        } else {
          *reinterpret_cast<u32x4_t*>(dk) = kr[j];
          *reinterpret_cast<u32x4_t*>(dv) = vr[j];
        }
      }
    };

    // applies a cut to item 0: it becomes the head piece of its row
    auto apply_cut = [&]() {
      pslot = 0;
      ntok = cut_own - part_start;
      ntiles = (ntok - tb + TT - 1) / TT;
      last_grp = (ntok - 1) & ~(RPI - 1);
      app_writer = false;   // the tail's workgroup stores the new row
      app_pos = -1;
    };
    // claimed tiles run over [0, nclaim); APP keeps the last one for wave 0
    int nclaim = APP ? ntiles - 1 : ntiles;
    int g = wave;
    u32x4_t app_k = {0u, 0u, 0u, 0u}, app_v = {0u, 0u, 0u, 0u};
    if constexpr (APP) {
      g = wave - 1;
      if (wave == 0 && ntiles > 0) {
        // the last tile, with the new row's K/V (fetched with it) in place of
        // the pool's row at ctx-1, whatever the pool held when it was read
        const int gl = ntiles - 1;
        fetch(gl);
        if (pairing) {
          plan();
          if (cut_own >= 0) apply_cut();   // that tile is the partner's
        }
        if (app_pos >= 0) app_load(app_k, app_v);
        if (app_pos >= 0) {
#pragma unroll
          for (int j = 0; j < LPI; ++j) {
            const int tok = min(min(tb + gl * TT + j * RPI, last_grp) + lrow, ntok - 1);
            if (tok == app_pos) {
              kr[j] = app_k;
              vr[j] = app_v;
            }
          }
        }
        if (cut_own >= 0) {
          nclaim = ntiles;
          g = claim();
          if (g < nclaim) fetch(g);
        } else {
          park();
          g = claim();
          if (g < nclaim) fetch(g);
          tile(gl);
        }
      } else {
        if (g < nclaim) fetch(g);
        if (pairing) {
          plan();
          if (cut_own >= 0) {
            apply_cut();
            nclaim = ntiles;
          }
        }
      }
    } else {
      if (g < ntiles) fetch(g);
      if (pairing) {
        plan();
        if (cut_own >= 0) {
          apply_cut();
          nclaim = ntiles;
        }
      }
    }
    while (g < nclaim) {
      park();
      const int gn = claim();
      if (gn < nclaim) fetch(gn);
      tile(g);
      g = gn;
    }
    // APP: the writer stores the new row once its walk is done. Stored right
    // after the first tile instead, with every workgroup's stream in flight,
    // the LLaMA-7B-shaped step took 1 us longer (47.95 against 46.95 us).
    if constexpr (APP) {
      if (wave == 0 && ntiles > 0 && app_pos >= 0 && app_writer) app_put(app_k, app_v);
    }

    // ---- merge lanes (the 4 lane groups) and waves ----
    l_run = sum_xor32(sum_xor16(l_run));
    __syncthreads();  // every wave is done with its K/V tiles
    float* s_ml = reinterpret_cast<float*>(s_mem);                 // [wave][16][2]
    float* s_o = s_ml + WAVES * 16 * 2;                            // [wave][16][oRow]
    // only lanes of real heads write; each writes its 4 consecutive dims at once
    if (head_ok) {
      if (g4 == 0) {
        s_ml[(wave * 16 + l16) * 2 + 0] = m_run;
        s_ml[(wave * 16 + l16) * 2 + 1] = l_run;
      }
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
        *reinterpret_cast<f32x4_t*>(s_o + (wave * 16 + l16) * L::oRow + 16 * nd + 4 * g4) = acc[nd];
    }
    __syncthreads();

    for (int idx = tid; idx < heads_per_wg * D; idx += NT) {
      const int hh = idx / D, d = idx % D;
      float mm = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) mm = fmaxf(mm, s_ml[(w * 16 + hh) * 2]);
      const float mr = safe_max_ref(mm);
      float ll = 0.f, a = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float wt = fast_exp2(s_ml[(w * 16 + hh) * 2] - mr);
        ll += s_ml[(w * 16 + hh) * 2 + 1] * wt;
        a += s_o[(w * 16 + hh) * L::oRow + d] * wt;
      }
      const size_t bh = (size_t)sb * num_q_heads + h0 + hh;
      a *= vsc;
      if (pslot >= 0) {   // a piece of a paired row: slots [bh, 2], device-coherent
        __hip_atomic_store(ws_o + (bh * 2 + pslot) * D + d, a, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(ws_ml + (bh * 2 + pslot) * 2 + 0, mm, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(ws_ml + (bh * 2 + pslot) * 2 + 1, ll, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      } else if (nparts_b == 1) {
        out[bh * D + d] = from_f32<Ty>(ll > 0.f ? a / ll : 0.f);
      } else {
        ws_o[(bh * num_parts + pp) * D + d] = a;
        if (d == 0) {
          ws_ml[(bh * num_parts + pp) * 2 + 0] = mm;
          ws_ml[(bh * num_parts + pp) * 2 + 1] = ll;
        }
      }
    }

    if (pslot >= 0) {
      // Hand-over between the two workgroups of a paired row. Each writes its
      // triple with device-coherent stores (through its XCD's own L2 to
      // memory) and waits until they are done; then one thread swaps the
      // call's epoch into the row's word. The workgroup that finds the epoch
      // already there is second: its device-coherent loads then see the
      // other triple, it merges, and it clears the word (so a replay with
      // the same epoch starts clean). Only the word and the triples cross
      // workgroups, all through device-scope atomics: no cache-wide
      // write-back or invalidation.
      unsigned long long* word = pair_words + (size_t)sb * num_q_heads + h0;
      wait_vmcnt<0>();
      __syncthreads();
      if (tid == 0) {
        const unsigned long long prev =
            __hip_atomic_exchange(word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_claim = prev == epoch ? 1 : 0;
      }
      __syncthreads();
      if (s_claim != 0) {
        auto ld = [](const float* x) {
          return __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        for (int idx = tid; idx < heads_per_wg * D; idx += NT) {
          const int hh = idx / D, d = idx % D;
          const size_t bh = (size_t)sb * num_q_heads + h0 + hh;
          const float m0 = ld(ws_ml + bh * 4 + 0), l0 = ld(ws_ml + bh * 4 + 1);
          const float m1 = ld(ws_ml + bh * 4 + 2), l1 = ld(ws_ml + bh * 4 + 3);
          const float mr = safe_max_ref(fmaxf(m0, m1));
          const float w0 = fast_exp2(m0 - mr), w1 = fast_exp2(m1 - mr);
          const float ll = l0 * w0 + l1 * w1;
          const float a = ld(ws_o + (bh * 2) * D + d) * w0 + ld(ws_o + (bh * 2 + 1) * D + d) * w1;
          out[bh * D + d] = from_f32<Ty>(ll > 0.f ? a / ll : 0.f);
        }
        if (tid == 0) __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  run_item(item_kind<false>{});
  if (tail_seq >= 0) {   // uniform over the workgroup
    __syncthreads();     // the LDS is reused by the tail
    run_item(item_kind<true>{});
  }
}

// ---------------------------------------------------------------------------
// Exact merge of the partition triples of one (sequence, query head):
//   M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p 2^(m_p - M) / L.
// 4 waves split the partitions; each lane owns D/64 output elements.
// ---------------------------------------------------------------------------
template <class Ty, int D>
__global__ __launch_bounds__(kDecThreads) void decode_reduce_kernel(
    typename Ty::storage* __restrict__ out, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens, int num_q_heads,
    int log2_bs, int max_blocks_per_seq, int num_parts, int part_tokens, int window_left) {
  constexpr int EPL = D / kWave;
  __shared__ float s_red[kDecWaves];
  __shared__ float s_acc[kDecWaves][D + 1];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int ctx = context_lens[b];
  ctx = max(0, min(ctx, max_blocks_per_seq << log2_bs));
  const int np = (ctx + part_tokens - 1) / part_tokens;
  if (np <= 1) return;
  // with a window, partitions wholly below it wrote nothing (same rule as the
  // partition kernel)
  const int p_lo =
      window_left >= 0 ? ((max(0, ctx - 1 - window_left) & ~15) / part_tokens) : 0;
  const size_t bh = (size_t)b * num_q_heads + h;
  const float* ml = ws_ml + bh * num_parts * 2;
  const float* o = ws_o + bh * num_parts * D;

  float mm = -INFINITY;
  for (int p = p_lo + tid; p < np; p += kDecThreads) mm = fmaxf(mm, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, kWave));
  if (lane == 0) s_red[wave] = mm;
  __syncthreads();
  mm = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float mr = safe_max_ref(mm);

  float a[EPL], ll = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = 0.f;
  int p = p_lo + wave;
  for (; p + 3 * kDecWaves < np; p += 4 * kDecWaves) {
    float w4[4], v4[4][EPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pp = p + u * kDecWaves;
      w4[u] = fast_exp2(ml[2 * pp] - mr);
      ll += ml[2 * pp + 1] * w4[u];
#pragma unroll
      for (int e = 0; e < EPL; ++e) v4[u][e] = o[(size_t)pp * D + lane * EPL + e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e) a[e] += v4[u][e] * w4[u];
  }
  for (; p < np; p += kDecWaves) {
    const float wt = fast_exp2(ml[2 * p] - mr);
    ll += ml[2 * p + 1] * wt;
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] += o[(size_t)p * D + lane * EPL + e] * wt;
  }
  __syncthreads();
  if (lane == 0) s_red[wave] = ll;
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][lane * EPL + e] = a[e];
  __syncthreads();
  if (tid < D) {
    const float lt = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    const float at = s_acc[0][tid] + s_acc[1][tid] + s_acc[2][tid] + s_acc[3][tid];
    out[bh * D + tid] = from_f32<Ty>(lt > 0.f ? at / lt : 0.f);
  }
}

template <class Ty, int D>
static hipError_t launch_reduce(const DecodeArgs& a, hipStream_t stream, int log2_bs,
                                int num_parts, int part_tokens) {
  using S = typename Ty::storage;
  launch_kernel((decode_reduce_kernel<Ty, D>), dim3(a.num_q_heads, a.num_seqs),
                     dim3(kDecThreads), 0, stream, static_cast<S*>(a.out), a.ws_ml, a.ws_o,
                     a.context_lens, a.num_q_heads, log2_bs, a.max_blocks_per_seq, num_parts,
                     part_tokens, a.window_left);
  return hipGetLastError();
}

template <class Ty, int D, int G>
static hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t stream) {
  using S = typename Ty::storage;
  const int log2_bs = __builtin_ctz(a.block_size);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int parts = decode_parts(a.max_blocks_per_seq, a.block_size, kDecodePart);
  dim3 grid(parts, a.num_q_heads / G, a.num_seqs);
  launch_kernel((decode_partition_kernel<Ty, D, G>), grid, dim3(kDecThreads), 0, stream,
                     static_cast<S*>(a.out), static_cast<const S*>(a.q),
                     static_cast<const S*>(a.k_cache), static_cast<const S*>(a.v_cache),
                     a.block_table, a.context_lens, a.ws_ml, a.ws_o, scale_log2, a.num_q_heads,
                     a.num_kv_heads, group, log2_bs, a.max_blocks_per_seq, a.num_blocks, parts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || parts <= 1) return err;
  return launch_reduce<Ty, D>(a, stream, log2_bs, parts, kDecodePart);
}

template <class Ty, int D, int WAVES, int TT, bool Q8, bool EXT, bool APP>
static hipError_t launch_mfma_cfg(const DecodeArgs& a, hipStream_t stream, int hpw,
                                  int part_tokens) {
  const int log2_bs = __builtin_ctz(a.block_size);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int parts = decode_parts(a.max_blocks_per_seq, a.block_size, part_tokens);
  dim3 grid(parts, a.num_q_heads / hpw, a.num_seqs);
  // pairing: whole contexts (one partition), a batch one wave can rank, and
  // the two slots per head the workspace holds
  const bool pair = !EXT && WAVES == 8 && parts == 1 && a.pair_words != nullptr &&
                    a.num_seqs >= 2 && a.num_seqs <= kWave;
  // the kernel forms the linear slot index in 32 bits
  const bool slots_fit = (long long)parts * grid.y * grid.z < (1LL << 31);
  const int xcd_bit = slots_fit ? decode_xcd_bit(a.num_kv_heads, group / hpw, D * (Q8 ? 1 : 2),
                                                 a.k_cache, a.v_cache)
                                : -1;
  launch_kernel((decode_mfma_kernel<Ty, D, WAVES, TT, Q8, EXT, APP>), grid, dim3(WAVES * kWave), 0,
                     stream, static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     a.k_cache, a.v_cache, a.block_table, a.context_lens, a.ws_ml, a.ws_o,
                     scale_log2, a.num_q_heads, a.num_kv_heads, group, hpw, log2_bs,
                     a.max_blocks_per_seq, a.num_blocks, parts, part_tokens, a.k_scale,
                     a.v_scale, a.alibi, a.window_left, static_cast<uint8_t*>(a.app_k_cache),
                     static_cast<uint8_t*>(a.app_v_cache), a.new_key, a.new_value,
                     a.slot_mapping, xcd_bit, pair ? a.pair_words : nullptr, a.epoch,
                     a.num_seqs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || parts <= 1) return err;
  return launch_reduce<Ty, D>(a, stream, log2_bs, parts, part_tokens);
}

template <class Ty, int D, bool Q8 = false, bool EXT = false, bool APP = false>
static hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  int hpw = 1;  // largest divisor of the group size that fits one 16-row tile
  for (int c = 16; c >= 1; --c)
    if (group % c == 0) { hpw = c; break; }
  const DecodePlan plan = plan_decode(a.num_seqs, a.num_q_heads / hpw, a.max_blocks_per_seq,
                                      a.block_size,
                                      decode_fine_ok(a.num_seqs, a.num_q_heads,
                                                     a.max_blocks_per_seq, a.block_size));
  if (plan.waves == 8)
    return launch_mfma_cfg<Ty, D, 8, 32, Q8, EXT, APP>(a, stream, hpw, plan.part_tokens);
  return launch_mfma_cfg<Ty, D, 4, 16, Q8, EXT, APP>(a, stream, hpw, plan.part_tokens);
}

template <int D>
static hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g % 8 == 0) return launch_decode_valu<F32, D, 8>(a, stream);
  if (g % 4 == 0) return launch_decode_valu<F32, D, 4>(a, stream);
  if (g % 2 == 0) return launch_decode_valu<F32, D, 2>(a, stream);
  return launch_decode_valu<F32, D, 1>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_dim == 64;
  switch (a.dtype) {
    case 0: return d64 ? launch_decode_f32<64>(a, stream) : launch_decode_f32<128>(a, stream);
    case 1: return d64 ? launch_decode_mfma<F16, 64>(a, stream)
                       : launch_decode_mfma<F16, 128>(a, stream);
    default: return d64 ? launch_decode_mfma<BF16, 64>(a, stream)
                        : launch_decode_mfma<BF16, 128>(a, stream);
  }
}

hipError_t launch_decode_ext(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_dim == 64;
  if (a.dtype == 1)
    return d64 ? launch_decode_mfma<F16, 64, false, true>(a, stream)
               : launch_decode_mfma<F16, 128, false, true>(a, stream);
  return d64 ? launch_decode_mfma<BF16, 64, false, true>(a, stream)
             : launch_decode_mfma<BF16, 128, false, true>(a, stream);
}

hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_dim == 64;
  if (a.dtype == 1)
    return d64 ? launch_decode_mfma<F16, 64, true>(a, stream)
               : launch_decode_mfma<F16, 128, true>(a, stream);
  return d64 ? launch_decode_mfma<BF16, 64, true>(a, stream)
             : launch_decode_mfma<BF16, 128, true>(a, stream);
}

hipError_t launch_write_decode_int8(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_dim == 64;
  if (a.dtype == 1)
    return d64 ? launch_decode_mfma<F16, 64, true, false, true>(a, stream)
               : launch_decode_mfma<F16, 128, true, false, true>(a, stream);
  return d64 ? launch_decode_mfma<BF16, 64, true, false, true>(a, stream)
             : launch_decode_mfma<BF16, 128, true, false, true>(a, stream);
}

hipError_t launch_write_decode(const DecodeArgs& a, hipStream_t stream) {
  const bool d64 = a.head_dim == 64;
  switch (a.dtype) {
    case 0: {   // fp32 pool: the vector-ALU decode has no fused form; write, then decode
      hipError_t err = launch_kv_write(a.app_k_cache, a.app_v_cache, a.new_key, a.new_value,
                                       a.slot_mapping, a.num_seqs,
                                       a.num_kv_heads * a.head_dim * 4,
                                       a.num_blocks * a.block_size, stream);
      return err != hipSuccess ? err : launch_decode(a, stream);
    }
    case 1: return d64 ? launch_decode_mfma<F16, 64, false, false, true>(a, stream)
                       : launch_decode_mfma<F16, 128, false, false, true>(a, stream);
    default: return d64 ? launch_decode_mfma<BF16, 64, false, false, true>(a, stream)
                        : launch_decode_mfma<BF16, 128, false, false, true>(a, stream);
  }
}

PKV_DBG_TAKE_FN(debug_take_decode)

}  // namespace pkv
