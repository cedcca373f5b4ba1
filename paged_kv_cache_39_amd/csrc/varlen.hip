// Packed variable-length prefill attention over the paged KV cache, on the
// gfx950 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation).
//
// Definition: sequence b owns query rows [cu[b], cu[b+1]) and keys 0..Lk-1
// read through its block_table row; with the causal flag, local query i sees
// keys j <= i + Lk - Lq ("Paged KV infra" page, section 3.1: each packed
// sequence gets its own causal mask over its own length, no padding; the
// skill page's Appendix C uses the causal mode for prefill). Scale 1/sqrt(D).
//
// Work split: one workgroup (4 waves) per (query tile, kv head). The tile's
// 128 "rows" are (query position, query head of the kv group) pairs, so a
// K/V tile fetched once through the block table serves every query head of
// the group (GQA batching). Each wave owns 32 rows.
//
// Orientation: the kernel computes S^T = K Q^T (K from LDS as the A operand,
// Q held in registers as the B operand) and O^T = V^T P^T (V^T from LDS as
// the A operand). With the 16x16 output layout (lane l holds column l%16),
// every lane then owns whole rows of S^T, of P and of O^T: the online-softmax
// statistics, the bf16/fp16 P operand and the O rescale all stay in the
// lane's registers, with only two cross-lane exchanges per row for the max.
// V is transposed once while it is staged into LDS.

#include "debug_checks.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kVlWaves = 4;
// compile-time stage index of the prefill key loop
template <int V>
struct stage_tag {
  static constexpr int value = V;
};
constexpr int kVlThreads = kVlWaves * kWave;

// K / V tiles live in LDS unpadded (D*2-byte rows) and XOR-swizzled in
// 16-byte slots: slot s of row r holds chunk s ^ f(r). The functions were
// chosen with the LDS bank-conflict counter on gfx950 (a conflict-free
// 16-byte read of a wave takes 4 LDS cycles, an 8-byte transpose read 2):
//   K operand reads (ds_read_b128, 16 rows x one chunk): f(r) = r mod spr;
//   V^T transpose reads (ds_read_b64_tr_b16, 4 rows x 2 adjacent chunks per
//   16 lanes): f(r) = r mod 8 at D = 64, and at D = 128 a one-bit rotation
//   of r mod 16 (plain r mod 16 conflicts 2-way there, as the rotation does
//   for the K reads).
template <int D>
struct VlLds {
  static constexpr int rowB = D * 2;
  static constexpr int spr = D / 8;                  // 16-byte slots per row
  static constexpr int tileB = kVlBN * rowB;         // one K or V tile
  static constexpr int stageB = 2 * tileB;           // K and V
  static __device__ __forceinline__ int fk(int r) { return r & (spr - 1); }
  static __device__ __forceinline__ int fv(int r) {
    const int x = r & (spr - 1);
    return spr == 16 ? (((x << 1) | (x >> 3)) & 15) : x;
  }
  static __device__ __forceinline__ int slot_k(int r, int chunk) { return chunk ^ fk(r); }
  static __device__ __forceinline__ int slot_v(int r, int chunk) { return chunk ^ fv(r); }
};

// Narrow sequences of the plain packed call: when all of a sequence's query
// rows fit one 16-row matrix-core tile (Lq x group <= 16: decode rows,
// multi-token decode), a 128-row query tile would leave most rows empty and
// keep one 64-key K/V stage in flight, which bounds a long row's stream (a
// decode row over 4096 keys took ~1.45 us per 64 keys). Such a sequence is
// taken per kv head the way the decode kernel takes a context: each wave
// walks its own 32-key tiles (wave w: tiles w, w + 4, ...), fetched into
// registers one tile ahead and parked in the wave's own padded LDS slice (no
// barrier in the loop, four tiles streaming at once), with its own online
// softmax over the 16 rows; the four partial states merge at the end. Row r
// of the tile (lane r mod 16) is query r / group, head r mod group of the kv
// head; query i sees keys j <= i + Lk - Lq under the causal mask.
template <int D>
struct VlNarrowLds {
  static constexpr int TT = 32;                      // keys per wave tile
  static constexpr int rowB = D * 2 + 16;            // padded row pitch (bytes)
  static constexpr int tileB = TT * rowB;            // one K or V tile
  static constexpr int waveB = 2 * tileB;
  static constexpr int tilesB = kVlWaves * waveB;
  static constexpr int oRow = D + 4;                 // merge row pitch (floats)
  static constexpr int mergeB = kVlWaves * 16 * (2 + oRow) * 4;
  static constexpr int bytes = tilesB > mergeB ? tilesB : mergeB;
};
// the most query rows a narrow sequence has
constexpr int kVlNarrowRows = 16;

template <class Ty, int D>
__device__ __forceinline__ void varlen_narrow(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint8_t* __restrict__ kbytes, const uint8_t* __restrict__ vbytes,
    const int32_t* __restrict__ bt_row, int r0, int lq, int lk, int kv_lo, int kv_hi, int causal,
    int num_q_heads, int kvh, int group, int log2_bs, uint32_t nblocks32, uint32_t row_bytes,
    float scale_log2, float* __restrict__ ws_ml, float* __restrict__ ws_o, int64_t ws_row0,
    uint8_t* lds, int tid, int wave, int lane) {
  using N = VlNarrowLds<D>;
  constexpr int TT = N::TT;
  constexpr int CPR = D / 8;          // 16-byte chunks per K/V row of one kv head
  constexpr int RPI = kWave / CPR;    // rows per load instruction
  constexpr int LPI = TT / RPI;       // load instructions per tile and matrix
  constexpr int KS = D / 32;          // k-steps of q.k
  constexpr int ND = D / 16;          // 16-dim tiles of the output
  const int l16 = lane & 15, g4 = lane >> 4;
  const int lrow = lane / CPR, lch = lane % CPR;
  const int bs = 1 << log2_bs;
  // the lane's row of the tile and its last visible key in [kv_lo, kv_hi)
  // (below kv_lo: none)
  const int qi = l16 / group;
  const bool row_ok = qi < lq;
  const int head = kvh * group + (l16 - qi * group);
  const int lim = row_ok ? (causal ? min(kv_hi - 1, qi + lk - lq) : kv_hi - 1) : kv_lo - 1;

  // queries as the B operand: lane holds row l16, dims 32s + 8*g4 .. +8
  u32x4_t qb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qb[s] = row_ok ? load16<false>(q + ((size_t)(r0 + qi) * num_q_heads + head) * D + 32 * s +
                                   8 * g4)
                   : u32x4_t{0u, 0u, 0u, 0u};

  uint8_t* s_k = lds + wave * N::waveB;
  uint8_t* s_v = s_k + N::tileB;
  const int ntiles = (kv_hi - kv_lo + TT - 1) / TT;
  const uint32_t head_off = (uint32_t)(kvh * D + lch * 8) * 2u;
  // Block ids of the lane's keys in a tile (keys past the range re-read its
  // last key: finite values, masked); the next tile's are requested with the
  // current tile's K/V, so the fetch never waits on a table lookup.
  int ids[LPI];
  auto load_ids = [&](int g) {
#pragma unroll
    for (int j = 0; j < LPI; ++j)
      ids[j] = bt_row[min(kv_lo + g * TT + j * RPI + lrow, kv_hi - 1) >> log2_bs];
  };
  u32x4_t kr[LPI], vr[LPI];
  auto fetch = [&](int g) {
#pragma unroll
    for (int j = 0; j < LPI; ++j) {
      const int t = min(kv_lo + g * TT + j * RPI + lrow, kv_hi - 1);
      PKV_DBG_REPORT((uint32_t)ids[j] >= nblocks32, kDbgBlockId);
      const uint32_t blk = (uint32_t)ids[j] < nblocks32 ? (uint32_t)ids[j] : 0u;
      const size_t off = ((size_t)blk * bs + (t & (bs - 1))) * row_bytes + head_off;
      kr[j] = load16<true>(kbytes + off);
      vr[j] = load16<true>(vbytes + off);
    }
  };
  auto park = [&]() {
#pragma unroll
    for (int j = 0; j < LPI; ++j) {
      *reinterpret_cast<u32x4_t*>(s_k + (j * RPI + lrow) * N::rowB + lch * 16) = kr[j];
      *reinterpret_cast<u32x4_t*>(s_v + (j * RPI + lrow) * N::rowB + lch * 16) = vr[j];
    }
  };

  f32x4_t acc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) acc[nd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // V^T operand: lane i of a 16-lane group reads key 4*g4 + i/4 (+16),
  // dims 16nd + 4*(i%4) .. +4, and receives dim 16nd + i of keys 4*g4 .. +4
  const uint8_t* vt = s_v + (4 * g4 + (l16 >> 2)) * N::rowB + (l16 & 3) * 8;
  auto tile = [&](int g) {
    f32x4_t st[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      st[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(s_k + (16 * n + l16) * N::rowB + 64 * s + 16 * g4);
        st[n] = Mma<Ty>::mfma(a, qb[s], st[n]);
      }
    }
    // lane holds keys kv_lo + g*TT + 16n + 4*g4 + i of its row
    const int tbase = kv_lo + g * TT + 4 * g4;
    float sv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[n][i] = tbase + 16 * n + i <= lim ? st[n][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[n][i]);
      }
    mx = max_xor32(max_xor16(mx));
    const float mnew = fmaxf(m_run, mx);
    const float mref = safe_max_ref(mnew);
    const float alpha = fast_exp2(m_run - mref);
    m_run = mnew;
    float pv[2][4];
    float psum = 0.f;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[n][i] = fast_exp2(sv[n][i] - mref);
        psum += pv[n][i];
      }
    l_run = l_run * alpha + psum;
    const u32x4_t pb = {Mma<Ty>::pack(pv[0][0], pv[0][1]), Mma<Ty>::pack(pv[0][2], pv[0][3]),
                        Mma<Ty>::pack(pv[1][0], pv[1][1]), Mma<Ty>::pack(pv[1][2], pv[1][3])};
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const u32x2_t lo = lds_read_tr16(vt + nd * 32);
      const u32x2_t hi = lds_read_tr16(vt + 16 * N::rowB + nd * 32);
      const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
      acc[nd] *= alpha;
      acc[nd] = Mma<Ty>::mfma(a, pb, acc[nd]);
    }
  };

  int g = wave;
  if (g < ntiles) {
    load_ids(g);
    fetch(g);
    if (g + kVlWaves < ntiles) load_ids(g + kVlWaves);
  }
  while (g < ntiles) {
    park();
    const int gn = g + kVlWaves;
    if (gn < ntiles) {
      fetch(gn);
      if (gn + kVlWaves < ntiles) load_ids(gn + kVlWaves);
    }
    tile(g);
    g = gn;
  }

  // ---- merge the lane groups, then the waves ----
  l_run = sum_xor32(sum_xor16(l_run));
  __syncthreads();   // every wave is done with its tiles
  float* s_ml = reinterpret_cast<float*>(lds);         // [wave][16][2]
  float* s_o = s_ml + kVlWaves * 16 * 2;                // [wave][16][oRow]
  if (g4 == 0) {
    s_ml[(wave * 16 + l16) * 2 + 0] = m_run;
    s_ml[(wave * 16 + l16) * 2 + 1] = l_run;
  }
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
    *reinterpret_cast<f32x4_t*>(s_o + (wave * 16 + l16) * N::oRow + 16 * nd + 4 * g4) = acc[nd];
  __syncthreads();
  // a thread merges 8 consecutive dims of a row: one 16-byte store of the
  // output (two of the fp32 chunk output)
  constexpr int TPR = D / 8;   // threads per row
  const int rows = lq * group;
  for (int idx = tid; idx < rows * TPR; idx += kVlThreads) {
    const int r = idx / TPR, d0 = (idx - r * TPR) * 8;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVlWaves; ++w) mm = fmaxf(mm, s_ml[(w * 16 + r) * 2]);
    const float mr = safe_max_ref(mm);
    float ll = 0.f;
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kVlWaves; ++w) {
      const float wt = fast_exp2(s_ml[(w * 16 + r) * 2] - mr);
      ll += s_ml[(w * 16 + r) * 2 + 1] * wt;
      const float* so = s_o + (w * 16 + r) * N::oRow + d0;
      a0 += *reinterpret_cast<const f32x4_t*>(so) * wt;
      a1 += *reinterpret_cast<const f32x4_t*>(so + 4) * wt;
    }
    if (ws_row0 >= 0) {
      // a chunk of a cut sequence: (max, sum, output) relative to 2^max for
      // the merge kernel, row r at slot ws_row0 + r
      const int64_t slot_i = ws_row0 + r;
      *reinterpret_cast<f32x4_t*>(ws_o + slot_i * D + d0) = a0;
      *reinterpret_cast<f32x4_t*>(ws_o + slot_i * D + d0 + 4) = a1;
      if (d0 == 0) {
        ws_ml[slot_i * 2 + 0] = mm;
        ws_ml[slot_i * 2 + 1] = ll;
      }
    } else {
      const int i = r / group;
      const float inv = ll > 0.f ? 1.f / ll : 0.f;
      *reinterpret_cast<u32x4_t*>(out + ((size_t)(r0 + i) * num_q_heads + kvh * group +
                                         (r - i * group)) * D + d0) =
          u32x4_t{Mma<Ty>::pack(a0[0] * inv, a0[1] * inv), Mma<Ty>::pack(a0[2] * inv, a0[3] * inv),
                  Mma<Ty>::pack(a1[0] * inv, a1[1] * inv), Mma<Ty>::pack(a1[2] * inv, a1[3] * inv)};
    }
  }
}

// Query-tile count of sequence s (0 past the end).
__device__ __forceinline__ int seq_tiles(const int32_t* __restrict__ cu, int num_seqs, int bq,
                                         int total_q, int s) {
  if (s >= num_seqs) return 0;
  const int lq = min(cu[s + 1], total_q) - max(0, min(cu[s], total_q));
  return lq > 0 ? (lq + bq - 1) / bq : 0;
}

// sum_b min(nt_b, cap) over the batch (cap < 0: no cap). `nt0` holds the
// count of sequence `lane` (the first 64 sequences, read once); further
// sequences are read from memory.
__device__ __forceinline__ int tiles_below(const int32_t* __restrict__ cu, int num_seqs, int bq,
                                           int total_q, int cap, int lane, int nt0) {
  int sum = cap < 0 ? nt0 : min(nt0, cap);
  for (int s0 = kWave; s0 < num_seqs; s0 += kWave) {
    const int nt = seq_tiles(cu, num_seqs, bq, total_q, s0 + lane);
    sum += cap < 0 ? nt : min(nt, cap);
  }
  return wave_sum_i(sum);
}

// Locate query tile `t` of one kv head (tiles of `bq` query positions).
// Tiles are handed out by rank from the end of their sequence: first the
// last tile of every sequence, then every second-to-last tile, and so on.
// Under the causal mask a sequence's later tiles see more keys, so the
// heaviest work is dispatched first and the short tiles fill the tail.
// One wave runs this; returns false when t is past the last tile.
// `nt0` is the tile count of sequence `lane` (0 past the batch).
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ cu, int num_seqs, int bq,
                                          int total_q, int t, int lane, int nt0, int& seq,
                                          int& q0) {
  if (t >= tiles_below(cu, num_seqs, bq, total_q, -1, lane, nt0)) return false;
  // largest rank j with sum_b min(nt_b, j) <= t
  int lo = 0, hi = 1;
  for (int s0 = 0; s0 < num_seqs; s0 += kWave) {
    const int nt = s0 == 0 ? nt0 : seq_tiles(cu, num_seqs, bq, total_q, s0 + lane);
    hi = max(hi, wave_max_i(nt) + 1);
  }
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tiles_below(cu, num_seqs, bq, total_q, mid, lane, nt0) <= t) lo = mid;
    else hi = mid;
  }
  const int j = lo;
  int r = t - tiles_below(cu, num_seqs, bq, total_q, j, lane, nt0);  // r-th sequence with nt > j
  for (int s0 = 0; s0 < num_seqs; s0 += kWave) {
    const int nt = s0 == 0 ? nt0 : seq_tiles(cu, num_seqs, bq, total_q, s0 + lane);
    const unsigned long long has = __ballot(nt > j);
    const int cnt = __popcll(has);
    if (r < cnt) {
      unsigned long long m = has;   // position of the r-th set bit
      for (int k = 0; k < r; ++k) m &= m - 1;
      const int first = __builtin_ctzll(m);
      const int ntile = lane_value(nt, first);
      seq = s0 + first;
      q0 = (ntile - 1 - j) * bq;
      return true;
    }
    r -= cnt;
  }
  return false;
}

// x / bq for x >= 0: a shift when bq is a power of two (P2, bq_log2 >= 0:
// the usual group sizes), else a division. The lookup below is compiled
// once per case and picked by a uniform branch: with a select per use, the
// compiler runs the division's ~25 instructions beside the shift every time.
template <bool P2>
__device__ __forceinline__ int div_bq(int x, int bq, int bq_log2) {
  return P2 ? (x >> bq_log2) : x / bq;
}

// Key tiles (of kVlBN keys) that a query tile's loop runs over: up to its
// rows' highest visible key, i + Lk - Lq for the tile's last row i under the
// causal mask, else Lk. That bound grows with the tile's position, so the
// tiles of a sequence needing at least w key tiles form a suffix; this
// returns its length (nt, lq, lk: the sequence's query tiles, query and key
// counts).
template <bool P2>
__device__ __forceinline__ int tiles_with_work(int w, int nt, int lq, int lk, int bq, int bq_log2,
                                               int causal) {
  if (lq <= 0) return 0;
  if (w <= 0) return nt;
  const int kmin = (w - 1) * kVlBN;   // the loop end must exceed this
  if (lk <= kmin) return 0;
  if (!causal) return nt;
  const int x = kmin - (lk - lq);      // needs min((t + 1) * bq, lq) > x
  if (lq <= x) return 0;
  return x < 0 ? nt : nt - div_bq<P2>(x, bq, bq_log2);
}

// Locate query tile `g` of one kv head in longest-first order: tiles sorted
// by their key-tile count, most first (ties by sequence, then position), so
// the longest loops start first and the shortest fill the tail. A binary
// search over the count finds g's bucket; a scan over the sequences finds
// the tile in it. One wave runs this; returns false when g is past the last
// tile. (my_lq, my_lk): sequence `lane`'s counts (the first 64 sequences;
// further ones are read from memory).
template <bool P2>
__device__ __forceinline__ bool find_tile_lpt(const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ seq_lens,
                                              int num_seqs, int total_q, int max_lk, int bq,
                                              int bq_log2, int causal, int g, int lane, int my_lq,
                                              int my_lk, int narrow_q, int& seq, int& q0) {
  const int my_nt = my_lq > 0 ? div_bq<P2>(my_lq + bq - 1, bq, bq_log2) : 0;
  auto meta = [&](int s0, int& lq, int& lk, int& nt) {
    if (s0 == 0) {
      lq = my_lq;
      lk = my_lk;
      nt = my_nt;
      return;
    }
    const int s = s0 + lane;
    lq = 0;
    lk = 0;
    if (s < num_seqs) {
      const int r0 = max(0, min(cu[s], total_q));
      lq = max(0, min(cu[s + 1], total_q) - r0);
      if (lq <= narrow_q) lq = 0;   // taken by the narrow path
      lk = max(0, min(seq_lens[s], max_lk));
    }
    nt = lq > 0 ? div_bq<P2>(lq + bq - 1, bq, bq_log2) : 0;
  };
  auto count = [&](int w) {   // tiles needing at least w key tiles
    int c = tiles_with_work<P2>(w, my_nt, my_lq, my_lk, bq, bq_log2, causal);
    for (int s0 = kWave; s0 < num_seqs; s0 += kWave) {
      int lq, lk, nt;
      meta(s0, lq, lk, nt);
      c += tiles_with_work<P2>(w, nt, lq, lk, bq, bq_log2, causal);
    }
    return wave_sum_i(c);
  };
  // (no test of g against count(0): a g past the last tile ends the search
  // below with lo = 0 and is not found by the scan)
  int wmax = (my_lk + kVlBN - 1) / kVlBN;
  for (int s0 = kWave; s0 < num_seqs; s0 += kWave) {
    int lq, lk, nt;
    meta(s0, lq, lk, nt);
    wmax = max(wmax, (lk + kVlBN - 1) / kVlBN);
  }
  wmax = wave_max_i(wmax);
  // count(lo) > g >= count(hi) (for lo >= 1); c_hi = count(hi), which is 0
  // past the longest key loop
  int lo = 0, hi = wmax + 1, c_hi = 0;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    const int c = count(mid);
    if (c > g) {
      lo = mid;
    } else {
      hi = mid;
      c_hi = c;
    }
  }
  int r = g - c_hi;   // rank among the tiles needing exactly lo key tiles
  for (int s0 = 0; s0 < num_seqs; s0 += kWave) {
    int lq, lk, nt;
    meta(s0, lq, lk, nt);
    const int ge = tiles_with_work<P2>(lo, nt, lq, lk, bq, bq_log2, causal);
    const int c = ge - tiles_with_work<P2>(lo + 1, nt, lq, lk, bq, bq_log2, causal);
    const int incl = wave_incl_scan_i(c);
    const int total = lane_value(incl, kWave - 1);
    if (r < total) {
      const unsigned long long hit = __ballot(incl - c <= r && r < incl);
      const int L = __builtin_ctzll(hit);
      const int t = lane_value(nt, L) - lane_value(ge, L) + (r - lane_value(incl - c, L));
      seq = s0 + L;
      q0 = t * bq;
      return true;
    }
    r -= total;
  }
  return false;
}

// EXT: the attention variants -- a sliding window (keys j >= p - window_left
// for the query at p = i + Lk - Lq, window_left >= 0) and ALiBi (score +
// alibi[h] * (j - p)); alibi may be NULL and window_left negative.
// Chunks the split call cuts a query tile's key loop into: only a tile whose
// rows fit one wave is cut -- a sequence's last, partial tile, such as a
// decode row or the tail of a prefill -- into chunks of chunk_tiles key tiles
// (full tiles already spread over many workgroups). (q0, lq, lk): the tile's
// first query and the sequence's query and key counts.
__device__ __forceinline__ int split_chunks(int q0, int lq, int lk, int bq, int group, int causal,
                                            int chunk_tiles) {
  const int nq = min(bq, lq - q0);
  if (nq <= 0 || nq * group > kVlRowsWave) return 1;
  const int kv_end = causal ? min(lk, q0 + nq + lk - lq) : lk;
  const int w = kv_end > 0 ? (kv_end + kVlBN - 1) / kVlBN : 0;
  return max(1, (w + chunk_tiles - 1) / chunk_tiles);
}

// SPLIT: the first n_tiles workgroup slots of each kv head are the tiles in
// longest-first order with their chunk 0; after them num_seqs x
// (max_splits - 1) slots take chunks 1 .. max_splits-1 of each sequence's
// last tile (they exit when it is not cut that far): the heavy uncut tiles
// start first and the short chunks fill in. A workgroup of a cut tile leaves
// its rows' partial (max, sum, output) in its chunk's slot of the workspace
// for the merge kernel.
template <class Ty, int D, bool EXT, bool SPLIT>
__global__ __launch_bounds__(kVlThreads, 2) void varlen_prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ cu_seqlens_q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int causal, int num_seqs, int total_q, int num_q_heads,
    int num_kv_heads, int log2_bs, int max_blocks_per_seq, int64_t num_blocks, float scale_log2,
    const float* __restrict__ alibi, int window_left, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, int chunk_tiles, int max_splits, int n_tiles, int narrow_seqs) {
  using L = VlLds<D>;
  constexpr int KS = D / 32;                 // k-steps of the QK product
  constexpr int ND = D / 16;                 // 16-wide dim tiles of the output
  constexpr int RPI = kWave / L::spr;        // rows per direct-to-LDS load of one wave
  constexpr int LPT = kVlBN / (kVlWaves * RPI);  // such loads per thread per matrix
  // lazy rescale: the running max used for the exponentials only moves when
  // a row max exceeds it by more than 2^8 (P then stays <= 256)
  constexpr float kRescale = 8.f;
  // the plain call's narrow sequences (narrow_seqs > 0) reuse the stages
  constexpr bool NARROW = !EXT && !SPLIT;
  // (the split call's chunks of narrow sequences take the narrow path too)
  constexpr int kLdsB = !EXT && VlNarrowLds<D>::bytes > 2 * L::stageB ? VlNarrowLds<D>::bytes
                                                                        : 2 * L::stageB;
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[kLdsB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps derived addresses scalar
  const int l16 = lane & 15, g4 = lane >> 4;
  // Workgroups are dispatched in index order, round-robin over the 8 XCDs
  // (each with its own L2). Index = tile rank x Hkv + kv head: every kv
  // head's heaviest tiles start first, and when Hkv is a multiple of 8 each
  // XCD serves fixed kv heads, whose K/V then stay in its L2 (with fewer kv
  // heads, a head's tiles alternate over the XCDs).
  // The plain call puts one workgroup per (narrow sequence candidate, kv
  // head) first: indexes below narrow_seqs x Hkv (sequences that are not
  // narrow leave at once); the query tiles follow.
  const int kvh = blockIdx.x % num_kv_heads;
  const int slot = (int)(blockIdx.x / num_kv_heads) - (NARROW ? narrow_seqs : 0);
  const bool extra = SPLIT && slot >= n_tiles;
  const int tile = slot;
  const int chunk = extra ? 1 + (slot - n_tiles) % (max_splits - 1) : 0;
  const int xseq = extra ? (slot - n_tiles) / (max_splits - 1) : 0;
  const int group = num_q_heads / num_kv_heads;
  const int bq = kVlRows / group;   // query positions per tile
  const int bq_log2 = (bq & (bq - 1)) == 0 ? __builtin_ctz(bq) : -1;
  const int bs = 1 << log2_bs;
  if constexpr (kDbgBuild) {   // the batch's metadata, checked once (workgroup 0)
    if (blockIdx.x == 0 && tid < kWave) {
      for (int s = lane; s < num_seqs; s += kWave) {
        const int c0 = cu_seqlens_q[s], c1 = cu_seqlens_q[s + 1], kl = seq_lens[s];
        PKV_DBG_REPORT(c0 < 0 || c1 < c0 || c1 > total_q || (s == 0 && c0 != 0) ||
                           (s == num_seqs - 1 && c1 != total_q),
                       kDbgCuSeqlens);
        PKV_DBG_REPORT(kl < 0 || kl > (max_blocks_per_seq << log2_bs), kDbgLength);
      }
    }
  }
  // rows of a sequence the narrow path takes (0: none); the tile lookup
  // below skips those sequences
  const int narrow_q = NARROW && narrow_seqs > 0 ? kVlNarrowRows / group : 0;   // queries
  if constexpr (NARROW) {
    if (slot < 0) {   // uniform: a (sequence, kv head) of the narrow path
      const int b = (int)(blockIdx.x / num_kv_heads);
      const int r0 = max(0, min(cu_seqlens_q[b], total_q));
      const int lq = max(0, min(cu_seqlens_q[b + 1], total_q) - r0);
      const int lk = max(0, min(seq_lens[b], max_blocks_per_seq << log2_bs));
      if (lq == 0 || lq > narrow_q) return;
      varlen_narrow<Ty, D>(out, q, reinterpret_cast<const uint8_t*>(k_cache),
                           reinterpret_cast<const uint8_t*>(v_cache),
                           block_table + (size_t)b * max_blocks_per_seq, r0, lq, lk, 0, lk,
                           causal, num_q_heads, kvh, group, log2_bs, (uint32_t)num_blocks,
                           (uint32_t)(num_kv_heads * D) * 2u, scale_log2, nullptr, nullptr, -1,
                           s_kv, tid, wave, lane);
      return;
    }
  }

  // Every wave locates the tile (same inputs, same result: no LDS hand-off
  // and no barrier). Lane s first reads sequence s's metadata (first row,
  // Lq, Lk) in one round trip; the tile's sequence then takes its metadata
  // from that lane.
  int tl[5];
  {
    int my_r0 = 0, my_lq = 0, my_lk = 0;
    if (lane < num_seqs) {
      my_r0 = max(0, min(cu_seqlens_q[lane], total_q));
      my_lq = max(0, min(cu_seqlens_q[lane + 1], total_q) - my_r0);
      if (my_lq <= narrow_q) my_lq = 0;   // taken by the narrow path
      my_lk = max(0, min(seq_lens[lane], max_blocks_per_seq << log2_bs));
    }
    // tile count of sequence `lane` (the windowed and split lookups only)
    auto lane_tiles = [&]() { return my_lq > 0 ? (my_lq + bq - 1) / bq : 0; };
    int seq = -1, q0 = 0, r0 = 0, lq_ = 0, lk_ = 0;
    // longest-first order; under a window a tile's key count is not
    // monotone in its position, so those tiles go by rank from the end
    bool found;
    if (SPLIT && extra) {   // the last tile of sequence xseq
      const int ntx = xseq < kWave ? lane_value(lane_tiles(), xseq)
                                   : seq_tiles(cu_seqlens_q, num_seqs, bq, total_q, xseq);
      found = ntx > 0;
      seq = xseq;
      q0 = (ntx - 1) * bq;
    } else {
      if (EXT && window_left >= 0)
        found = find_tile(cu_seqlens_q, num_seqs, bq, total_q, tile, lane, lane_tiles(), seq, q0);
      else if (bq_log2 >= 0)   // uniform
        found = find_tile_lpt<true>(cu_seqlens_q, seq_lens, num_seqs, total_q,
                                    max_blocks_per_seq << log2_bs, bq, bq_log2, causal, tile,
                                    lane, my_lq, my_lk, narrow_q, seq, q0);
      else
        found = find_tile_lpt<false>(cu_seqlens_q, seq_lens, num_seqs, total_q,
                                     max_blocks_per_seq << log2_bs, bq, bq_log2, causal, tile,
                                     lane, my_lq, my_lk, narrow_q, seq, q0);
    }
    if (!found) seq = -1;
    if (seq >= 0 && seq < kWave) {
      r0 = lane_value(my_r0, seq);
      lq_ = lane_value(my_lq, seq);
      lk_ = lane_value(my_lk, seq);
    } else if (seq >= kWave) {
      r0 = max(0, min(cu_seqlens_q[seq], total_q));
      lq_ = max(0, min(cu_seqlens_q[seq + 1], total_q) - r0);
      lk_ = max(0, min(seq_lens[seq], max_blocks_per_seq << log2_bs));
    }
    tl[0] = seq;
    tl[1] = q0;
    tl[2] = r0;
    tl[3] = lq_;
    tl[4] = lk_;
  }
  const int b = __builtin_amdgcn_readfirstlane(tl[0]);
  if (b < 0) return;   // the same in every wave
  const int q0 = __builtin_amdgcn_readfirstlane(tl[1]);
  const int row0 = __builtin_amdgcn_readfirstlane(tl[2]);
  const int lq = __builtin_amdgcn_readfirstlane(tl[3]);
  const int lk = __builtin_amdgcn_readfirstlane(tl[4]);
  const int delta = lk - lq;

  // rows of this lane: r = wave*32 + mt*16 + l16 -> (query i = r / group, head r % group)
  int q_pos[2], head[2], lim[2];
  bool row_ok[2];
  // r / group for r < 128 as (r * ceil(2^16 / group)) >> 16: exact, since
  // the reciprocal's excess (< group <= 128) times r stays below 2^16
  const int group_inv16 = (65536 + group - 1) / group;   // uniform
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = wave * kVlRowsWave + mt * 16 + l16;
    const int i = (r * group_inv16) >> 16;
    q_pos[mt] = q0 + i;
    head[mt] = kvh * group + (r - i * group);
    row_ok[mt] = (i < bq) && (q_pos[mt] < lq);
    lim[mt] = row_ok[mt] ? (causal ? min(lk - 1, q_pos[mt] + delta) : lk - 1) : -1;
  }

  // keys this tile needs (up to the largest lim over its rows); keys below
  // `nomask_end` are visible to every row of the tile
  const int last_q = min(q0 + bq, lq) - 1;
  const int kv_end = causal ? min(lk, last_q + delta + 1) : lk;
  const int nomask_end = causal ? min(lk, q0 + delta + 1) : lk;
  // variants: row r's lowest visible key (window) and ALiBi slope (log2
  // units); the tile starts at its rows' lowest bound, 64-aligned, and keys
  // below `mask_lo_end` are hidden from some row of the tile
  const bool windowed = EXT && window_left >= 0;
  int wlo[2] = {0, 0}, p_abs[2] = {0, 0};
  float al2[2] = {0.f, 0.f};
  if constexpr (EXT) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      p_abs[mt] = q_pos[mt] + delta;
      wlo[mt] = windowed ? max(0, p_abs[mt] - window_left) : 0;
      al2[mt] = (alibi != nullptr && row_ok[mt]) ? alibi[head[mt]] * 1.4426950408889634f : 0.f;
    }
  }
  const int kv_begin = windowed ? (max(0, q0 + delta - window_left) & ~(kVlBN - 1)) : 0;
  // this workgroup's part of the key loop: [kv_lo, kv_hi)
  int n_chunks = 1, kv_lo = kv_begin, kv_hi = kv_end;
  if constexpr (SPLIT) {
    n_chunks = split_chunks(q0, lq, lk, bq, group, causal, chunk_tiles);
    if (chunk >= n_chunks) return;   // uniform over the workgroup
    if (n_chunks > 1) {              // a tile that is not cut keeps its whole loop
      kv_lo = kv_begin + chunk * chunk_tiles * kVlBN;
      kv_hi = min(kv_end, kv_lo + chunk_tiles * kVlBN);
    }
    // a narrow sequence (one tile of at most 16 rows): its whole tile or
    // this chunk of it through the narrow path, the chunk's triple into the
    // same slots as below
    if (lq <= kVlNarrowRows / group) {   // uniform
      const int64_t ws_row0 =
          n_chunks > 1 ? (((int64_t)chunk * num_seqs + b) * num_kv_heads + kvh) * kVlRowsWave : -1;
      varlen_narrow<Ty, D>(out, q, reinterpret_cast<const uint8_t*>(k_cache),
                           reinterpret_cast<const uint8_t*>(v_cache),
                           block_table + (size_t)b * max_blocks_per_seq, row0, lq, lk, kv_lo,
                           kv_hi, causal, num_q_heads, kvh, group, log2_bs, (uint32_t)num_blocks,
                           (uint32_t)(num_kv_heads * D) * 2u, scale_log2, ws_ml, ws_o, ws_row0,
                           s_kv, tid, wave, lane);
      return;
    }
  }
  const int mask_lo_end = windowed ? max(0, last_q + delta - window_left) : 0;

  const int row_stride = num_kv_heads * D;
  const int32_t* bt_row = block_table + (size_t)b * max_blocks_per_seq;

  // Stage keys kv0 .. kv0+63 into stage `st`: each lane fetches one 16-byte
  // chunk straight into LDS. A copy instruction covers RPI consecutive keys,
  // which always lie in one cache block, so its source is a wave-uniform
  // block address (from a scalar load of the block id) plus a loop-invariant
  // 32-bit lane offset. In the last tile, keys past Lk fetch the last valid
  // key instead (finite values whose probabilities are masked to zero).
  // per-lane parts (loop invariant): row of the tile, swizzled source
  // chunk, kv head -> byte offset from the tile's first row, so that every
  // copy of a tile that lies in one block shares one scalar base address
  const uint32_t row_bytes = (uint32_t)row_stride * 2u;
  uint32_t voffk_[LPT], voffv_[LPT];
  int lrow_[LPT], loffk_[LPT], loffv_[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int rbase = (j * kVlWaves + wave) * RPI;
    lrow_[j] = rbase + lane / L::spr;
    // the lane's LDS slot is lane % spr; it holds chunk slot ^ f(row)
    loffk_[j] = kvh * D + L::slot_k(lrow_[j], lane % L::spr) * 8;
    loffv_[j] = kvh * D + L::slot_v(lrow_[j], lane % L::spr) * 8;
    voffk_[j] = (uint32_t)lrow_[j] * row_bytes + (uint32_t)loffk_[j] * 2u;
    voffv_[j] = (uint32_t)lrow_[j] * row_bytes + (uint32_t)loffv_[j] * 2u;
  }
  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(k_cache);
  const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(v_cache);
  const uint32_t lds_kv = lds_address(s_kv);
  // the pool's block count fits 32 bits (num_blocks * block_size is checked
  // against INT32_MAX by the caller)
  const uint32_t nblocks32 = (uint32_t)num_blocks;
  auto valid_block = [&](int blk) {   // out-of-range ids read block 0
    return (uint32_t)blk < nblocks32 ? blk : 0;
  };
  // byte offset of pool row r (a 32-bit row index) as a signed 64-bit value
  auto row_offset = [&](int r) { return (int64_t)r * (int64_t)row_bytes; };
  // (debug build) an out-of-range id of a block the tile uses: one holding
  // keys below Lk and, under a window, not wholly before the first row's
  auto dbg_block = [&](int raw, int blk_index) {
    PKV_DBG_REPORT((uint32_t)raw >= nblocks32 && (blk_index << log2_bs) < lk &&
                       ((blk_index + 1) << log2_bs) > (windowed ? q0 + delta - window_left : 0),
                   kDbgBlockId);
  };
  auto stage = [&](int st, int kv0) {
    const uint32_t lds_st = lds_kv + (uint32_t)(st * L::stageB);
    const int i0 = kv0 >> log2_bs;
    if (kv0 + kVlBN <= lk) {
      if (bs >= kVlBN) {   // the whole tile lies in one block: one base
        const int raw = __builtin_amdgcn_readfirstlane(bt_row[i0]);
        dbg_block(raw, i0);
        const int blk = valid_block(raw);
        const int64_t base = row_offset(blk * bs + (kv0 & (bs - 1)));
        const uint8_t* kb = kbytes + base;
        const uint8_t* vb = vbytes + base;
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int rbase = (j * kVlWaves + wave) * RPI;
          async_copy16_to_lds(kb, voffk_[j], lds_st + rbase * L::rowB);
          async_copy16_to_lds(vb, voffv_[j], lds_st + L::tileB + rbase * L::rowB);
        }
      } else {
        // copy j covers rows rbase .. rbase+RPI-1, all in table entry
        // i0 + rbase / bs (kv0 is a multiple of the tile, hence of bs); the
        // lane offsets count rows from the tile's first key, so the base is
        // that block's start less the block's first row within the tile.
        // The ids are requested together, one wait for all.
        int ids[LPT];
#pragma unroll
        for (int j = 0; j < LPT; ++j)
          ids[j] = __builtin_amdgcn_readfirstlane(
              bt_row[i0 + (((j * kVlWaves + wave) * RPI) >> log2_bs)]);
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int rbase = (j * kVlWaves + wave) * RPI;
          dbg_block(ids[j], i0 + (rbase >> log2_bs));
          const int64_t src = row_offset(valid_block(ids[j]) * bs - (rbase & ~(bs - 1)));
          async_copy16_to_lds(kbytes + src, voffk_[j], lds_st + rbase * L::rowB);
          async_copy16_to_lds(vbytes + src, voffv_[j], lds_st + L::tileB + rbase * L::rowB);
        }
      }
      return;
    }
    // the tile's keys span at most four blocks (block_size >= 16): their ids
    // come from scalar loads (a per-lane load would make the next vmcnt wait
    // cover the copies in flight)
    int ids[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int raw = __builtin_amdgcn_readfirstlane(bt_row[min(i0 + e, max_blocks_per_seq - 1)]);
      dbg_block(raw, i0 + e);
      ids[e] = valid_block(raw);
    }
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int rbase = (j * kVlWaves + wave) * RPI;
      const int key = min(kv0 + lrow_[j], lk - 1);
      const int e = (key >> log2_bs) - i0;
      const int blk = e == 0 ? ids[0] : e == 1 ? ids[1] : e == 2 ? ids[2] : ids[3];
      const size_t off = ((size_t)blk * bs + (key & (bs - 1))) * row_stride;
      async_copy16_to_lds(k_cache + off + loffk_[j], lds_st + rbase * L::rowB);
      async_copy16_to_lds(v_cache + off + loffv_[j], lds_st + L::tileB + rbase * L::rowB);
    }
  };

  // Q^T operands (B of S^T = K Q^T): lane holds Q[row][32s + 8*g4 .. +8]
  u32x4_t qb[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qb[mt][s] = row_ok[mt]
                      ? load16<false>(q + ((size_t)(row0 + q_pos[mt]) * num_q_heads + head[mt]) * D +
                                      32 * s + 8 * g4)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  if (kv_lo < kv_hi) stage(0, kv_lo);

  // the queries and the first stage are needed before anything else; waiting
  // for both here keeps the compiler from placing a full wait later, when
  // the next stage's copies are in flight
  wait_vmcnt<0>();

  f32x4_t acc[2][ND];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[mt][nd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_use[2] = {-INFINITY, -INFINITY};   // max the exponentials are taken against
  float nref[2] = {0.f, 0.f};                // -safe_max_ref(m_use): the exponent offset
  // row sums of P, accumulated as O^T of an all-ones V^T: every register of
  // the lane holds its row's sum
  f32x4_t lacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const uint32_t one2 = Mma<Ty>::pack(1.f, 1.f);
  const u32x4_t ones = {one2, one2, one2, one2};

  // per-lane LDS offsets (within a stage)
  // K operand, key block n, k-step s: row 16n + l16, chunk 4s + g4
  // V^T operand: lane i of a 16-lane group -> row 4*g4 + i/4 (+16), chunk
  // 2nd + (i%4)/2, byte 8*(i%2) within the chunk
  const int vrow = 4 * g4 + (l16 >> 2);
  const int vbyte = 8 * (l16 & 1);
  const int vchunk = (l16 & 3) >> 1;
  // Their lane parts do not depend on the stage or the half: the swizzle
  // function sees a row only modulo 16 (8 at D = 64), and rows 32hh + 16n +
  // l16 (K) or 32hh + vrow (+16) (V^T) agree with l16 / vrow there. So a
  // lane keeps KS + ND byte offsets, and the stage, the half and the row
  // block are immediate offsets of the LDS reads.
  uint32_t kofs[KS], vofs[ND];
#pragma unroll
  for (int s = 0; s < KS; ++s) kofs[s] = l16 * L::rowB + L::slot_k(l16, 4 * s + g4) * 16;
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
    vofs[nd] = L::tileB + vrow * L::rowB + L::slot_v(vrow, 2 * nd + vchunk) * 16 + vbyte;

  // A wave whose rows are all padding (a tile of a few queries, such as the
  // decode rows of a mixed batch) only helps stage the tiles and skips the
  // arithmetic.
  const bool wave_live = __builtin_amdgcn_ballot_w64(row_ok[0] || row_ok[1]) != 0;

  // One 64-key tile; CUR, the stage it reads, is a compile-time constant in
  // each of the two copies the loop below inlines.
  auto key_tile = [&](auto cur_tag, int kv0, int it) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_tag)::value;
    const bool more = kv0 + kVlBN < kv_hi;
    // this tile's copies (issued one iteration earlier) have landed in LDS,
    // and every wave is past the previous iteration, so the other stage,
    // read there, may be refilled: one barrier per tile
    wait_vmcnt<0>();
    barrier_lds_ops();
    if (more) stage(cur ^ 1, kv0 + kVlBN);
    const uint8_t* sk = s_kv + cur * L::stageB;   // this stage; V^T at sk + tileB
    // (kept in registers: not hoisted as per-stage sums)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(kofs[s]));
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) asm volatile("" : "+v"(vofs[nd]));
    const bool need_mask = kv0 + kVlBN > nomask_end || (windowed && kv0 < mask_lo_end);
    if (wave_live) {
      // Operand reads from LDS are issued a phase ahead of the MFMAs that use
      // them, so their latency hides behind the softmax arithmetic:
      //   K operands of half h+1 and V^T operands of half h are read, the
      //   softmax of half h runs, then q.k of half h+1 and p.v of half h issue.
      auto read_k = [&](int hh, u32x4_t (&ka)[2][KS]) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
#pragma unroll
          for (int s = 0; s < KS; ++s)
            ka[n][s] = *reinterpret_cast<const u32x4_t*>(sk + kofs[s] + (32 * hh + 16 * n) * L::rowB);
        }
      };
      auto qk = [&](const u32x4_t (&ka)[2][KS], f32x4_t (&st)[2][2]) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          st[n][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          st[n][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            st[n][0] = Mma<Ty>::mfma(ka[n][s], qb[0][s], st[n][0]);
            st[n][1] = Mma<Ty>::mfma(ka[n][s], qb[1][s], st[n][1]);
          }
        }
      };
      auto read_v = [&](int hh, u32x4_t (&va)[ND]) {
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          const u32x2_t lo = lds_read_tr16(sk + vofs[nd] + 32 * hh * L::rowB);
          const u32x2_t hi = lds_read_tr16(sk + vofs[nd] + (32 * hh + 16) * L::rowB);
          va[nd] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
      };

      f32x4_t st_cur[2][2];
      {
        u32x4_t ka[2][KS];
        read_k(0, ka);
        qk(ka, st_cur);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {   // two halves of 32 keys
        u32x4_t ka[2][KS];
        u32x4_t va[ND];
        if (hh == 0) read_k(1, ka);
        read_v(hh, va);
        // ---- online softmax; lane's keys: kv0 + 32hh + 16n + 4*g4 + i ----
        // Scores stay unscaled: the max is taken on raw q.k (the scale is
        // positive) and the exponent is one fma, s*scale - m.
        if (need_mask) {
          // key kv0 + 32hh + 16n + 4*g4 + i is visible iff 32hh + 16n + i <= thr
          // (and, with a window, >= thr_lo)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const int thr = lim[mt] - kv0 - 4 * g4;
            const int thr_lo = wlo[mt] - kv0 - 4 * g4;
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int o = 32 * hh + 16 * n + i;
                const bool vis = EXT ? (o <= thr && o >= thr_lo) : (o <= thr);
                st_cur[n][mt][i] = vis ? st_cur[n][mt][i] : -INFINITY;
              }
          }
        }
        // variants: scores are scaled and biased here (the max must see the
        // bias), so the exponent below takes a unit scale
        if constexpr (EXT) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const float dj0 = (float)(kv0 + 32 * hh + 4 * g4 - p_abs[mt]);
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                st_cur[n][mt][i] =
                    fmaf(st_cur[n][mt][i], scale_log2, al2[mt] * (dj0 + (float)(16 * n + i)));
          }
        }
        constexpr float one = 1.f;
        const float sc = EXT ? one : scale_log2;
        // lane-local maxima (raw scores); the row max over the 4 lane groups is
        // only needed when the running max has to move
        // (maximum, not fmax: no NaN canonicalisation of the MFMA results)
        float mx[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float a = st_cur[0][mt][0];
#pragma unroll
          for (int k = 1; k < 8; ++k) a = __builtin_elementwise_maximum(a, st_cur[k >> 2][mt][k & 3]);
          mx[mt] = a * sc;
        }
        const bool grow = (mx[0] > m_use[0] + kRescale) || (mx[1] > m_use[1] + kRescale);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform, rare
          // before the first half is accumulated the sums are still zero
          const bool rescale = it > 0 || hh > 0;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            float m = mx[mt];
            m = fmaxf(m, shfl_xor_f(m, 16));
            m = fmaxf(m, shfl_xor_f(m, 32));
            const float mnew = fmaxf(m_use[mt], m);
            const float alpha = fast_exp2(m_use[mt] - safe_max_ref(mnew));
            m_use[mt] = mnew;
            nref[mt] = -safe_max_ref(mnew);
            if (rescale) {
              lacc[mt] *= alpha;
#pragma unroll
              for (int nd = 0; nd < ND; ++nd) acc[mt][nd] *= alpha;
            }
          }
        }
        u32x4_t pb[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          float pv[2][4];
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[n][i] = fast_exp2(fmaf(st_cur[n][mt][i], sc, nref[mt]));
          pb[mt][0] = Mma<Ty>::pack(pv[0][0], pv[0][1]);
          pb[mt][1] = Mma<Ty>::pack(pv[0][2], pv[0][3]);
          pb[mt][2] = Mma<Ty>::pack(pv[1][0], pv[1][1]);
          pb[mt][3] = Mma<Ty>::pack(pv[1][2], pv[1][3]);
        }
        // ---- q.k of the next half, then O^T += V^T P^T over these 32 keys ----
        if (hh == 0) qk(ka, st_cur);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          // row sums of the rounded P on the matrix cores: a V^T tile of ones
          lacc[mt] = Mma<Ty>::mfma(ones, pb[mt], lacc[mt]);
        }
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) {
          acc[0][nd] = Mma<Ty>::mfma(va[nd], pb[0], acc[0][nd]);
          acc[1][nd] = Mma<Ty>::mfma(va[nd], pb[1], acc[1][nd]);
        }
      }
    }
  };
  for (int kv0 = kv_lo, it = 0; kv0 < kv_hi; kv0 += 2 * kVlBN, it += 2) {
    key_tile(stage_tag<0>{}, kv0, it);
    if (kv0 + kVlBN < kv_hi) key_tile(stage_tag<1>{}, kv0 + kVlBN, it + 1);
  }

  if (SPLIT && n_chunks > 1) {
    // partial triple of this chunk (o and the row sum relative to 2^m_use)
    // for the rows of a cut tile, all in wave 0: slot [chunk, b, kv head, row]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      if (!row_ok[mt]) continue;
      const int r = wave * kVlRowsWave + mt * 16 + l16;
      const size_t slot_i =
          (((size_t)chunk * num_seqs + b) * num_kv_heads + kvh) * kVlRowsWave + r;
      float* o = ws_o + slot_i * D + 4 * g4;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) *reinterpret_cast<f32x4_t*>(o + 16 * nd) = acc[mt][nd];
      if (g4 == 0) {
        ws_ml[slot_i * 2 + 0] = m_use[mt];
        ws_ml[slot_i * 2 + 1] = lacc[mt][0];
      }
    }
    return;
  }
  // ---- normalise and store: lane holds O^T[16nd + 4*g4 + i][row] ----
  // Each pair of 16-dim tiles (2p, 2p+1) is exchanged between the lane
  // groups g4 and g4 ^ 1 (v_permlane16_swap swaps the odd 16-lane rows of
  // its first operand with the even rows of its second), after which group
  // g4 holds the 8 consecutive dims 32p + 8 * (g4 with its two bits
  // swapped) .. + 7 of its row: a row's 64 bytes of the pair go out as one
  // 16-byte store from each of its four lanes (half the store instructions
  // of 8-byte stores of each tile).
  const int g4s = ((g4 & 1) << 1) | (g4 >> 1);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const float lt = lacc[mt][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* dst = out + ((size_t)(row0 + q_pos[mt]) * num_q_heads + head[mt]) * D + 8 * g4s;
#pragma unroll
    for (int p = 0; p < ND / 2; ++p) {
      const f32x4_t& a = acc[mt][2 * p];
      const f32x4_t& c = acc[mt][2 * p + 1];
      const auto s0 = __builtin_amdgcn_permlane16_swap(Mma<Ty>::pack(a[0] * inv, a[1] * inv),
                                                       Mma<Ty>::pack(c[0] * inv, c[1] * inv),
                                                       false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(Mma<Ty>::pack(a[2] * inv, a[3] * inv),
                                                       Mma<Ty>::pack(c[2] * inv, c[3] * inv),
                                                       false, false);
      if (row_ok[mt])
        *reinterpret_cast<u32x4_t*>(dst + 32 * p) = u32x4_t{s0[0], s1[0], s0[1], s1[1]};
    }
  }
}

// Exact merge of the chunk triples of the cut tiles, as the decode reduce:
// M = max m_c, L = sum l_c 2^(m_c - M), out = sum o_c 2^(m_c - M) / L. One
// workgroup per (sequence, kv head) recomputes the cut of the sequence's last
// tile from its lengths (as the attention kernel did) and merges its rows; a
// thread owns 4 consecutive output elements of a row.
template <class Ty, int D>
__global__ __launch_bounds__(256) void varlen_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_lens, int num_seqs,
    int total_q, int num_q_heads, int num_kv_heads, int max_lk, int causal, int chunk_tiles,
    int max_splits) {
  constexpr int TPP = D / 4;      // threads per row
  constexpr int RPP = 256 / TPP;  // rows per pass
  const int s = blockIdx.x / num_kv_heads, kvh = blockIdx.x % num_kv_heads;
  const int group = num_q_heads / num_kv_heads, bq = kVlRows / group;
  const int r0 = max(0, min(cu[s], total_q));
  const int lq = max(0, min(cu[s + 1], total_q) - r0);
  const int lk = max(0, min(seq_lens[s], max_lk));
  if (lq <= 0) return;
  const int q0 = (lq - 1) / bq * bq;   // the last tile
  const int n = min(split_chunks(q0, lq, lk, bq, group, causal, chunk_tiles), max_splits);
  if (n <= 1) return;
  const int rows = min(bq, lq - q0) * group;
  const int d0 = (threadIdx.x % TPP) * 4;
  for (int r = threadIdx.x / TPP; r < rows; r += RPP) {
    auto slot_i = [&](int c) {
      return (((size_t)c * num_seqs + s) * num_kv_heads + kvh) * kVlRowsWave + r;
    };
    // every chunk's triple is loaded before any is used (one round trip)
    float mc[kVlMaxSplits], lc[kVlMaxSplits];
    f32x4_t oc[kVlMaxSplits];
#pragma unroll
    for (int c = 0; c < kVlMaxSplits; ++c) {
      mc[c] = -INFINITY;
      lc[c] = 0.f;
      oc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (c < n) {
        mc[c] = ws_ml[slot_i(c) * 2];
        lc[c] = ws_ml[slot_i(c) * 2 + 1];
        oc[c] = *reinterpret_cast<const f32x4_t*>(ws_o + slot_i(c) * D + d0);
      }
    }
    float mm = -INFINITY;
#pragma unroll
    for (int c = 0; c < kVlMaxSplits; ++c) mm = fmaxf(mm, mc[c]);
    const float mr = safe_max_ref(mm);
    float ll = 0.f;
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kVlMaxSplits; ++c) {
      const float wt = c < n ? fast_exp2(mc[c] - mr) : 0.f;
      ll += lc[c] * wt;
      a += oc[c] * wt;
    }
    const float inv = ll > 0.f ? 1.f / ll : 0.f;
    u32x2_t w;
    w[0] = Mma<Ty>::pack(a[0] * inv, a[1] * inv);
    w[1] = Mma<Ty>::pack(a[2] * inv, a[3] * inv);
    const int i = r / group, head = kvh * group + r % group;
    *reinterpret_cast<u32x2_t*>(out + ((size_t)(r0 + q0 + i) * num_q_heads + head) * D + d0) = w;
  }
}

template <class Ty, int D, bool EXT, bool SPLIT>
static hipError_t launch_varlen_t(const VarlenArgs& a, hipStream_t stream) {
  const int64_t tiles = varlen_tiles(a.total_q, a.num_seqs, a.num_q_heads / a.num_kv_heads);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)a.head_dim);
  const VarlenSplit sp = SPLIT ? plan_varlen_split(a.max_blocks_per_seq, a.block_size)
                               : VarlenSplit{1, 1};
  const int64_t extra = SPLIT ? (int64_t)a.num_seqs * (sp.max_splits - 1) : 0;
  // the plain call's narrow-path workgroups: one per (sequence, kv head)
  const int narrow_seqs = !EXT && !SPLIT ? a.num_seqs : 0;
  dim3 grid((unsigned)((narrow_seqs + tiles + extra) * a.num_kv_heads));
  launch_kernel((varlen_prefill_kernel<Ty, D, EXT, SPLIT>), grid, dim3(kVlThreads), 0, stream,
                static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                a.cu_seqlens_q, static_cast<const uint16_t*>(a.k_cache),
                static_cast<const uint16_t*>(a.v_cache), a.block_table, a.seq_lens, a.causal,
                a.num_seqs, (int)a.total_q, a.num_q_heads, a.num_kv_heads,
                __builtin_ctz(a.block_size), a.max_blocks_per_seq, a.num_blocks, scale_log2,
                a.alibi, a.window_left, a.ws_ml, a.ws_o, sp.chunk_tiles, sp.max_splits,
                (int)tiles, narrow_seqs);
  hipError_t err = hipGetLastError();
  if (!SPLIT || err != hipSuccess) return err;
  launch_kernel((varlen_merge_kernel<Ty, D>), dim3((unsigned)(a.num_seqs * a.num_kv_heads)),
                dim3(256), 0, stream, static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o,
                a.cu_seqlens_q, a.seq_lens, a.num_seqs, (int)a.total_q, a.num_q_heads,
                a.num_kv_heads, a.max_blocks_per_seq * a.block_size, a.causal, sp.chunk_tiles,
                sp.max_splits);
  return hipGetLastError();
}

template <bool EXT, bool SPLIT>
static hipError_t launch_varlen_any(const VarlenArgs& a, hipStream_t stream) {
  if (a.dtype == 1) {
    return a.head_dim == 64 ? launch_varlen_t<F16, 64, EXT, SPLIT>(a, stream)
                            : launch_varlen_t<F16, 128, EXT, SPLIT>(a, stream);
  }
  return a.head_dim == 64 ? launch_varlen_t<BF16, 64, EXT, SPLIT>(a, stream)
                          : launch_varlen_t<BF16, 128, EXT, SPLIT>(a, stream);
}

hipError_t launch_varlen(const VarlenArgs& a, hipStream_t stream) {
  return launch_varlen_any<false, false>(a, stream);
}

hipError_t launch_varlen_ext(const VarlenArgs& a, hipStream_t stream) {
  return launch_varlen_any<true, false>(a, stream);
}

hipError_t launch_varlen_split(const VarlenArgs& a, hipStream_t stream) {
  if (plan_varlen_split(a.max_blocks_per_seq, a.block_size).max_splits <= 1)
    return launch_varlen_any<false, false>(a, stream);
  return launch_varlen_any<false, true>(a, stream);
}

PKV_DBG_TAKE_FN(debug_take_varlen)

}  // namespace pkv
