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

#include "pkv_launch.h"

namespace pkv {

constexpr int kVlWaves = 4;
constexpr int kVlThreads = kVlWaves * kWave;
constexpr int kVlRows = 128;      // rows per workgroup = query positions x heads of the group
constexpr int kVlRowsWave = 32;   // two 16-row MFMA tiles per wave
constexpr int kVlBN = 64;         // keys per KV tile

template <int D>
struct VlLds {
  static constexpr int kRowB = D * 2 + 16;        // K tile row pitch (bytes), padded
  static constexpr int vRowB = kVlBN * 2 + 16;     // V^T tile row pitch (bytes), padded
  static constexpr int kBytes = kVlBN * kRowB;
  static constexpr int vBytes = D * vRowB;
};

// Locate query tile `t` (0-based over the whole batch, tiles of `bq` rows per
// sequence) by a wave-wide prefix scan of per-sequence tile counts.
// Returns false when t is past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ cu, int num_seqs, int bq,
                                          int t, int lane, int& seq, int& q0) {
  int base_tiles = 0;
  for (int s0 = 0; s0 < num_seqs; s0 += kWave) {
    const int s = s0 + lane;
    int nt = 0;
    if (s < num_seqs) {
      const int lq = cu[s + 1] - cu[s];
      nt = lq > 0 ? (lq + bq - 1) / bq : 0;
    }
    int incl = nt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    if (t < base_tiles + total) {
      const unsigned long long hit = __ballot(base_tiles + incl > t);
      const int first = __builtin_ctzll(hit);
      const int excl = __shfl(incl - nt, first, kWave);
      seq = s0 + first;
      q0 = (t - base_tiles - excl) * bq;
      return true;
    }
    base_tiles += total;
  }
  return false;
}

template <class Ty, int D>
__global__ __launch_bounds__(kVlThreads) void varlen_prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ cu_seqlens_q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int causal, int num_seqs, int total_q, int num_q_heads,
    int num_kv_heads, int log2_bs, int max_blocks_per_seq, int64_t num_blocks, float scale_log2) {
  using L = VlLds<D>;
  constexpr int KS = D / 32;   // k-steps of the QK product
  constexpr int ND = D / 16;   // 16-wide dim tiles of the output
  constexpr int CPT = D / 8;   // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) uint8_t s_k[L::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[L::vBytes];
  __shared__ int s_tile[2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int kvh = blockIdx.y;
  const int group = num_q_heads / num_kv_heads;
  const int bq = kVlRows / group;   // query positions per tile
  const int bs = 1 << log2_bs;

  if (wave == 0) {
    int seq = -1, q0 = 0;
    if (!find_tile(cu_seqlens_q, num_seqs, bq, blockIdx.x, lane, seq, q0)) seq = -1;
    if (lane == 0) {
      s_tile[0] = seq;
      s_tile[1] = q0;
    }
  }
  __syncthreads();
  const int b = s_tile[0];
  if (b < 0) return;
  const int q0 = s_tile[1];
  const int row0 = max(0, min(cu_seqlens_q[b], total_q));
  const int lq = max(0, min(cu_seqlens_q[b + 1], total_q) - row0);
  const int lk = max(0, min(seq_lens[b], max_blocks_per_seq << log2_bs));
  const int delta = lk - lq;

  // rows of this lane: r = wave*32 + mt*16 + l16 -> (query i = r / group, head r % group)
  int q_pos[2], head[2], lim[2];
  bool row_ok[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = wave * kVlRowsWave + mt * 16 + l16;
    const int i = r / group;
    q_pos[mt] = q0 + i;
    head[mt] = kvh * group + r % group;
    row_ok[mt] = (i < bq) && (q_pos[mt] < lq);
    // last key index this row may see (-1: none)
    lim[mt] = row_ok[mt] ? (causal ? min(lk - 1, q_pos[mt] + delta) : lk - 1) : -1;
  }

  // Q^T operands (B of S^T = K Q^T): lane holds Q[row][32s + 8*g4 .. +8]
  u32x4_t qb[2][KS];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const bool ok = row_ok[mt];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (ok) {
        const uint16_t* src = q + ((size_t)(row0 + q_pos[mt]) * num_q_heads + head[mt]) * D +
                              32 * s + 8 * g4;
        qb[mt][s] = *reinterpret_cast<const u32x4_t*>(src);
      } else {
        qb[mt][s] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  // keys this tile needs: up to the largest lim over the tile's rows
  const int last_q = min(q0 + bq, lq) - 1;
  const int kv_end = causal ? min(lk, last_q + delta + 1) : lk;

  f32x4_t acc[2][ND];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[mt][nd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int row_stride = num_kv_heads * D;
  const int32_t* bt_row = block_table + (size_t)b * max_blocks_per_seq;

  for (int kv0 = 0; kv0 < kv_end; kv0 += kVlBN) {
    // ---- stage K (row-major) and V^T (dim-major) for keys kv0 .. kv0+63 ----
    __syncthreads();  // previous tile's LDS reads are done
#pragma unroll
    for (int j = 0; j < (kVlBN * CPT) / kVlThreads; ++j) {
      const int id = j * kVlThreads + tid;
      const int t = id / CPT, ch = id % CPT;
      const int key = kv0 + t;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (key < lk) {
        int blk = bt_row[key >> log2_bs];
        if (blk >= 0 && blk < num_blocks) {
          const uint16_t* src = k_cache + ((size_t)blk * bs + (key & (bs - 1))) * row_stride +
                                kvh * D + ch * 8;
          v = *reinterpret_cast<const u32x4_t*>(src);
        }
      }
      *reinterpret_cast<u32x4_t*>(s_k + t * L::kRowB + ch * 16) = v;
    }
#pragma unroll
    for (int j = 0; j < (kVlBN / 2 * CPT) / kVlThreads; ++j) {
      const int id = j * kVlThreads + tid;
      const int tp = id / CPT, ch = id % CPT;
      u32x4_t v2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = kv0 + 2 * tp + h;
        v2[h] = u32x4_t{0u, 0u, 0u, 0u};
        if (key < lk) {
          int blk = bt_row[key >> log2_bs];
          if (blk >= 0 && blk < num_blocks) {
            const uint16_t* src = v_cache + ((size_t)blk * bs + (key & (bs - 1))) * row_stride +
                                  kvh * D + ch * 8;
            v2[h] = *reinterpret_cast<const u32x4_t*>(src);
          }
        }
      }
      // element e of the chunk is dim ch*8+e; write (key 2tp, key 2tp+1) as one dword
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = v2[0][w], c = v2[1][w];
        const uint32_t lo = (a & 0xffffu) | (c << 16);          // dim ch*8 + 2w
        const uint32_t hi = (a >> 16) | (c & 0xffff0000u);      // dim ch*8 + 2w + 1
        *reinterpret_cast<uint32_t*>(s_v + (ch * 8 + 2 * w) * L::vRowB + tp * 4) = lo;
        *reinterpret_cast<uint32_t*>(s_v + (ch * 8 + 2 * w + 1) * L::vRowB + tp * 4) = hi;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: 4 key tiles x 2 row tiles ----
    f32x4_t st[4][2];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      st[n][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st[n][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(s_k + (16 * n + l16) * L::kRowB + 64 * s + 16 * g4);
        st[n][0] = Mma<Ty>::mfma(a, qb[0][s], st[n][0]);
        st[n][1] = Mma<Ty>::mfma(a, qb[1][s], st[n][1]);
      }
    }

    // ---- online softmax per row; lane's keys: kv0 + 16n + 4*g4 + i ----
    u32x4_t pb[2][2];   // P^T operands for the two 32-key halves
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float sv[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kv0 + 16 * n + 4 * g4 + i;
          const float x = st[n][mt][i] * scale_log2;
          sv[n][i] = key <= lim[mt] ? x : -INFINITY;
          mx = fmaxf(mx, sv[n][i]);
        }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float mnew = fmaxf(m_run[mt], mx);
      const float mref = safe_max_ref(mnew);
      const float alpha = fast_exp2(m_run[mt] - mref);
      m_run[mt] = mnew;
      float psum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[n][i] = fast_exp2(sv[n][i] - mref);
          psum += pv[n][i];
        }
      l_run[mt] = l_run[mt] * alpha + psum;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) acc[mt][nd] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pb[mt][kk][0] = Mma<Ty>::pack(pv[2 * kk][0], pv[2 * kk][1]);
        pb[mt][kk][1] = Mma<Ty>::pack(pv[2 * kk][2], pv[2 * kk][3]);
        pb[mt][kk][2] = Mma<Ty>::pack(pv[2 * kk + 1][0], pv[2 * kk + 1][1]);
        pb[mt][kk][3] = Mma<Ty>::pack(pv[2 * kk + 1][2], pv[2 * kk + 1][3]);
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint8_t* vrow = s_v + (16 * nd + l16) * L::vRowB + (32 * kk + 4 * g4) * 2;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 32);
        const u32x4_t a = {lo[0], lo[1], hi[0], hi[1]};
        acc[0][nd] = Mma<Ty>::mfma(a, pb[0][kk], acc[0][nd]);
        acc[1][nd] = Mma<Ty>::mfma(a, pb[1][kk], acc[1][nd]);
      }
    }
  }

  // ---- normalise and store: lane holds O^T[16nd + 4*g4 + i][row] ----
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    float lt = l_run[mt];
    lt += shfl_xor_f(lt, 16);
    lt += shfl_xor_f(lt, 32);
    if (!row_ok[mt]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* dst = out + ((size_t)(row0 + q_pos[mt]) * num_q_heads + head[mt]) * D + 4 * g4;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      u32x2_t w;
      w[0] = Mma<Ty>::pack(acc[mt][nd][0] * inv, acc[mt][nd][1] * inv);
      w[1] = Mma<Ty>::pack(acc[mt][nd][2] * inv, acc[mt][nd][3] * inv);
      *reinterpret_cast<u32x2_t*>(dst + 16 * nd) = w;
    }
  }
}

template <class Ty, int D>
static hipError_t launch_varlen_t(const VarlenArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int bq = kVlRows / group;
  const int64_t tiles = (a.total_q + bq - 1) / bq + a.num_seqs;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)a.head_dim);
  dim3 grid((unsigned)tiles, a.num_kv_heads);
  hipLaunchKernelGGL((varlen_prefill_kernel<Ty, D>), grid, dim3(kVlThreads), 0, stream,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.q),
                     a.cu_seqlens_q, static_cast<const uint16_t*>(a.k_cache),
                     static_cast<const uint16_t*>(a.v_cache), a.block_table, a.seq_lens,
                     a.causal, a.num_seqs, (int)a.total_q, a.num_q_heads, a.num_kv_heads,
                     __builtin_ctz(a.block_size), a.max_blocks_per_seq, a.num_blocks,
                     scale_log2);
  return hipGetLastError();
}

hipError_t launch_varlen(const VarlenArgs& a, hipStream_t stream) {
  if (a.dtype == 1) {
    return a.head_dim == 64 ? launch_varlen_t<F16, 64>(a, stream)
                            : launch_varlen_t<F16, 128>(a, stream);
  }
  return a.head_dim == 64 ? launch_varlen_t<BF16, 64>(a, stream)
                          : launch_varlen_t<BF16, 128>(a, stream);
}

}  // namespace pkv
