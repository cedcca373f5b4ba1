// Paged decode attention: one query token per sequence attends over its
// context, read block by block through the block table.
//
// Definition: out[b,h] = sum_j softmax_j(scale * <q[b,h], K_j>) V_j over the
// context_lens[b] tokens of sequence b ("model-infer-kvcache" skill page,
// Appendix C: decode uses no mask and the KV length bounds the keys; the
// "ATB PagedAttention" page computes it page by page with an online softmax).
//
// Split-KV: the context is cut into partitions of kDecodePart tokens. One
// workgroup handles one (partition, group of query heads sharing a kv head,
// sequence) and produces, per query head, the partial triple
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

#include "pkv_launch.h"

namespace pkv {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kQuadsPerIter = 8;                  // each row handles 8 tokens per iteration
constexpr int kTokPerIter = 4 * kQuadsPerIter;    // 32 tokens per wave iteration

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
  const size_t part_base = (size_t)part_start;  // block aligned: kDecodePart % bs == 0
  (void)part_base;

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
      kr[u] = load_chunk<Ty, EPL>(kb + off);
      vr[u] = load_chunk<Ty, EPL>(vb + off);
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

// Exact merge of the partition triples of one (sequence, query head):
// M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p 2^(m_p - M) / L.
template <class Ty, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    typename Ty::storage* __restrict__ out, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens, int num_q_heads,
    int log2_bs, int max_blocks_per_seq, int num_parts) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int ctx = context_lens[b];
  ctx = max(0, min(ctx, max_blocks_per_seq << log2_bs));
  const int np = (ctx + kDecodePart - 1) / kDecodePart;
  if (np <= 1) return;
  const size_t bh = (size_t)b * num_q_heads + h;
  const float* ml = ws_ml + bh * num_parts * 2;
  const float* o = ws_o + bh * num_parts * D;
  float mm = -INFINITY;
  for (int p = 0; p < np; ++p) mm = fmaxf(mm, ml[2 * p]);
  const float mr = safe_max_ref(mm);
  float ll = 0.f, acc = 0.f;
  for (int p = 0; p < np; ++p) {
    const float wt = fast_exp2(ml[2 * p] - mr);
    ll += ml[2 * p + 1] * wt;
    acc += o[(size_t)p * D + d] * wt;
  }
  out[bh * D + d] = from_f32<Ty>(ll > 0.f ? acc / ll : 0.f);
}

template <class Ty, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  using S = typename Ty::storage;
  const int log2_bs = __builtin_ctz(a.block_size);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const int group = a.num_q_heads / a.num_kv_heads;
  dim3 grid(a.num_parts, a.num_q_heads / G, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<Ty, D, G>), grid, dim3(kDecThreads), 0, stream,
                     static_cast<S*>(a.out), static_cast<const S*>(a.q),
                     static_cast<const S*>(a.k_cache), static_cast<const S*>(a.v_cache),
                     a.block_table, a.context_lens, a.ws_ml, a.ws_o, scale_log2, a.num_q_heads,
                     a.num_kv_heads, group, log2_bs, a.max_blocks_per_seq, a.num_blocks,
                     a.num_parts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.num_parts <= 1) return err;
  hipLaunchKernelGGL((decode_reduce_kernel<Ty, D>), dim3(a.num_q_heads, a.num_seqs), dim3(D), 0,
                     stream, static_cast<S*>(a.out), a.ws_ml, a.ws_o, a.context_lens,
                     a.num_q_heads, log2_bs, a.max_blocks_per_seq, a.num_parts);
  return hipGetLastError();
}

template <class Ty, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (g % 8 == 0) return launch_decode_t<Ty, D, 8>(a, stream);
  if (g % 4 == 0) return launch_decode_t<Ty, D, 4>(a, stream);
  if (g % 2 == 0) return launch_decode_t<Ty, D, 2>(a, stream);
  return launch_decode_t<Ty, D, 1>(a, stream);
}

template <class Ty>
static hipError_t launch_decode_ty(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 64) return launch_decode_d<Ty, 64>(a, stream);
  return launch_decode_d<Ty, 128>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return launch_decode_ty<F32>(a, stream);
    case 1: return launch_decode_ty<F16>(a, stream);
    default: return launch_decode_ty<BF16>(a, stream);
  }
}

}  // namespace pkv
