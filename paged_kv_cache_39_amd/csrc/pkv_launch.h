// Internal launcher declarations (host side). Sizes are validated by the
// C-ABI entry points before any of these is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_common.h"

namespace pkv {

// Events the calling thread's next kernel launch records at its own dispatch
// start and end (set by pkv_time_next_kernel; consumed by one launch).
struct KernelTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
KernelTiming& pending_timing();
// Partition length the calling thread's 16-bit decode calls use instead of
// the launch plan's (0: the plan decides; set by
// pkv_decode_partition_override).
int& decode_partition_override();

// Every kernel of the library is launched through here.
template <typename... Formals, typename... Actuals>
inline void launch_kernel(void (*kernel)(Formals...), dim3 grid, dim3 block, uint32_t shmem,
                          hipStream_t stream, Actuals... args) {
  KernelTiming& t = pending_timing();
  if (t.start != nullptr || t.stop != nullptr) {
    const KernelTiming use = t;
    t = KernelTiming{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, use.start, use.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  }
}

// Tokens per split-KV partition of the decode path (the long-context split),
// and the longest single partition a decode workgroup takes when the batch
// alone already fills the chip.
constexpr int kDecodePart = 512;
constexpr int kDecodeWidePart = 2048;
constexpr int kNumCUs = 256;

inline int decode_parts(int max_blocks_per_seq, int block_size, int part_tokens) {
  const long long max_ctx = (long long)max_blocks_per_seq * block_size;
  return (int)((max_ctx + part_tokens - 1) / part_tokens);
}

// Launch plan of the matrix-core decode: `rows` = sequences x head groups.
// - With at least one row per compute unit and contexts up to 2048 tokens,
//   one 8-wave workgroup takes a whole context (no split, no reduce).
// - Otherwise the context is split into partitions merged by the reduce
//   kernel: the longest of 4096, 2048 or 1024 tokens that still gives at
//   least kDecodeWgsPerCU workgroups per compute unit, for 8-wave workgroups
//   (fewer, longer partitions: fewer workgroup start-ups and a smaller
//   reduce); when even 1024-token partitions leave the chip short of work,
//   512-token partitions for 4-wave workgroups.
// - Small problems (fine_ok): when 512-token partitions still leave CUs
//   without a workgroup, 256- or 128-token partitions.
struct DecodePlan {
  int waves;
  int part_tokens;
};
constexpr int kDecodeMaxPart = 4096;
constexpr int kDecodeWgsPerCU = 4;
constexpr int kDecodeFinePart = 128;
// Whether a call may take partitions shorter than 512 tokens: decided from
// what the workspace-size function is given (no kv head count), and true
// only for small problems, whose workspace stays small at that granularity.
inline bool decode_fine_ok(long long num_seqs, long long num_q_heads, int max_blocks_per_seq,
                           int block_size) {
  return num_seqs * num_q_heads * decode_parts(max_blocks_per_seq, block_size, kDecodePart) <
         16LL * kNumCUs;
}
// Decode workgroups are dispatched round-robin over the 8 XCDs (slot i on
// XCD i mod 8). Measured with 256-byte kv slices (D = 128, 16-bit cache),
// workgroups stream faster when bit 8 of the addresses they read differs
// from their XCD's parity than when the two agree: the LLaMA-7B-shaped
// decode 46.3 against 47.8 us, the long-context one 331 against 335 us (the
// ragged GQA batch, bound by its longest rows rather than by the chip's
// bandwidth, 0.5-0.8 us slower). Over the int8 cache (128-byte slices)
// pairing bit 8 or bit 7 that way was 0.5 us slower than not pairing, so
// only 256-byte slices are paired. When both pool bases are 512-byte
// aligned and the kv head count is even (rows a multiple of 512 bytes), bit
// 8 of every slice address is the kv head's parity. Returns that bit's
// position in the head-group index (head groups per kv head must be a power
// of two), or -1.
inline int decode_xcd_bit(int num_kv_heads, int groups_per_kv_head, int slice_bytes,
                          const void* k_cache, const void* v_cache) {
  if (slice_bytes != 256 || num_kv_heads % 2 != 0) return -1;
  if (groups_per_kv_head <= 0 || (groups_per_kv_head & (groups_per_kv_head - 1)) != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(k_cache) & 511) || (reinterpret_cast<uintptr_t>(v_cache) & 511))
    return -1;
  return __builtin_ctz(groups_per_kv_head);
}

inline DecodePlan plan_decode(int num_seqs, int groups, int max_blocks_per_seq, int block_size,
                              bool fine_ok) {
  const int forced = decode_partition_override();
  if (forced > 0) return {forced >= 2 * kDecodePart ? 8 : 4, forced};
  const long long rows = (long long)num_seqs * groups;
  const long long max_ctx = (long long)max_blocks_per_seq * block_size;
  if (rows >= kNumCUs && max_ctx <= kDecodeWidePart) {
    const int part = (int)((max_ctx + kDecodePart - 1) / kDecodePart * kDecodePart);
    return {8, part};
  }
  for (int part = kDecodeMaxPart; part >= 2 * kDecodePart; part /= 2)
    if (rows * ((max_ctx + part - 1) / part) >= (long long)kDecodeWgsPerCU * kNumCUs)
      return {8, part};
  int part = kDecodePart;
  if (fine_ok)
    while (part > kDecodeFinePart && part > block_size &&
           rows * ((max_ctx + part - 1) / part) < kNumCUs)
      part /= 2;
  return {4, part};
}

hipError_t launch_kv_write(void* k_cache, void* v_cache, const void* key, const void* value,
                           const int32_t* slot_mapping, int64_t num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream);
// whole-block copies: pieces_per_block 16-byte pieces per block, pairs [n, 2] (src, dst)
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int64_t num_pairs, int pieces_per_block, int64_t num_blocks,
                              hipStream_t stream);
// quantise rows of row_elems elements (dtype 0/1/2) to int8 codes and scatter them
hipError_t launch_kv_write_int8(void* k_cache, void* v_cache, const void* key, const void* value,
                                const float* k_scale, const float* v_scale,
                                const int32_t* slot_mapping, int64_t num_tokens, int row_elems,
                                int head_dim, int64_t num_slots, int dtype, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  float scale;
  int num_seqs, num_q_heads, num_kv_heads, head_dim;
  int block_size, max_blocks_per_seq;
  int64_t num_blocks;
  int dtype;
  float* ws_ml;   // [B, Hq, P, 2] (max in log2 units, sum), P = parts at 512 tokens
  float* ws_o;    // [B, Hq, P, D] unnormalised partial outputs
  // int8 cache only: per-kv-head dequantisation scales ([Hkv] fp32)
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  // variants: ALiBi slopes [Hq] fp32 (NULL = none), window (negative = none)
  const float* alibi = nullptr;
  int window_left = -1;
  // fused KV write (launch_write_decode): the pool again, writable, and one
  // new token per sequence: new_key / new_value [B, Hkv, D], slot_mapping [B]
  void* app_k_cache = nullptr;
  void* app_v_cache = nullptr;
  const void* new_key = nullptr;
  const void* new_value = nullptr;
  const int32_t* slot_mapping = nullptr;
  // pairing of whole-context rows (NULL: off): one exchange word per
  // (sequence, query head) in the workspace, and the call's epoch (unique
  // per call, never 0)
  unsigned long long* pair_words = nullptr;
  unsigned long long epoch = 0;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// window / ALiBi variants, q/out of a.dtype (fp16 or bf16)
hipError_t launch_decode_ext(const DecodeArgs& a, hipStream_t stream);
// the decode step's KV write (one new token per sequence) and the decode in
// one launch (fp16 / bf16; an fp32 pool takes the two kernels in turn)
hipError_t launch_write_decode(const DecodeArgs& a, hipStream_t stream);
// the same over an int8 cache: the new rows are quantised with the kv head's
// scales (as the int8 write does), stored and attended in one launch
hipError_t launch_write_decode_int8(const DecodeArgs& a, hipStream_t stream);
// int8 cache (codes), q/out of a.dtype (fp16 or bf16)
hipError_t launch_decode_int8(const DecodeArgs& a, hipStream_t stream);

struct VarlenArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int causal;
  int num_seqs;
  int64_t total_q;
  int num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  int64_t num_blocks;
  int dtype;
  // variants: ALiBi slopes [Hq] fp32 (NULL = none), window (negative = none)
  const float* alibi = nullptr;
  int window_left = -1;
  // split plan (workspace): [S, B, Hkv, 32, 2] (max in log2 units, sum) and
  // [S, B, Hkv, 32, D] unnormalised outputs of the rows of cut tiles
  float* ws_ml = nullptr;
  float* ws_o = nullptr;
};

// Rows per workgroup of the packed prefill kernel (query positions x the
// heads of a GQA group) and keys per KV tile.
constexpr int kVlRows = 128;
constexpr int kVlBN = 64;
// Query tiles per kv head the grid provides: every sequence may end in a
// partial tile.
inline int64_t varlen_tiles(int64_t total_q, int num_seqs, int group) {
  const int bq = kVlRows / group;
  return (total_q + bq - 1) / bq + num_seqs;
}
// Split plan of the packed varlen call with a workspace: a query tile whose
// rows fit one wave (a sequence's last, partial tile) and whose loop runs
// over more key tiles than one chunk is cut into chunks of chunk_tiles key
// tiles, each attended by its own workgroup; chunks hold at least
// kVlChunkMin key tiles, and a tile is cut into at most kVlMaxSplits.
constexpr int kVlChunkMin = 8;
constexpr int kVlRowsWave = 32;   // query rows one wave of the prefill kernel owns
constexpr int kVlMaxSplits = 16;
struct VarlenSplit {
  int chunk_tiles;
  int max_splits;   // S: most chunks any tile of these sizes is cut into
};
inline VarlenSplit plan_varlen_split(int max_blocks_per_seq, int block_size) {
  const long long wmax = ((long long)max_blocks_per_seq * block_size + kVlBN - 1) / kVlBN;
  const long long ck = wmax > (long long)kVlChunkMin * kVlMaxSplits
                           ? (wmax + kVlMaxSplits - 1) / kVlMaxSplits
                           : kVlChunkMin;
  const long long s = (wmax + ck - 1) / ck;
  return {(int)ck, (int)(s > 1 ? s : 1)};
}

hipError_t launch_varlen(const VarlenArgs& a, hipStream_t stream);
hipError_t launch_varlen_ext(const VarlenArgs& a, hipStream_t stream);
hipError_t launch_varlen_split(const VarlenArgs& a, hipStream_t stream);

// the debug build's per-source report words (debug_checks.h) on the current
// device, read and cleared; the default build returns 0 bits
hipError_t debug_take_kv_write(uint32_t* bits);
hipError_t debug_take_decode(uint32_t* bits);
hipError_t debug_take_varlen(uint32_t* bits);

}  // namespace pkv
