// Internal launcher declarations (host side). Sizes are validated by the
// C-ABI entry points before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_common.h"

namespace pkv {

// Tokens per split-KV partition of the decode path.
constexpr int kDecodePart = 512;

hipError_t launch_kv_write(void* k_cache, void* v_cache, const void* key, const void* value,
                           const int32_t* slot_mapping, int64_t num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream);

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
  float* ws_ml;  // [B, Hq, P, 2] (max in log2 units, sum)
  float* ws_o;   // [B, Hq, P, D] unnormalised partial outputs
  int num_parts; // P
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

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
};

hipError_t launch_varlen(const VarlenArgs& a, hipStream_t stream);

}  // namespace pkv
