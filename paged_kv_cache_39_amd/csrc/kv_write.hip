// KV write scatter: new K/V token rows are copied into the block pool at the
// row named by slot_mapping ("model-infer-kvcache" skill page, section 3.3:
// the write op is addressed by slot; section 3.1: slot = block * block_size +
// offset, so with the pool viewed as [num_blocks * block_size, Hkv * D] rows
// the slot is the row index).
//
// Dtype-agnostic: rows are moved as 16-byte pieces, so the copy is bit-exact.
// One thread per 16-byte piece; consecutive threads cover consecutive bytes
// of a row, so both the read of key/value and the write into the pool are
// fully coalesced.

#include "pkv_launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(uint4* __restrict__ k_cache,
                                                       uint4* __restrict__ v_cache,
                                                       const uint4* __restrict__ key,
                                                       const uint4* __restrict__ value,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int64_t num_pieces, int pieces_per_row,
                                                       int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= num_pieces) return;
  const int64_t t = gid / pieces_per_row;
  const int piece = (int)(gid - t * pieces_per_row);
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t dst = (int64_t)slot * pieces_per_row + piece;
  const uint4 kk = key[gid];
  const uint4 vv = value[gid];
  k_cache[dst] = kk;
  v_cache[dst] = vv;
}

hipError_t launch_kv_write(void* k_cache, void* v_cache, const void* key, const void* value,
                           const int32_t* slot_mapping, int64_t num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream) {
  const int pieces_per_row = row_bytes / 16;
  const int64_t num_pieces = num_tokens * pieces_per_row;
  const int threads = 256;
  const int64_t blocks = (num_pieces + threads - 1) / threads;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     slot_mapping, num_pieces, pieces_per_row, num_slots);
  return hipGetLastError();
}

}  // namespace pkv
