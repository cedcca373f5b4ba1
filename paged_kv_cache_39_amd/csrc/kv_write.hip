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

#include "debug_checks.h"
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
  // the new rows are read together with their slot (one round trip), also
  // for a skipped slot: those reads stay inside key / value
  const uint4 kk = key[gid];
  const uint4 vv = value[gid];
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) {
    PKV_DBG_REPORT(slot >= 0 && piece == 0, kDbgSlot);   // (a negative slot is a skip)
    return;
  }
  const int64_t dst = (int64_t)slot * pieces_per_row + piece;
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
  launch_kernel(kv_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     slot_mapping, num_pieces, pieces_per_row, num_slots);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block copies (the device half of copy-on-write): one thread per 16-byte
// piece of a block; pair i copies block pairs[2i] to block pairs[2i+1] in
// both pools. Pairs naming a block outside the pool are skipped.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t num_pieces, int pieces_per_block,
                                                          int64_t num_blocks) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= num_pieces) return;
  const int64_t i = gid / pieces_per_block;
  const int piece = (int)(gid - i * pieces_per_block);
  const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
    PKV_DBG_REPORT(piece == 0, kDbgCopyPair);
    return;
  }
  const int64_t s = (int64_t)src * pieces_per_block + piece;
  const int64_t d = (int64_t)dst * pieces_per_block + piece;
  const uint4 kk = k_cache[s];
  const uint4 vv = v_cache[s];
  k_cache[d] = kk;
  v_cache[d] = vv;
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs,
                              int64_t num_pairs, int pieces_per_block, int64_t num_blocks,
                              hipStream_t stream) {
  const int64_t num_pieces = num_pairs * pieces_per_block;
  const int threads = 256;
  launch_kernel(copy_blocks_kernel, dim3((unsigned)((num_pieces + threads - 1) / threads)),
                     dim3(threads), 0, stream, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), pairs, num_pieces, pieces_per_block,
                     num_blocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int8 cache write: quantise, then scatter by slot. Code of element x of kv
// head h: clamp(rne(x / scale[h]), -127, 127), the quotient an IEEE float32
// division (the int8 KV-cache entry points in include/pagedkv.h state the
// reading). One thread per 16 elements of a token row, i.e. 16 codes = one
// 16-byte store into the pool.
// ---------------------------------------------------------------------------

template <class Ty>
__global__ __launch_bounds__(256) void kv_write_int8_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const typename Ty::storage* __restrict__ key, const typename Ty::storage* __restrict__ value,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ slot_mapping, int64_t num_pieces, int pieces_per_row,
    int pieces_per_head, int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= num_pieces) return;
  const int64_t t = gid / pieces_per_row;
  const int piece = (int)(gid - t * pieces_per_row);
  // codes are made while the slot is read (one round trip for both)
  const int head = piece / pieces_per_head;
  const uint4 kq = quantize16<Ty>(key + gid * 16, k_scale[head]);
  const uint4 vq = quantize16<Ty>(value + gid * 16, v_scale[head]);
  const int32_t slot = slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= num_slots) {
    PKV_DBG_REPORT(slot >= 0 && piece == 0, kDbgSlot);
    return;
  }
  const int64_t dst = (int64_t)slot * pieces_per_row + piece;
  k_cache[dst] = kq;
  v_cache[dst] = vq;
}

hipError_t launch_kv_write_int8(void* k_cache, void* v_cache, const void* key, const void* value,
                                const float* k_scale, const float* v_scale,
                                const int32_t* slot_mapping, int64_t num_tokens, int row_elems,
                                int head_dim, int64_t num_slots, int dtype, hipStream_t stream) {
  const int pieces_per_row = row_elems / 16;
  const int pieces_per_head = head_dim / 16;
  const int64_t num_pieces = num_tokens * pieces_per_row;
  const int threads = 256;
  const dim3 grid((unsigned)((num_pieces + threads - 1) / threads));
  uint4* kc = static_cast<uint4*>(k_cache);
  uint4* vc = static_cast<uint4*>(v_cache);
  if (dtype == 0) {
    launch_kernel(kv_write_int8_kernel<F32>, grid, dim3(threads), 0, stream, kc, vc,
                       static_cast<const float*>(key), static_cast<const float*>(value), k_scale,
                       v_scale, slot_mapping, num_pieces, pieces_per_row, pieces_per_head,
                       num_slots);
  } else if (dtype == 1) {
    launch_kernel(kv_write_int8_kernel<F16>, grid, dim3(threads), 0, stream, kc, vc,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       k_scale, v_scale, slot_mapping, num_pieces, pieces_per_row,
                       pieces_per_head, num_slots);
  } else {
    launch_kernel(kv_write_int8_kernel<BF16>, grid, dim3(threads), 0, stream, kc, vc,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       k_scale, v_scale, slot_mapping, num_pieces, pieces_per_row,
                       pieces_per_head, num_slots);
  }
  return hipGetLastError();
}

PKV_DBG_TAKE_FN(debug_take_kv_write)

}  // namespace pkv
