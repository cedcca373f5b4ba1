// Device-side helpers shared by the paged KV-cache kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// element types: storage form and exact widening to fp32
// ---------------------------------------------------------------------------

struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// round-to-nearest-even fp32 -> bf16 bits (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Widen `n` packed storage words holding 32/bits-per-elem elements each.
template <class Ty, int EPL>
struct Chunk;

// EPL elements of a 16-bit type live in EPL/2 dwords.
template <int EPL>
struct Chunk<BF16, EPL> {
  uint32_t w[EPL / 2];
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <int EPL>
struct Chunk<F16, EPL> {
  uint32_t w[EPL / 2];
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? f16_hi(w[e >> 1]) : f16_lo(w[e >> 1]);
  }
};
template <int EPL>
struct Chunk<F32, EPL> {
  uint32_t w[EPL];
  __device__ __forceinline__ float get(int e) const { return __uint_as_float(w[e]); }
};

// Load one lane's chunk (EPL consecutive elements) with 16-byte / 8-byte
// vector loads. `p` must be aligned to the chunk size.
template <class Ty, int EPL>
__device__ __forceinline__ Chunk<Ty, EPL> load_chunk(const typename Ty::storage* p) {
  Chunk<Ty, EPL> c;
  constexpr int words = sizeof(c.w) / 4;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(p);
  if constexpr (words % 4 == 0) {
#pragma unroll
    for (int i = 0; i < words; i += 4) {
      uint4 v = *reinterpret_cast<const uint4*>(src + i);
      c.w[i] = v.x; c.w[i + 1] = v.y; c.w[i + 2] = v.z; c.w[i + 3] = v.w;
    }
  } else if constexpr (words == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(src);
    c.w[0] = v.x; c.w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < words; ++i) c.w[i] = src[i];
  }
  return c;
}

template <class Ty>
__device__ __forceinline__ typename Ty::storage from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<F32>(float f) { return f; }
template <>
__device__ __forceinline__ uint16_t from_f32<F16>(float f) { return (uint16_t)f32_to_f16_bits(f); }
template <>
__device__ __forceinline__ uint16_t from_f32<BF16>(float f) { return (uint16_t)f32_to_bf16_bits(f); }

template <class Ty>
__device__ __forceinline__ float to_f32(typename Ty::storage s);
template <>
__device__ __forceinline__ float to_f32<F32>(float s) { return s; }
template <>
__device__ __forceinline__ float to_f32<F16>(uint16_t s) { return (float)__builtin_bit_cast(_Float16, s); }
template <>
__device__ __forceinline__ float to_f32<BF16>(uint16_t s) { return __uint_as_float((uint32_t)s << 16); }

// ---------------------------------------------------------------------------
// cross-lane reductions
// ---------------------------------------------------------------------------

// DPP controls (GFX9 encoding)
constexpr int kDppQuadPerm1032 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadPerm2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of 16 lanes; every lane receives its group's sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadPerm1032>(x);
  x += dpp<kDppQuadPerm2301>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppQuadPerm1032>(x));
  x = fmaxf(x, dpp<kDppQuadPerm2301>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge weight for a partial with running max m against the merged max
// `mref`, where mref == -inf means "nothing seen yet" (weight 0 for m=-inf).
__device__ __forceinline__ float safe_max_ref(float m) { return m == -INFINITY ? 0.f : m; }

}  // namespace pkv
