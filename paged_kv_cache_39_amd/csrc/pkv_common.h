// Device-side helpers shared by the paged KV-cache kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// 16-byte global load, optionally non-temporal
template <bool NT>
__device__ __forceinline__ u32x4_t load16(const void* p) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

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
// vector loads. `p` must be aligned to the chunk size. NT marks the load
// non-temporal: data streamed once (the KV pool) then does not displace
// reusable lines, and it is not slowed down by dirty lines in the caches.
template <class Ty, int EPL, bool NT = false>
__device__ __forceinline__ Chunk<Ty, EPL> load_chunk(const typename Ty::storage* p) {
  Chunk<Ty, EPL> c;
  constexpr int words = sizeof(c.w) / 4;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(p);
  if constexpr (words % 4 == 0) {
#pragma unroll
    for (int i = 0; i < words; i += 4) {
      const u32x4_t v = load16<NT>(src + i);
      c.w[i] = v[0]; c.w[i + 1] = v[1]; c.w[i + 2] = v[2]; c.w[i + 3] = v[3];
    }
  } else if constexpr (words == 2) {
    const u32x2_t* q = reinterpret_cast<const u32x2_t*>(src);
    const u32x2_t v = NT ? __builtin_nontemporal_load(q) : *q;
    c.w[0] = v[0]; c.w[1] = v[1];
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

// Max / sum with the lane 16 (resp. 32) positions away through gfx950's
// v_permlane16_swap / v_permlane32_swap, without LDS: swapping a register
// with itself leaves every lane i holding its own value and lane
// i ^ 16 (i ^ 32)'s, in either order (measured on the GPU), so the max and
// the sum of the two results are those of the pair.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide reductions and scans of 32-bit integers that stay out of LDS:
// DPP moves within each row of 16 lanes, then the four row results through
// scalar registers (v_readlane). Every lane of the wave must be active; the
// reductions return a wave-uniform value.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int lane_value(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dpp_i<kDppQuadPerm1032>(x);
  x += dpp_i<kDppQuadPerm2301>(x);
  x += dpp_i<kDppRowHalfMirror>(x);
  x += dpp_i<kDppRowMirror>(x);
  return lane_value(x, 0) + lane_value(x, 16) + lane_value(x, 32) + lane_value(x, 48);
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<kDppQuadPerm1032>(x));
  x = max(x, dpp_i<kDppQuadPerm2301>(x));
  x = max(x, dpp_i<kDppRowHalfMirror>(x));
  x = max(x, dpp_i<kDppRowMirror>(x));
  return max(max(lane_value(x, 0), lane_value(x, 16)), max(lane_value(x, 32), lane_value(x, 48)));
}
// Inclusive prefix sum over the lanes: shifts right by 1, 2, 4, 8 within
// each row (lanes whose source lies before the row start add 0), then the
// totals of the preceding rows.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  x += dpp_i<0x111>(x);   // row_shr:1
  x += dpp_i<0x112>(x);   // row_shr:2
  x += dpp_i<0x114>(x);   // row_shr:4
  x += dpp_i<0x118>(x);   // row_shr:8
  const int t0 = lane_value(x, 15), t1 = lane_value(x, 31), t2 = lane_value(x, 47);
  const int lane = (int)__lane_id();
  return x + (lane >= 16 ? t0 : 0) + (lane >= 32 ? t1 : 0) + (lane >= 48 ? t2 : 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Asynchronous 16-byte global -> LDS copies per lane: lane l's 16 bytes land
// at LDS byte address lds + 16*l (lds wave-uniform). Issued through inline
// asm so that the compiler does not track them; the caller waits for
// completion with an explicit s_waitcnt vmcnt before the data is read.
// (Tracked by the compiler, a pending copy into LDS makes it wait for every
// outstanding load before any later LDS access.)

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Source = wave-uniform base + per-lane unsigned 32-bit byte offset.
__device__ __forceinline__ void async_copy16_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  // (the builtin returns int: zero-extend both halves)
  const uint64_t sb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Source = per-lane 64-bit address.
__device__ __forceinline__ void async_copy16_to_lds(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// s_waitcnt encodings (gfx9 family): wait until at most n vector-memory
// operations of this wave are outstanding (lgkm and exp counters untouched)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Barrier without a memory-model fence: this wave's LDS operations complete
// (lgkmcnt 0), then s_barrier. Outstanding global loads and LDS copies are
// not waited for; the compiler is kept from moving memory accesses across.
__device__ __forceinline__ void barrier_lds_ops() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS accesses only. __syncthreads() also waits
// for every outstanding global load (its fence covers global memory), which
// would stall on loads prefetched for the next tile.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Merge weight for a partial with running max m against the merged max
// `mref`, where mref == -inf means "nothing seen yet" (weight 0 for m=-inf).
__device__ __forceinline__ float safe_max_ref(float m) { return m == -INFINITY ? 0.f : m; }

// ---------------------------------------------------------------------------
// matrix cores: v_mfma_f32_16x16x32_{bf16,f16} (mfma) and the k = 16 forms
// v_mfma_f32_16x16x16{bf16_1k,f16} (mfma16)
//   A (16 x K): lane l holds row l%16, k = (K/4)*(l/16) .. +K/4
//   B (K x 16): lane l holds column l%16, k = (K/4)*(l/16) .. +K/4
//   D (16 x 16): lane l, register i holds row 4*(l/16) + i, column l%16
// ---------------------------------------------------------------------------

template <class Ty>
struct Mma;
template <>
struct Mma<BF16> {
  static __device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // k = 16 variant: lane l holds k = 4*(l/16) .. +4 of its row / column
  static __device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <>
struct Mma<F16> {
  static __device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// 16 int8 codes (one 16-byte chunk, byte k = code k) -> the same 16 values
// as Ty (two 16-byte chunks, 8 values each). Exact: |code| <= 127 has at
// most 7 significant bits.
template <class Ty>
__device__ __forceinline__ void widen_i8x16(const u32x4_t c, u32x4_t& lo, u32x4_t& hi);
// fp16: two codes at a time. A code x placed as the byte (x + 128) under the
// exponent bits of 1024.0 gives the fp16 number 1024 + 128 + x exactly (ten
// mantissa bits), so one packed subtraction of 1152 yields x exactly.
template <>
__device__ __forceinline__ void widen_i8x16<F16>(const u32x4_t c, u32x4_t& lo, u32x4_t& hi) {
  uint32_t r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // bytes 0,1 (2,3) of the word into bits 7:0 and 23:16, the rest zero
    const uint32_t p01 = __builtin_amdgcn_perm(0u, c[w], 0x0C010C00u);
    const uint32_t p23 = __builtin_amdgcn_perm(0u, c[w], 0x0C030C02u);
    const f16x2_t bias = {(_Float16)1152.f, (_Float16)1152.f};
    const f16x2_t a = __builtin_bit_cast(f16x2_t, (p01 ^ 0x00800080u) | 0x64006400u) - bias;
    const f16x2_t b = __builtin_bit_cast(f16x2_t, (p23 ^ 0x00800080u) | 0x64006400u) - bias;
    r[2 * w] = __builtin_bit_cast(uint32_t, a);
    r[2 * w + 1] = __builtin_bit_cast(uint32_t, b);
  }
  lo = u32x4_t{r[0], r[1], r[2], r[3]};
  hi = u32x4_t{r[4], r[5], r[6], r[7]};
}
template <>
__device__ __forceinline__ void widen_i8x16<BF16>(const u32x4_t c, u32x4_t& lo, u32x4_t& hi) {
  using Ty = BF16;
  uint32_t r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = c[w];
    r[2 * w] = Mma<Ty>::pack((float)(int8_t)(x & 0xFFu), (float)(int8_t)((x >> 8) & 0xFFu));
    r[2 * w + 1] = Mma<Ty>::pack((float)(int8_t)((x >> 16) & 0xFFu), (float)(int8_t)(x >> 24));
  }
  lo = u32x4_t{r[0], r[1], r[2], r[3]};
  hi = u32x4_t{r[4], r[5], r[6], r[7]};
}

// int8 code of x under a per-kv-head scale s: clamp(rne(x / s), -127, 127),
// the quotient an IEEE binary32 division. quantize16: 16 consecutive
// elements of a row -> 16 codes (byte k = code k).
__device__ __forceinline__ uint32_t quantize4(float a, float b, float c, float d, float s) {
  auto q = [s](float x) -> uint32_t {
    const float r = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.f), 127.f);
    return (uint32_t)(int32_t)r & 0xFFu;
  };
  return q(a) | (q(b) << 8) | (q(c) << 16) | (q(d) << 24);
}

template <class Ty>
__device__ __forceinline__ uint4 quantize16(const typename Ty::storage* x, float s) {
  const Chunk<Ty, 16> c = load_chunk<Ty, 16>(x);
  uint4 r;
  r.x = quantize4(c.get(0), c.get(1), c.get(2), c.get(3), s);
  r.y = quantize4(c.get(4), c.get(5), c.get(6), c.get(7), s);
  r.z = quantize4(c.get(8), c.get(9), c.get(10), c.get(11), s);
  r.w = quantize4(c.get(12), c.get(13), c.get(14), c.get(15), s);
  return r;
}

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i supplies the address of a row R_i of four 16-bit elements; lane
// 4a+b receives (R_a[b], R_{a+4}[b], R_{a+8}[b], R_{a+12}[b]).
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(reinterpret_cast<uintptr_t>(lds_ptr)));
  return __builtin_bit_cast(u32x2_t, v);
}

}  // namespace pkv
