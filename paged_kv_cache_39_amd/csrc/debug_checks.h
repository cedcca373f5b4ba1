// Opt-in device-side reports of caller contract violations.
//
// Block ids, lengths, cu_seqlens and slots live in device memory, so the
// host cannot check them, and on the pages they are the caller's contract
// (an out-of-range index crashes or returns garbage). The kernels keep such
// inputs in bounds on their own: an out-of-range block id reads block 0 or is
// masked, a length is clamped to what the block table can address, cu_seqlens
// are clamped to [0, total_q], an out-of-pool slot or copy pair is skipped.
// That gives the caller no signal. Built with PKV_DEBUG_CHECKS=1 (the
// libpagedkv_debug.so build), every such clamp also ORs a bit into a device
// word that the host reads and clears through pkv_debug_take_errors; the
// default build compiles every report out.
//
// The word is a file-scope device variable, one per translation unit (the
// library is not built with relocatable device code), so each kernel source
// defines its own reader with PKV_DBG_TAKE_FN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef PKV_DEBUG_CHECKS
#define PKV_DEBUG_CHECKS 0
#endif

namespace pkv {
// bit values (the same numbers as the PKV_DBG_* constants of pagedkv.h)
constexpr uint32_t kDbgBlockId = 1u;     // a block id of a used block outside [0, num_blocks)
constexpr uint32_t kDbgLength = 2u;      // a context / KV length < 0 or beyond the block table
constexpr uint32_t kDbgCuSeqlens = 4u;   // cu_seqlens_q not 0 .. total_q, non-decreasing
constexpr uint32_t kDbgSlot = 8u;        // a slot >= num_blocks * block_size
constexpr uint32_t kDbgCopyPair = 16u;   // a copy pair with an id outside [0, num_blocks)
constexpr bool kDbgBuild = PKV_DEBUG_CHECKS != 0;
}  // namespace pkv

#if PKV_DEBUG_CHECKS
static __device__ uint32_t pkv_dbg_word;
// (a vector atomic from every lane where `cond` holds)
#define PKV_DBG_REPORT(cond, bit)                                                     \
  do {                                                                               \
    if (cond)                                                                        \
      __hip_atomic_fetch_or(&pkv_dbg_word, (bit), __ATOMIC_RELAXED,                  \
                            __HIP_MEMORY_SCOPE_AGENT);                               \
  } while (0)
// hipError_t name(uint32_t* bits): this file's word on the current device,
// then cleared (synchronous copies; the caller has synchronised the device)
#define PKV_DBG_TAKE_FN(name)                                                        \
  hipError_t name(uint32_t* bits) {                                                  \
    uint32_t v = 0;                                                                  \
    const uint32_t zero = 0;                                                         \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(pkv_dbg_word), sizeof v, 0,    \
                                       hipMemcpyDeviceToHost);                       \
    if (e == hipSuccess)                                                             \
      e = hipMemcpyToSymbol(HIP_SYMBOL(pkv_dbg_word), &zero, sizeof zero, 0,         \
                            hipMemcpyHostToDevice);                                  \
    *bits = e == hipSuccess ? v : 0u;                                                \
    return e;                                                                        \
  }
#else
// (the condition is named, unevaluated, so that its operands count as used)
#define PKV_DBG_REPORT(cond, bit) \
  do {                            \
    (void)sizeof((cond) && (bit)); \
  } while (0)
#define PKV_DBG_TAKE_FN(name)       \
  hipError_t name(uint32_t* bits) { \
    *bits = 0u;                     \
    return hipSuccess;              \
  }
#endif
