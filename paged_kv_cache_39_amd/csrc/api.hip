// C-ABI entry points of libpagedkv.so: argument validation, workspace
// layout and dispatch to the HIP launchers. Declared in include/pagedkv.h.
//
// Every check here runs before any HIP call, so an invalid call returns its
// status without touching the device (and works on a machine with no GPU).

#include <initializer_list>
#include <limits.h>

#include <atomic>
#include <mutex>

#include "pagedkv.h"
#include "debug_checks.h"
#include "pkv_launch.h"

namespace pkv {
KernelTiming& pending_timing() {
  thread_local KernelTiming t;
  return t;
}
int& decode_partition_override() {
  thread_local int tokens = 0;
  return tokens;
}
}  // namespace pkv

int pkv_decode_partition_override(int32_t partition_tokens) {
  if (partition_tokens != 0 && partition_tokens != 512 && partition_tokens != 1024 &&
      partition_tokens != 2048 && partition_tokens != 4096)
    return PKV_ERR_SHAPE;
  pkv::decode_partition_override() = partition_tokens;
  return PKV_OK;
}

int pkv_time_next_kernel(void* start_event, void* stop_event) {
  pkv::KernelTiming& t = pkv::pending_timing();
  t.start = static_cast<hipEvent_t>(start_event);
  t.stop = static_cast<hipEvent_t>(stop_event);
  return PKV_OK;
}

namespace {

bool valid_dtype(int32_t d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
int elem_bytes(int32_t d) { return d == PKV_F32 ? 4 : 2; }
bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_block_size(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// Common pool checks; returns PKV_OK or the first failing status.
int check_pool(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks) {
  if (num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_blocks > (int64_t)INT32_MAX / block_size) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// The kernels move tensor data (queries, outputs, new rows, the pool) in
// 16-byte pieces: every such pointer must be 16-byte aligned, as every
// device allocator's blocks are.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;
  return true;
}

int decode_num_parts(int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                     int32_t block_size) {
  // the finest split any launch plan for these sizes uses
  const bool fine = pkv::decode_fine_ok(num_seqs, num_q_heads, max_blocks_per_seq, block_size);
  return pkv::decode_parts(max_blocks_per_seq, block_size,
                           fine ? pkv::kDecodeFinePart : pkv::kDecodePart);
}

// Epoch of a decode call that may pair rows: unique per call within the
// process, never 0 (the value a paired row's word holds between calls).
unsigned long long next_pair_epoch() {
  static std::atomic<unsigned long long> counter{0};
  return counter.fetch_add(1, std::memory_order_relaxed) + 1;
}

// Points the decode arguments at the workspace: [B, Hq, P, 2] (max, sum),
// [B, Hq, P, D] partial outputs, P = the finest split, then (when P >= 2)
// [B, Hq] 64-bit exchange words for paired rows, which use two slots per
// (sequence, head) of the partials.
void set_decode_workspace(pkv::DecodeArgs& a, void* workspace, int32_t max_blocks_per_seq) {
  const int parts = decode_num_parts(a.num_seqs, a.num_q_heads, max_blocks_per_seq, a.block_size);
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads * parts;
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_o = workspace ? a.ws_ml + rows * 2 : nullptr;
  if (workspace && parts >= 2) {
    a.pair_words = reinterpret_cast<unsigned long long*>(a.ws_o + rows * a.head_dim);
    a.epoch = next_pair_epoch();
  }
}

}  // namespace

// Split-KV scratch of the no-allocation decode step: one copy per GPU the
// library runs on (the code object's global, allocated when the runtime
// loads the library's kernels onto a device and held until the process
// ends). In host code `scratch` names a host-side stand-in; the device
// address of a GPU's copy comes from hipGetSymbolAddress with that GPU
// current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The copy of `scratch` on the device that `stream` launches on (the current
// device for the null stream), looked up once per device with that device
// current; NULL if the runtime reports an error.
void* scratch_for_stream(hipStream_t stream) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (err != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

// The fused decode step; with `noalloc` the partials go to the library's
// scratch instead of the caller's workspace.
static int write_decode_impl(void* out, const void* q, void* k_cache, void* v_cache,
                             const void* key, const void* value, const int32_t* slot_mapping,
                             const int32_t* block_table, const int32_t* context_lens,
                             int32_t block_size, float scale, int32_t num_seqs,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                             void* workspace, size_t workspace_bytes, void* stream,
                             bool noalloc) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !key || !value || !slot_mapping || !block_table ||
      !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache, key, value})) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_blocks_per_seq, block_size);
  if (noalloc) {
    // the split-KV partials go to this device's copy of `scratch`
    if (need > kScratchBytes) return PKV_ERR_SCRATCH;
    if (need > 0) {
      workspace = scratch_for_stream(static_cast<hipStream_t>(stream));
      if (!workspace) return PKV_ERR_HIP;
      workspace_bytes = kScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  set_decode_workspace(a, workspace, max_blocks_per_seq);
  a.app_k_cache = k_cache;
  a.app_v_cache = v_cache;
  a.new_key = key;
  a.new_value = value;
  a.slot_mapping = slot_mapping;
  hipError_t err = pkv::launch_write_decode(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

static int varlen_impl(void* out, const void* q, const int32_t* cu_seqlens_q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int causal,
                           int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                           void* stream, const float* alibi, int32_t window_left, bool ext,
                           void* workspace = nullptr, size_t workspace_bytes = 0,
                           bool split = false) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (dtype == PKV_F32) return PKV_ERR_DTYPE;  // matrix-core path: 16-bit inputs only
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 128) return PKV_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (total_q > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (!out || !q || !cu_seqlens_q || !k_cache || !v_cache || !block_table || !seq_lens)
    return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PKV_ERR_UNSUPPORTED;
  // the one-dimensional grid: (query tiles [+ split chunk slots]) x kv heads
  const int64_t splits =
      split ? pkv::plan_varlen_split(max_blocks_per_seq, block_size).max_splits : 1;
  // (the plain call also has one workgroup per (sequence, kv head) for the
  // sequences whose rows fit one 16-row tile)
  const int64_t wgs =
      (pkv::varlen_tiles(total_q, num_seqs, num_q_heads / num_kv_heads) * splits +
       (split || ext ? 0 : num_seqs)) * num_kv_heads;
  if (wgs > INT32_MAX) return PKV_ERR_SHAPE;
  if (split) {
    const size_t need = paged_attention_varlen_workspace_size(
        num_seqs, num_kv_heads, head_dim, max_blocks_per_seq, block_size);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  }

  pkv::VarlenArgs a;
  a.out = out;
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.causal = causal ? 1 : 0;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  a.alibi = alibi;
  a.window_left = window_left < 0 ? -1 : window_left;
  if (split && workspace) {
    const int64_t rows = (int64_t)pkv::plan_varlen_split(max_blocks_per_seq, block_size).max_splits *
                         num_seqs * num_kv_heads * pkv::kVlRowsWave;
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_o = a.ws_ml + rows * 2;
  }
  hipError_t err = split ? pkv::launch_varlen_split(a, static_cast<hipStream_t>(stream))
                   : ext ? pkv::launch_varlen_ext(a, static_cast<hipStream_t>(stream))
                         : pkv::launch_varlen(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case PKV_ERR_DTYPE: return "dtype code unknown or not accepted by this call";
    case PKV_ERR_UNSUPPORTED: return "head_dim, block_size or GQA group outside the supported set, or a tensor pointer not 16-byte aligned";
    case PKV_ERR_WORKSPACE: return "decode workspace missing or too small";
    case PKV_ERR_HIP: return "the HIP runtime rejected a launch";
    case PKV_ERR_NO_BLOCKS: return "not enough free cache blocks";
    case PKV_ERR_PENDING_COPY: return "pending block copies must be taken and applied first";
    case PKV_ERR_SCRATCH:
      return "the split-KV partials need more than the no-allocation call's scratch";
    default: return "unknown status";
  }
}

int pkv_debug_checks(void) { return pkv::kDbgBuild ? 1 : 0; }

int pkv_debug_take_errors(uint32_t* bits) {
  if (!bits) return PKV_ERR_NULL;
  *bits = 0;
  if (!pkv::kDbgBuild) return PKV_ERR_UNSUPPORTED;
  if (hipDeviceSynchronize() != hipSuccess) return PKV_ERR_HIP;
  uint32_t all = 0;
  for (auto take : {pkv::debug_take_kv_write, pkv::debug_take_decode, pkv::debug_take_varlen}) {
    uint32_t b = 0;
    if (take(&b) != hipSuccess) return PKV_ERR_HIP;
    all |= b;
  }
  *bits = all;
  return PKV_OK;
}

int32_t pkv_decode_partition_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size, int32_t dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_q_heads % num_kv_heads != 0 || !supported_block_size(block_size))
    return 0;
  if (dtype == PKV_F32) return pkv::kDecodePart;
  const int group = num_q_heads / num_kv_heads;
  int hpw = 1;
  for (int c = 16; c >= 1; --c)
    if (group % c == 0) { hpw = c; break; }
  return pkv::plan_decode(num_seqs, num_q_heads / hpw, max_blocks_per_seq, block_size,
                          pkv::decode_fine_ok(num_seqs, num_q_heads, max_blocks_per_seq,
                                              block_size))
      .part_tokens;
}

int paged_kv_write(void* k_cache, void* v_cache, const void* key, const void* value,
                   const int32_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
                   void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !key || !value || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16({k_cache, v_cache, key, value})) return PKV_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
  if (row_bytes > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_tokens > INT64_MAX / (row_bytes / 16)) return PKV_ERR_SHAPE;
  hipError_t err = pkv::launch_kv_write(k_cache, v_cache, key, value, slot_mapping, num_tokens,
                                        (int)row_bytes, num_blocks * block_size,
                                        static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// Workspace layout (set_decode_workspace): [B, Hq, P, 2] fp32 (max, sum),
// [B, Hq, P, D] fp32 partial outputs, P = partitions at the finest split,
// then [B, Hq] 64-bit exchange words of paired rows.
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return 0;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return 0;
  const int64_t parts = decode_num_parts(num_seqs, num_q_heads, max_blocks_per_seq, block_size);
  if (parts <= 1) return 0;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * parts;
  return (size_t)(rows * 2 + rows * head_dim) * sizeof(float) +
         (size_t)num_seqs * num_q_heads * sizeof(unsigned long long);
}

int paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* context_lens,
                           int32_t block_size, float scale, int32_t num_seqs,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens) return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_blocks_per_seq, block_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  set_decode_workspace(a, workspace, max_blocks_per_seq);
  hipError_t err = pkv::launch_decode(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_write_decode(void* out, const void* q, void* k_cache, void* v_cache,
                          const void* key, const void* value, const int32_t* slot_mapping,
                          const int32_t* block_table, const int32_t* context_lens,
                          int32_t block_size, float scale, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return write_decode_impl(out, q, k_cache, v_cache, key, value, slot_mapping, block_table,
                           context_lens, block_size, scale, num_seqs, num_q_heads, num_kv_heads,
                           head_dim, max_blocks_per_seq, num_blocks, dtype, workspace,
                           workspace_bytes, stream, false);
}

int paged_kv_write_decode_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                  const void* key, const void* value,
                                  const int32_t* slot_mapping, const int32_t* block_table,
                                  const int32_t* context_lens, int32_t block_size, float scale,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t dtype, void* stream) {
  return write_decode_impl(out, q, k_cache, v_cache, key, value, slot_mapping, block_table,
                           context_lens, block_size, scale, num_seqs, num_q_heads, num_kv_heads,
                           head_dim, max_blocks_per_seq, num_blocks, dtype, nullptr, 0, stream,
                           true);
}

int paged_attention_varlen(void* out, const void* q, const int32_t* cu_seqlens_q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int causal,
                           int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                           void* stream) {
  return varlen_impl(out, q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, causal,
                     num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, dtype, stream, nullptr, -1, false);
}

int paged_attention_varlen_ex(void* out, const void* q, const int32_t* cu_seqlens_q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int causal,
                              const float* alibi_slopes, int32_t window_left, int32_t num_seqs,
                              int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t dtype, void* stream) {
  return varlen_impl(out, q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, causal,
                     num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, dtype, stream, alibi_slopes, window_left,
                     true);
}

// Workspace layout of the split varlen call: [S, B, Hkv, 32, 2] fp32 (max,
// sum) and [S, B, Hkv, 32, D] fp32 partial outputs of the rows (at most one
// wave's 32) of each sequence's last query tile per kv head; S = the most
// chunks a tile of these sizes is cut into.
size_t paged_attention_varlen_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0) return 0;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return 0;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return 0;
  const int64_t s = pkv::plan_varlen_split(max_blocks_per_seq, block_size).max_splits;
  if (s <= 1) return 0;
  const int64_t rows = s * num_seqs * num_kv_heads * pkv::kVlRowsWave;
  return (size_t)(rows * (2 + head_dim)) * sizeof(float);
}

int paged_attention_varlen_split(void* out, const void* q, const int32_t* cu_seqlens_q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens, int causal,
                                 int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return varlen_impl(out, q, cu_seqlens_q, k_cache, v_cache, block_table, seq_lens, causal,
                     num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, num_blocks, dtype, stream, nullptr, -1, false, workspace,
                     workspace_bytes, true);
}

int paged_attention_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* context_lens,
                              int32_t block_size, float scale, const float* alibi_slopes,
                              int32_t window_left, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_DTYPE;  // matrix-core path
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens) return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_blocks_per_seq, block_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  set_decode_workspace(a, workspace, max_blocks_per_seq);
  a.alibi = alibi_slopes;
  a.window_left = window_left < 0 ? -1 : window_left;
  hipError_t err = pkv::launch_decode_ext(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_write_int8(void* k_cache, void* v_cache, const void* key, const void* value,
                        const float* k_scale, const float* v_scale, const int32_t* slot_mapping,
                        int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream) {
  if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !key || !value || !k_scale || !v_scale || !slot_mapping)
    return PKV_ERR_NULL;
  if (!aligned16({k_cache, v_cache, key, value})) return PKV_ERR_UNSUPPORTED;
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
  if (row_elems * 4 > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_tokens > INT64_MAX / (row_elems / 16)) return PKV_ERR_SHAPE;
  hipError_t err = pkv::launch_kv_write_int8(k_cache, v_cache, key, value, k_scale, v_scale,
                                             slot_mapping, num_tokens, (int)row_elems, head_dim,
                                             num_blocks * block_size, dtype,
                                             static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attention_decode_int8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const float* k_scale, const float* v_scale,
                                const int32_t* block_table, const int32_t* context_lens,
                                int32_t block_size, float scale, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_DTYPE;  // matrix-core path
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table ||
      !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache})) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_blocks_per_seq, block_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  set_decode_workspace(a, workspace, max_blocks_per_seq);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  hipError_t err = pkv::launch_decode_int8(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_write_decode_int8(void* out, const void* q, void* k_cache, void* v_cache,
                               const void* key, const void* value, const float* k_scale,
                               const float* v_scale, const int32_t* slot_mapping,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t block_size, float scale, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int64_t num_blocks, int32_t dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_DTYPE;  // matrix-core path
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || num_q_heads > 65535) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !key || !value || !k_scale || !v_scale ||
      !slot_mapping || !block_table || !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16({out, q, k_cache, v_cache, key, value})) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, head_dim,
                                                            max_blocks_per_seq, block_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;

  pkv::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.scale = scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.dtype = dtype;
  set_decode_workspace(a, workspace, max_blocks_per_seq);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.app_k_cache = k_cache;
  a.app_v_cache = v_cache;
  a.new_key = key;
  a.new_value = value;
  a.slot_mapping = slot_mapping;
  hipError_t err = pkv::launch_write_decode_int8(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t dtype, void* stream) {
  if (!valid_dtype(dtype) && dtype != PKV_I8) return PKV_ERR_DTYPE;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  int st = check_pool(num_kv_heads, head_dim, block_size, num_blocks);
  if (st != PKV_OK) return st;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_ERR_NULL;
  if (!aligned16({k_cache, v_cache})) return PKV_ERR_UNSUPPORTED;
  const int eb = dtype == PKV_I8 ? 1 : elem_bytes(dtype);
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * eb;
  if (block_bytes / 16 > INT32_MAX) return PKV_ERR_SHAPE;
  if (num_pairs > INT64_MAX / (block_bytes / 16)) return PKV_ERR_SHAPE;
  hipError_t err = pkv::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs,
                                           (int)(block_bytes / 16), num_blocks,
                                           static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
