// C-ABI layer of libinkattn: argument validation, split-count heuristic,
// workspace sizing, and dispatch to the kernel launchers.  Declarations and
// the meaning of every argument are in include/inkattn.h.
#include "inkattn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>

#include "launch.h"

using inkattn::AttnShape;

namespace {

constexpr int kDefaultCUs = 256;            // MI355X, when no device answers the query
constexpr int kMaxDecodeQueries = inkattn::kMaxMqTokens;  // query tokens per sequence in one decode call

// Compute units of the current device: the split heuristic aims at about one
// (sequence, kv-head, split) work-group per CU.  Read once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kDefaultCUs;
  if (dev < kMaxDevices) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    n = kDefaultCUs;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// A cache scale must be positive and finite, with a finite reciprocal.
bool fp8_scale_ok(float s) { return s > 0.0f && std::isfinite(s) && std::isfinite(1.0f / s); }

inkattn_status_t check_desc(const inkattn_attn_desc_t* d) {
  if (!d) return INKATTN_EINVAL;
  if (d->dtype != INKATTN_FP32 && d->dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (d->head_dim != 128 || d->block_size != 128) return INKATTN_ENOTSUP;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1) return INKATTN_EINVAL;
  if (d->num_q_heads % d->num_kv_heads != 0) return INKATTN_EINVAL;
  if (d->num_q_heads / d->num_kv_heads > 16) return INKATTN_ENOTSUP;
  if (d->window < 0 || d->bias_len < 1) return INKATTN_EINVAL;
  return INKATTN_OK;
}

AttnShape shape_of(const inkattn_attn_desc_t* d) {
  return AttnShape{d->dtype, d->num_q_heads, d->num_kv_heads, d->window, d->bias_len};
}

// Number of 128-token blocks that the attended key range of the longest
// sequence can touch (its q_len query tokens together see window + q_len - 1
// keys).
int64_t blocks_in_range(const inkattn_attn_desc_t* d, int64_t max_seq_len, int64_t max_q_len) {
  const int64_t all = (max_seq_len + 127) / 128;
  if (d->window == 0) return all;
  const int64_t want = (int64_t)d->window + max_q_len - 1;
  const int64_t keys = want < max_seq_len ? want : max_seq_len;
  const int64_t span = (keys + 127) / 128 + 1;   // +1: range need not be block aligned
  return span < all ? span : all;
}

// Splits so that the (sequence, kv-head, column tile, split) work-groups
// about fill the GPU once, never more splits than blocks in the range.
int32_t auto_splits(const inkattn_attn_desc_t* d, int32_t num_seqs, int32_t max_seq_len,
                    int32_t max_q_len = 1) {
  const int64_t pairs = (int64_t)num_seqs * d->num_kv_heads *
                        inkattn::decode_groups_per_pair(d->dtype, d->num_q_heads / d->num_kv_heads,
                                                        max_q_len);
  const int64_t nblk = blocks_in_range(d, max_seq_len, max_q_len);
  if (pairs <= 0 || nblk <= 0) return 1;
  const int64_t target = device_cus();
  int64_t s = (target + pairs - 1) / pairs;
  if (s > nblk) s = nblk;
  if (s < 1) s = 1;
  return (int32_t)s;
}

// The kernels address the [Hq][R] bias table with 32-bit byte offsets.
bool bias_table_too_large(const inkattn_attn_desc_t* d) {
  const uint64_t elem = d->dtype == INKATTN_BF16 ? 2 : 4;
  return (uint64_t)d->num_q_heads * (uint64_t)d->bias_len * elem >= (1ull << 31);
}

// The decode grid is one dimension of (split, kv-head, sequence) x column
// tile work-groups, with 32-bit indices inside the kernel; the merge grid is
// one dimension of (query token, q-head) work-groups.
bool decode_grid_too_large(const inkattn_attn_desc_t* d, int64_t num_seqs, int64_t num_tokens,
                           int64_t splits, int32_t max_q_len) {
  const int64_t rest = splits * d->num_kv_heads * num_seqs;
  const int64_t n_ct = inkattn::decode_column_tiles(d->num_q_heads / d->num_kv_heads, max_q_len);
  if ((int64_t)d->num_q_heads * num_tokens > 0x7fffffffLL) return true;
  return (rest + 7) / 8 * 8 * n_ct > 0x7fffffffLL;   // (covers the LDS-staged grid, rest)
}

inkattn_status_t from_hip(hipError_t e) { return e == hipSuccess ? INKATTN_OK : INKATTN_EHIP; }

// Scratch of inkattn_relattn_decode_noalloc: each GPU the library runs on
// holds its own copy of this array until the process ends.
__device__ __align__(256) unsigned char scratch[INKATTN_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on the current device, taken once per
// device with that device current (nullptr if the runtime cannot say).
void* scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
    return nullptr;
  addr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" {

const char* inkattn_status_string(int32_t status) {
  switch (status) {
    case INKATTN_OK: return "ok";
    case INKATTN_EINVAL: return "invalid argument";
    case INKATTN_ENOTSUP: return "unsupported configuration";
    case INKATTN_EHIP: return "HIP runtime error";
    case INKATTN_ESCRATCH: return "request exceeds the library's static scratch buffer";
    default: return "unknown status";
  }
}

static inkattn_status_t sconv_common(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t num_seqs, int32_t num_tokens,
                                     int32_t max_chunk_len, const void* k_in, const void* v_in,
                                     const void* conv_w, void* conv_state,
                                     const int32_t* state_slot, const int32_t* cu_seqlens,
                                     const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                     const float* fp8_scales, void* stream) {
  if (dtype != INKATTN_FP32 && dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (head_dim != 128) return INKATTN_ENOTSUP;
  if (num_kv_heads < 1) return INKATTN_EINVAL;
  if (num_kv_heads > 64) return INKATTN_ENOTSUP;       // one thread per 8 channels, <= 1024
  if (num_seqs < 0 || num_tokens < 0 || max_chunk_len < 0) return INKATTN_EINVAL;
  if (fp8_scales != nullptr && !(fp8_scale_ok(fp8_scales[0]) && fp8_scale_ok(fp8_scales[1])))
    return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_chunk_len == 0) return INKATTN_OK;
  if (!k_in || !v_in || !conv_w || !conv_state || !state_slot || !cu_seqlens ||
      !slot_mapping || !k_cache || !v_cache)
    return INKATTN_EINVAL;
  if (!aligned16(k_in) || !aligned16(v_in) || !aligned16(conv_w) || !aligned16(conv_state) ||
      !aligned16(k_cache) || !aligned16(v_cache))
    return INKATTN_EINVAL;
  return from_hip(inkattn::launch_sconv(dtype, num_kv_heads, num_seqs, max_chunk_len, k_in,
                                        v_in, conv_w, conv_state, state_slot, cu_seqlens,
                                        slot_mapping, k_cache, v_cache, fp8_scales,
                                        (hipStream_t)stream));
}

inkattn_status_t inkattn_sconv(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                               int32_t num_seqs, int32_t num_tokens, int32_t max_chunk_len,
                               const void* k_in, const void* v_in, const void* conv_w,
                               void* conv_state, const int32_t* state_slot,
                               const int32_t* cu_seqlens, const int32_t* slot_mapping,
                               void* k_cache, void* v_cache, void* stream) {
  return sconv_common(dtype, num_kv_heads, head_dim, num_seqs, num_tokens, max_chunk_len, k_in,
                      v_in, conv_w, conv_state, state_slot, cu_seqlens, slot_mapping, k_cache,
                      v_cache, nullptr, stream);
}

inkattn_status_t inkattn_sconv_fp8(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_chunk_len,
                                   const void* k_in, const void* v_in, const void* conv_w,
                                   void* conv_state, const int32_t* state_slot,
                                   const int32_t* cu_seqlens, const int32_t* slot_mapping,
                                   float k_scale, float v_scale, void* k_cache, void* v_cache,
                                   void* stream) {
  const float scales[2] = {k_scale, v_scale};
  return sconv_common(dtype, num_kv_heads, head_dim, num_seqs, num_tokens, max_chunk_len, k_in,
                      v_in, conv_w, conv_state, state_slot, cu_seqlens, slot_mapping, k_cache,
                      v_cache, scales, stream);
}

inkattn_status_t inkattn_sconv_paged(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t num_seqs, int32_t num_tokens,
                                     int32_t max_chunk_len, const void* k_in, const void* v_in,
                                     const void* conv_w, const int32_t* cu_seqlens,
                                     const int32_t* seq_lens, const int32_t* state_block_table,
                                     int32_t max_state_blocks, void* k_state, void* v_state,
                                     const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                     void* stream) {
  if (dtype != INKATTN_FP32 && dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (head_dim != 128) return INKATTN_ENOTSUP;
  if (num_kv_heads < 1) return INKATTN_EINVAL;
  if (num_kv_heads > 64) return INKATTN_ENOTSUP;       // one thread per 8 channels, <= 1024
  if (num_seqs < 0 || num_tokens < 0 || max_chunk_len < 0) return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_chunk_len == 0) return INKATTN_OK;
  if (max_state_blocks < 1) return INKATTN_EINVAL;
  if (!k_in || !v_in || !conv_w || !cu_seqlens || !seq_lens || !state_block_table || !k_state ||
      !v_state || !slot_mapping || !k_cache || !v_cache)
    return INKATTN_EINVAL;
  if (!aligned16(k_in) || !aligned16(v_in) || !aligned16(conv_w) || !aligned16(k_state) ||
      !aligned16(v_state) || !aligned16(k_cache) || !aligned16(v_cache))
    return INKATTN_EINVAL;
  return from_hip(inkattn::launch_sconv_paged(dtype, num_kv_heads, num_seqs, max_chunk_len,
                                              k_in, v_in, conv_w, cu_seqlens, seq_lens,
                                              state_block_table, max_state_blocks, k_state,
                                              v_state, slot_mapping, k_cache, v_cache,
                                              (hipStream_t)stream));
}

inkattn_status_t inkattn_sconv_out(int32_t dtype, int32_t channels, int32_t num_seqs,
                                   int32_t num_tokens, int32_t max_chunk_len, const void* x,
                                   const void* conv_w, void* conv_state,
                                   const int32_t* state_slot, const int32_t* cu_seqlens, void* y,
                                   void* stream) {
  if (dtype != INKATTN_FP32 && dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (channels < 8 || channels % 8 != 0) return INKATTN_EINVAL;
  if (channels > 8192) return INKATTN_ENOTSUP;          // one thread per 8 channels, <= 1024
  if (num_seqs < 0 || num_tokens < 0 || max_chunk_len < 0) return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_chunk_len == 0) return INKATTN_OK;
  if (!x || !conv_w || !conv_state || !state_slot || !cu_seqlens || !y) return INKATTN_EINVAL;
  if (!aligned16(x) || !aligned16(conv_w) || !aligned16(conv_state) || !aligned16(y))
    return INKATTN_EINVAL;
  {
    // threads read halo rows of x that other threads would overwrite in y
    const size_t bytes = (size_t)num_tokens * channels * (dtype == INKATTN_BF16 ? 2 : 4);
    const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
    if (xb < yb + bytes && yb < xb + bytes) return INKATTN_EINVAL;
  }
  return from_hip(inkattn::launch_sconv_out(dtype, channels, num_seqs, max_chunk_len, x,
                                            conv_w, conv_state, state_slot, cu_seqlens, y,
                                            (hipStream_t)stream));
}

inkattn_status_t inkattn_relattn_prefill(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                         int32_t num_tokens, int32_t max_q_len,
                                         const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* block_table,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                         const void* bias, void* out, float* lse,
                                         void* stream) {
  inkattn_status_t st = check_desc(desc);
  if (st != INKATTN_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0) return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return INKATTN_OK;
  if (max_blocks_per_seq < 1) return INKATTN_EINVAL;
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seq_lens || !bias ||
      !out)
    return INKATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return INKATTN_EINVAL;
  if (bias_table_too_large(desc)) return INKATTN_ENOTSUP;
  return from_hip(inkattn::launch_prefill(shape_of(desc), num_seqs, max_q_len, q, k_cache,
                                          v_cache, block_table, max_blocks_per_seq,
                                          cu_seqlens_q, seq_lens, bias, out, lse,
                                          (hipStream_t)stream));
}

size_t inkattn_relattn_prefill_fp8_workspace_size(const inkattn_attn_desc_t* desc,
                                                  int32_t num_seqs, int32_t max_blocks_per_seq) {
  if (check_desc(desc) != INKATTN_OK || desc->dtype != INKATTN_BF16 || num_seqs < 0 ||
      max_blocks_per_seq < 0)
    return 0;
  const size_t pages = (size_t)num_seqs * (size_t)max_blocks_per_seq;
  const size_t page_bytes = (size_t)desc->num_kv_heads * 128 * 128 * 2;   // bf16
  return 2 * pages * page_bytes + ((pages * 4 + 15) & ~(size_t)15);
}

inkattn_status_t inkattn_relattn_prefill_fp8(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                             int32_t num_tokens, int32_t max_q_len,
                                             const void* q, const void* k_cache,
                                             const void* v_cache, float k_scale, float v_scale,
                                             const int32_t* block_table,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* cu_seqlens_q,
                                             const int32_t* seq_lens, const void* bias,
                                             void* out, float* lse, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  inkattn_status_t st = check_desc(desc);
  if (st != INKATTN_OK) return st;
  if (desc->dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return INKATTN_EINVAL;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0) return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return INKATTN_OK;
  if (max_blocks_per_seq < 1) return INKATTN_EINVAL;
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seq_lens || !bias ||
      !out || !workspace)
    return INKATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return INKATTN_EINVAL;
  if (bias_table_too_large(desc)) return INKATTN_ENOTSUP;
  // Workspace pages are numbered with 32-bit block-table entries, and the
  // conversion grid has one row per sequence.
  const size_t pages = (size_t)num_seqs * (size_t)max_blocks_per_seq;
  if (pages > 0x7fffffffULL || num_seqs > 65535) return INKATTN_ENOTSUP;
  if (workspace_bytes < inkattn_relattn_prefill_fp8_workspace_size(desc, num_seqs,
                                                                   max_blocks_per_seq))
    return INKATTN_EINVAL;
  const size_t page_bytes = (size_t)desc->num_kv_heads * 128 * 128 * 2;
  char* ws = static_cast<char*>(workspace);
  void* ws_k = ws;
  void* ws_v = ws + pages * page_bytes;
  int32_t* ws_table = reinterpret_cast<int32_t*>(ws + 2 * pages * page_bytes);
  hipError_t e = inkattn::launch_fp8_pages_to_bf16(
      desc->num_kv_heads, desc->window, num_seqs, max_blocks_per_seq, k_cache, v_cache,
      block_table, cu_seqlens_q, seq_lens, ws_k, ws_v, ws_table, (hipStream_t)stream);
  if (e != hipSuccess) return INKATTN_EHIP;
  return from_hip(inkattn::launch_prefill(shape_of(desc), num_seqs, max_q_len, q, ws_k, ws_v,
                                          ws_table, max_blocks_per_seq, cu_seqlens_q, seq_lens,
                                          bias, out, lse, (hipStream_t)stream, k_scale,
                                          v_scale));
}

inkattn_status_t inkattn_relattn_prefill_fp8_mma(const inkattn_attn_desc_t* desc,
                                                 int32_t num_seqs, int32_t num_tokens,
                                                 int32_t max_q_len, const void* q,
                                                 const void* k_cache, const void* v_cache,
                                                 float k_scale, float v_scale,
                                                 const int32_t* block_table,
                                                 int32_t max_blocks_per_seq,
                                                 const int32_t* cu_seqlens_q,
                                                 const int32_t* seq_lens, const void* bias,
                                                 void* out, float* lse, void* stream) {
  inkattn_status_t st = check_desc(desc);
  if (st != INKATTN_OK) return st;
  if (desc->dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
  if (!fp8_scale_ok(k_scale) || !fp8_scale_ok(v_scale)) return INKATTN_EINVAL;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0) return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_q_len == 0) return INKATTN_OK;
  if (max_blocks_per_seq < 1) return INKATTN_EINVAL;
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seq_lens || !bias || !out)
    return INKATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return INKATTN_EINVAL;
  if (bias_table_too_large(desc)) return INKATTN_ENOTSUP;
  return from_hip(inkattn::launch_prefill_f8(shape_of(desc), num_seqs, max_q_len, q, k_cache,
                                             v_cache, block_table, max_blocks_per_seq,
                                             cu_seqlens_q, seq_lens, bias, out, lse,
                                             (hipStream_t)stream, k_scale, v_scale));
}

int32_t inkattn_relattn_decode_num_splits(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                          int32_t max_seq_len) {
  if (check_desc(desc) != INKATTN_OK || num_seqs < 1 || max_seq_len < 1) return 1;
  return auto_splits(desc, num_seqs, max_seq_len);
}

size_t inkattn_relattn_decode_workspace_size(const inkattn_attn_desc_t* desc,
                                             int32_t num_seqs, int32_t max_seq_len,
                                             int32_t num_splits) {
  if (check_desc(desc) != INKATTN_OK || num_seqs < 0 || max_seq_len < 0 || num_splits < 0)
    return 0;
  const int64_t s = num_splits == 0 ? auto_splits(desc, num_seqs, max_seq_len) : num_splits;
  const size_t rows = (size_t)num_seqs * desc->num_q_heads * (size_t)s;
  return rows * 128 * sizeof(float) + ((rows * sizeof(float) + 15) & ~(size_t)15);
}

// Host checks of a one-token decode (every argument but the workspace);
// *splits receives the split count the call runs with.
static inkattn_status_t decode_check(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                     int32_t max_seq_len, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                     const void* bias, const void* out, int32_t num_splits,
                                     int32_t* splits) {
  inkattn_status_t st = check_desc(desc);
  if (st != INKATTN_OK) return st;
  if (num_seqs < 0 || max_seq_len < 0 || num_splits < 0) return INKATTN_EINVAL;
  *splits = 0;
  if (num_seqs == 0) return INKATTN_OK;
  if (max_seq_len < 1 || max_blocks_per_seq < 1) return INKATTN_EINVAL;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !bias || !out)
    return INKATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return INKATTN_EINVAL;
  if (bias_table_too_large(desc)) return INKATTN_ENOTSUP;
  const int32_t s = num_splits == 0 ? auto_splits(desc, num_seqs, max_seq_len) : num_splits;
  if (decode_grid_too_large(desc, num_seqs, num_seqs, s, 1)) return INKATTN_ENOTSUP;
  *splits = s;
  return INKATTN_OK;
}

// Launch of a checked one-token decode; the partial results of its splits
// (when there are several) go to `workspace`.
static inkattn_status_t decode_launch(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                      const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, const void* bias, void* out,
                                      float* lse, int32_t s, void* workspace, void* stream) {
  const size_t rows = (size_t)num_seqs * desc->num_q_heads * (size_t)s;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + rows * 128;
  return from_hip(inkattn::launch_decode(shape_of(desc), num_seqs, num_seqs, 1, s, q, k_cache,
                                         v_cache, block_table, max_blocks_per_seq, nullptr,
                                         seq_lens, bias, out, lse, part_o, part_lse, nullptr,
                                         (hipStream_t)stream));
}

inkattn_status_t inkattn_relattn_decode(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                        int32_t max_seq_len, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                        const void* bias, void* out, float* lse,
                                        int32_t num_splits, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  int32_t s = 0;
  inkattn_status_t st = decode_check(desc, num_seqs, max_seq_len, q, k_cache, v_cache,
                                     block_table, max_blocks_per_seq, seq_lens, bias, out,
                                     num_splits, &s);
  if (st != INKATTN_OK || num_seqs == 0) return st;
  if (!workspace || !aligned16(workspace)) return INKATTN_EINVAL;
  const size_t need = inkattn_relattn_decode_workspace_size(desc, num_seqs, max_seq_len, s);
  if (workspace_bytes < need) return INKATTN_EINVAL;
  return decode_launch(desc, num_seqs, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                       seq_lens, bias, out, lse, s, workspace, stream);
}

int32_t inkattn_relattn_decode_mq_num_splits(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                             int32_t max_q_len, int32_t max_seq_len) {
  if (check_desc(desc) != INKATTN_OK || num_seqs < 1 || max_seq_len < 1 || max_q_len < 1 ||
      max_q_len > kMaxDecodeQueries)
    return 1;
  return auto_splits(desc, num_seqs, max_seq_len, max_q_len);
}

size_t inkattn_relattn_decode_mq_workspace_size(const inkattn_attn_desc_t* desc,
                                                int32_t num_seqs, int32_t num_tokens,
                                                int32_t max_q_len, int32_t max_seq_len,
                                                int32_t num_splits) {
  if (check_desc(desc) != INKATTN_OK || num_seqs < 0 || num_tokens < 0 || max_seq_len < 0 ||
      num_splits < 0 || max_q_len < 1 || max_q_len > kMaxDecodeQueries)
    return 0;
  const int64_t s =
      num_splits == 0 ? auto_splits(desc, num_seqs, max_seq_len, max_q_len) : num_splits;
  const size_t rows = (size_t)num_tokens * desc->num_q_heads * (size_t)s;
  return rows * 128 * sizeof(float) + ((rows * sizeof(float) + 15) & ~(size_t)15);
}

static inkattn_status_t decode_mq_common(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                         int32_t num_tokens, int32_t max_q_len,
                                         int32_t max_seq_len, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_table,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                         const void* bias, void* out, float* lse,
                                         int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, const float* fp8_scales,
                                         void* stream) {
  inkattn_status_t st = check_desc(desc);
  if (st != INKATTN_OK) return st;
  if (fp8_scales != nullptr) {
    if (desc->dtype != INKATTN_BF16) return INKATTN_ENOTSUP;
    if (!fp8_scale_ok(fp8_scales[0]) || !fp8_scale_ok(fp8_scales[1])) return INKATTN_EINVAL;
  }
  if (num_seqs < 0 || num_tokens < 0 || max_seq_len < 0 || num_splits < 0 || max_q_len < 0)
    return INKATTN_EINVAL;
  if (num_seqs == 0 || num_tokens == 0) return INKATTN_OK;
  if (max_q_len < 1 || num_tokens < num_seqs || max_seq_len < 1 || max_blocks_per_seq < 1)
    return INKATTN_EINVAL;
  if (max_q_len > kMaxDecodeQueries) return INKATTN_ENOTSUP;
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seq_lens || !bias ||
      !out || !workspace)
    return INKATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return INKATTN_EINVAL;
  if (bias_table_too_large(desc)) return INKATTN_ENOTSUP;
  const int32_t s =
      num_splits == 0 ? auto_splits(desc, num_seqs, max_seq_len, max_q_len) : num_splits;
  if (decode_grid_too_large(desc, num_seqs, num_tokens, s, max_q_len)) return INKATTN_ENOTSUP;
  const size_t need = inkattn_relattn_decode_mq_workspace_size(desc, num_seqs, num_tokens,
                                                               max_q_len, max_seq_len, s);
  if (workspace_bytes < need) return INKATTN_EINVAL;
  const size_t rows = (size_t)num_tokens * desc->num_q_heads * (size_t)s;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + rows * 128;
  return from_hip(inkattn::launch_decode(shape_of(desc), num_seqs, num_tokens, max_q_len, s, q,
                                         k_cache, v_cache, block_table, max_blocks_per_seq,
                                         cu_seqlens_q, seq_lens, bias, out, lse, part_o,
                                         part_lse, fp8_scales, (hipStream_t)stream));
}

inkattn_status_t inkattn_relattn_decode_mq(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                           int32_t num_tokens, int32_t max_q_len,
                                           int32_t max_seq_len, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_table,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                           const void* bias, void* out, float* lse,
                                           int32_t num_splits, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return decode_mq_common(desc, num_seqs, num_tokens, max_q_len, max_seq_len, q, k_cache,
                          v_cache, block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens, bias,
                          out, lse, num_splits, workspace, workspace_bytes, nullptr, stream);
}

inkattn_status_t inkattn_relattn_decode_fp8(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                            int32_t num_tokens, int32_t max_q_len,
                                            int32_t max_seq_len, const void* q,
                                            const void* k_cache, const void* v_cache,
                                            float k_scale, float v_scale,
                                            const int32_t* block_table,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* cu_seqlens_q,
                                            const int32_t* seq_lens, const void* bias, void* out,
                                            float* lse, int32_t num_splits, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  const float scales[2] = {k_scale, v_scale};
  return decode_mq_common(desc, num_seqs, num_tokens, max_q_len, max_seq_len, q, k_cache,
                          v_cache, block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens, bias,
                          out, lse, num_splits, workspace, workspace_bytes, scales, stream);
}

// The decode that allocates nothing: its split partials live in `scratch`,
// a static device array of INKATTN_NOALLOC_SCRATCH_BYTES.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address); it takes the array's address on the current device once
// through hipGetSymbolAddress and uses that.  Every call on one device
// shares that device's array.
inkattn_status_t inkattn_relattn_decode_noalloc(const inkattn_attn_desc_t* desc,
                                                int32_t num_seqs, int32_t max_seq_len,
                                                const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* block_table,
                                                int32_t max_blocks_per_seq,
                                                const int32_t* seq_lens, const void* bias,
                                                void* out, float* lse, int32_t num_splits,
                                                void* stream) {
  int32_t s = 0;
  inkattn_status_t st = decode_check(desc, num_seqs, max_seq_len, q, k_cache, v_cache,
                                     block_table, max_blocks_per_seq, seq_lens, bias, out,
                                     num_splits, &s);
  if (st != INKATTN_OK || num_seqs == 0) return st;
  // One split writes the output directly and uses no partials.
  const size_t need =
      s > 1 ? inkattn_relattn_decode_workspace_size(desc, num_seqs, max_seq_len, s) : 0;
  if (need > (size_t)INKATTN_NOALLOC_SCRATCH_BYTES) return INKATTN_ESCRATCH;
  void* ws = nullptr;
  if (s > 1) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return INKATTN_EHIP;
  }
  return decode_launch(desc, num_seqs, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                       seq_lens, bias, out, lse, s, ws, stream);
}

}  // extern "C"
