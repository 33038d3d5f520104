// Prefill over an E4M3 (OCP FP8) KV cache: the pages each sequence's chunk
// attends are converted to bf16 codes in a workspace cache, and the bf16
// prefill kernel runs over that copy with the cache scales.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Roadmap (FP8 for
// the global-attention layers) and Model Architecture / Attention.  A cached
// code e of a key means e * k_scale (of a value, e * v_scale); every E4M3
// value is a bf16 value, so the conversion is exact and the scales enter the
// prefill as factors of the logits and of the output.
//
// The prefill is bound by its matrix cores (≈1,600 flop per K/V byte at 8K
// tokens with a 2K window), so one extra pass over the attended pages -- read
// E4M3, write bf16, which the prefill then reads -- costs a few percent of
// its time, and the tuned kernel is used unchanged.
#include "device_common.h"
#include "launch.h"

namespace inkattn {

namespace {

constexpr int kConvThreads = 256;

// One work-group per (block index, sequence); blocks outside the range the
// sequence's chunk attends exit at once.
__global__ __launch_bounds__(kConvThreads) void fp8_pages_to_bf16_kernel(
    int Hkv, int window, int max_blocks, const uint8_t* __restrict__ k_cache,
    const uint8_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    bf16* __restrict__ ws_k, bf16* __restrict__ ws_v, int32_t* __restrict__ ws_table) {
  const int blk = blockIdx.x;
  const int b = blockIdx.y;
  // Every entry of the workspace table names its own page, converted or not,
  // so that no entry of it can address memory outside the workspace.
  const size_t ws_page = (size_t)b * max_blocks + blk;
  if (threadIdx.x == 0) ws_table[ws_page] = (int32_t)ws_page;
  const int q_len = cu_q[b + 1] - cu_q[b];
  const int L = seq_lens[b];
  if (q_len <= 0 || L <= 0) return;
  const int key_lo = window > 0 ? max(0, L - q_len - window + 1) : 0;
  if (blk < (key_lo >> 7) || blk > ((L - 1) >> 7)) return;
  const size_t page_elems = (size_t)Hkv * kPage * kHeadDim;     // codes (bytes) per page
  const size_t phys = (size_t)block_table[ws_page];
  const u32x4* ks = reinterpret_cast<const u32x4*>(k_cache + phys * page_elems);
  const u32x4* vs = reinterpret_cast<const u32x4*>(v_cache + phys * page_elems);
  bf16* kd = ws_k + ws_page * page_elems;
  bf16* vd = ws_v + ws_page * page_elems;
  const int n16 = (int)(page_elems / 16);                      // 16-code chunks per page
  for (int i = threadIdx.x; i < n16; i += kConvThreads) {
    const u32x4 k = ks[i], v = vs[i];
    fp8x8_to_bf16(k[0], k[1]).store(kd + 16 * (size_t)i);
    fp8x8_to_bf16(k[2], k[3]).store(kd + 16 * (size_t)i + 8);
    fp8x8_to_bf16(v[0], v[1]).store(vd + 16 * (size_t)i);
    fp8x8_to_bf16(v[2], v[3]).store(vd + 16 * (size_t)i + 8);
  }
}

}  // namespace

hipError_t launch_fp8_pages_to_bf16(int Hkv, int window, int num_seqs, int max_blocks,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens, void* ws_k, void* ws_v,
                                    int32_t* ws_table, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_pages_to_bf16_kernel, dim3(max_blocks, num_seqs), dim3(kConvThreads),
                     0, stream, Hkv, window, max_blocks, (const uint8_t*)k_cache,
                     (const uint8_t*)v_cache, block_table, cu_seqlens_q, seq_lens,
                     (bf16*)ws_k, (bf16*)ws_v, ws_table);
  return hipGetLastError();
}

}  // namespace inkattn
