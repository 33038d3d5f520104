// Internal launcher interface between the C-ABI layer (api.hip) and the
// kernel translation units.  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace inkattn {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// fp8_scales: host pointer to {key scale, value scale} for an E4M3 cache, or
// nullptr for a cache in the activation dtype.
hipError_t launch_sconv(int dtype, int Hkv, int num_seqs, int max_chunk_len,
                        const void* k_in, const void* v_in, const void* conv_w,
                        void* conv_state, const int32_t* state_slot,
                        const int32_t* cu_seqlens, const int32_t* slot_mapping,
                        void* k_cache, void* v_cache, const float* fp8_scales,
                        hipStream_t stream);

hipError_t launch_sconv_paged(int dtype, int Hkv, int num_seqs, int max_chunk_len,
                              const void* k_in, const void* v_in, const void* conv_w,
                              const int32_t* cu_seqlens, const int32_t* seq_lens,
                              const int32_t* state_block_table, int max_state_blocks,
                              void* k_state, void* v_state, const int32_t* slot_mapping,
                              void* k_cache, void* v_cache, hipStream_t stream);

hipError_t launch_sconv_out(int dtype, int C, int num_seqs, int max_chunk_len, const void* x,
                            const void* conv_w, void* conv_state, const int32_t* state_slot,
                            const int32_t* cu_seqlens, void* y, hipStream_t stream);

struct AttnShape {
  int dtype, Hq, Hkv, window, bias_len;
};

hipError_t launch_prefill(const AttnShape& s, int num_seqs, int max_q_len, const void* q,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                          const void* bias, void* out, float* lse, hipStream_t stream,
                          float k_scale = 1.0f, float v_scale = 1.0f);
// E4M3 cache with FP8 matrix products (prefill_f8.hip).
hipError_t launch_prefill_f8(const AttnShape& s, int num_seqs, int max_q_len, const void* q,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                          const void* bias, void* out, float* lse, hipStream_t stream,
                          float k_scale = 1.0f, float v_scale = 1.0f);

// Pages of an E4M3 cache that the prefill of each sequence attends, as bf16
// codes (exact) in a workspace cache: sequence b's block blk goes to
// workspace page b * max_blocks + blk, which ws_table records.
hipError_t launch_fp8_pages_to_bf16(int Hkv, int window, int num_seqs, int max_blocks,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* cu_seqlens_q,
                                    const int32_t* seq_lens, void* ws_k, void* ws_v,
                                    int32_t* ws_table, hipStream_t stream);

// Decode over num_seqs sequences with 1 .. max_q_len query tokens each
// (cu_seqlens_q == nullptr: exactly one token per sequence, token b of
// sequence b).  The (token, head) columns of a kv-head group are computed in
// tiles of 16.  fp8_scales: host pointer to {key scale, value scale} for an
// E4M3 cache (bf16 queries), or nullptr for a cache in the activation dtype.
constexpr int decode_column_tiles(int G, int max_q_len) { return (G * max_q_len + 15) / 16; }

// bf16 queries with 2 .. 8 column tiles run the LDS-staged multi-query kernel:
// one work-group per (split, kv-head, sequence) holds every column.  Other
// shapes run one work-group per (split, kv-head, sequence) and column group.
constexpr bool decode_uses_lds_mq(int dtype, int G, int max_q_len) {
  return dtype == kDtypeBf16 && decode_column_tiles(G, max_q_len) >= 2 &&
         decode_column_tiles(G, max_q_len) <= 8;
}
// Query tokens per sequence in one decode call.
constexpr int kMaxMqTokens = 16;
// Of those, bf16 queries with 2 .. 5 column tiles run the register-resident
// multi-query kernel (decode_mqr.hip) when the bias band of a 32-key item
// (G heads x 31 + max_q_len distances) fits its 6 staged entries per lane,
// R fits a 24-bit multiply and the bias table a 32-bit byte offset.
constexpr int kMaxRegMqTiles = 5;
constexpr int kMaxRegMqG = 16;
constexpr int kRegMqBandEntries = 384;
constexpr bool decode_uses_reg_mq(int dtype, int G, int max_q_len, long Hq, long R) {
  return decode_uses_lds_mq(dtype, G, max_q_len) &&
         decode_column_tiles(G, max_q_len) <= kMaxRegMqTiles && G <= kMaxRegMqG &&
         max_q_len <= kMaxMqTokens && G * (31 + max_q_len) <= kRegMqBandEntries &&
         R < (1L << 24) && Hq * R * 2 < (1L << 32);
}
// Work-groups per (split, kv-head, sequence).
constexpr int decode_groups_per_pair(int dtype, int G, int max_q_len) {
  return decode_uses_lds_mq(dtype, G, max_q_len) ? 1 : decode_column_tiles(G, max_q_len);
}

hipError_t launch_decode(const AttnShape& s, int num_seqs, int num_tokens, int max_q_len,
                         int num_splits, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         int max_blocks_per_seq, const int32_t* cu_seqlens_q,
                         const int32_t* seq_lens, const void* bias, void* out, float* lse,
                         float* part_o, float* part_lse, const float* fp8_scales,
                         hipStream_t stream);

// The LDS-staged multi-query split kernel alone (no merge); bf16 queries,
// bf16 cache or (fp8_scales != nullptr) E4M3 cache.
void launch_decode_mq_lds(const AttnShape& s, int num_seqs, int num_splits, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens, const void* bias, void* out, float* lse,
                          float* part_o, float* part_lse, const float* fp8_scales,
                          hipStream_t stream);
// The register-resident multi-query split kernel alone (no merge), for the
// shapes decode_uses_reg_mq admits.
void launch_decode_mq_reg(const AttnShape& s, int num_seqs, int num_splits, int max_q_len,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                          const void* bias, void* out, float* lse, float* part_o,
                          float* part_lse, const float* fp8_scales, hipStream_t stream);

}  // namespace inkattn
