/*
 * libinkattn -- the Inkling attention-block hot path on AMD Instinct MI355X
 * (gfx950): short convolution of keys and values fused into the paged
 * KV-cache write, and relative-position grouped-query attention (prefill and
 * split-K decode).
 *
 * Sources (web pages this library is built from):
 *   [A] news article "vLLM, TML Inkling Day-0 support" (news.ainew.jp),
 *       sections Model Architecture / Attention, Model Architecture / Sconv,
 *       vLLM Integration & Optimization / Managing the sconv cache and
 *       / FA4 with sheared bias;
 *   [B] vLLM recipe "thinkingmachines/Inkling", Guide / Overview and
 *       Client Usage (MI355X launch with a KV block size of 128);
 *   [C] vLLM recipe "thinkingmachines/Inkling-Small", Client Usage (same).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers into memory the caller owns.
 *   The library never allocates, frees or synchronises; every launch is
 *   asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null
 *   stream).  The library keeps no global state and is thread-safe, except
 *   the static scratch array of inkattn_relattn_decode_noalloc (see there).
 * - Scalar arguments (counts, maxima) are host values.
 * - Storage dtype INKATTN_FP32 (float) or INKATTN_BF16 (bfloat16 bits);
 *   all arithmetic is fp32.  q, K/V, conv weights/state, bias and out share
 *   the dtype; lse and the decode workspace are always float.
 * - head_dim must be 128 and the KV block (page) 128 tokens ([A] Attention;
 *   [B], [C] MI355X launch).
 * - KV-cache layout, one 32 KiB (bf16) tile per (block, kv-head):
 *       k_cache [num_blocks][num_kv_heads][128 tokens][128 dims]
 *       v_cache [num_blocks][num_kv_heads][128 dims][128 tokens]   (V^T)
 *   Token position p of sequence b is slot
 *       block_table[b][p / 128] * 128 + p % 128.
 * - Device-side preconditions are not checked (that would need a sync):
 *   indices in range, distinct state slots per call, every cache entry of
 *   positions < seq_len finite, 1 <= q_len <= seq_len.
 * - Errors: host-side checks run before any launch.  INKATTN_EINVAL for a
 *   NULL required pointer, a bad size or a misaligned pointer (16 B);
 *   INKATTN_ENOTSUP for an unsupported dtype, head_dim, block size or GQA
 *   group; INKATTN_EHIP when the HIP runtime reports a launch failure.
 *   Nothing aborts and no exception crosses the ABI.
 */
#ifndef INKATTN_H_
#define INKATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INKATTN_OK = 0,
  INKATTN_EINVAL = 1,
  INKATTN_ENOTSUP = 2,
  INKATTN_EHIP = 3,
  INKATTN_ESCRATCH = 4    /* inkattn_relattn_decode_noalloc: the request's split
                             partials exceed INKATTN_NOALLOC_SCRATCH_BYTES */
} inkattn_status_t;

/* Size of the static device scratch of inkattn_relattn_decode_noalloc. */
#define INKATTN_NOALLOC_SCRATCH_BYTES (8u << 20)

typedef enum { INKATTN_FP32 = 0, INKATTN_BF16 = 1 } inkattn_dtype_t;

/* Attention layer description.
 *   window   : sliding window W (query i sees keys j with 0 <= i-j <= W-1);
 *              0 = full causal ([A] Attention: sliding-window and full layers).
 *   bias_len : R >= 1, length of each row of the relative-position table;
 *              distances >= R use entry R-1. */
typedef struct {
  int32_t dtype;          /* inkattn_dtype_t */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv; Hq % Hkv == 0, Hq/Hkv <= 16 */
  int32_t head_dim;       /* must be 128 */
  int32_t block_size;     /* must be 128 */
  int32_t window;         /* W >= 0 */
  int32_t bias_len;       /* R >= 1 */
} inkattn_attn_desc_t;

/* Short convolution of keys and values, fused with the paged KV-cache write
 * ([A] Sconv: window-4 convolution over key and value channels;
 *  [A] Managing the sconv cache: the last W-1 = 3 tokens are cached).
 *
 * For each sequence b (tokens cu_seqlens[b] .. cu_seqlens[b+1]-1) and each
 * channel c of K (and separately of V):
 *   xp = [conv_state[state_slot[b]][which][0..2][c]; x[tokens][c]]
 *   y[t][c] = sum_{k=0..3} conv_w[which][c][k] * xp[t+k][c]
 *   (tap 3 weights the current token), y is rounded to dtype and written to
 *   the cache slot slot_mapping[t]; afterwards conv_state[state_slot[b]][which]
 *   holds the last 3 rows of xp (pre-convolution values).  A fresh sequence
 *   passes a zeroed state.
 *
 *   k_in, v_in   [num_tokens][Hkv*128]      pre-convolution keys / values
 *   conv_w       [2][Hkv*128][4]            [0] keys, [1] values
 *   conv_state   [num_slots][2][3][Hkv*128] read, then updated in place
 *   state_slot   int32 [num_seqs]           distinct within one call
 *   cu_seqlens   int32 [num_seqs+1]
 *   slot_mapping int32 [num_tokens]
 *   k_cache, v_cache                        layouts above
 *   max_chunk_len: host upper bound of cu_seqlens[b+1]-cu_seqlens[b].
 * num_tokens == 0 or num_seqs == 0 is a no-op returning INKATTN_OK. */
inkattn_status_t inkattn_sconv(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                               int32_t num_seqs, int32_t num_tokens, int32_t max_chunk_len,
                               const void* k_in, const void* v_in, const void* conv_w,
                               void* conv_state, const int32_t* state_slot,
                               const int32_t* cu_seqlens, const int32_t* slot_mapping,
                               void* k_cache, void* v_cache, void* stream);

/* The same short convolution with the sconv state kept in a paged cache of
 * its own, as the K/V cache of a virtual sliding-window layer of window 3
 * ([A] Managing the sconv cache: blocks outside the window can be evicted,
 * and prefix caching covers the sconv state too).  Instead of a per-sequence
 * state slot, every token's pre-convolution key and value rows are kept:
 *   k_state, v_state  [num_state_blocks][128 tokens][Hkv*128]
 * Position p of sequence b is row p % 128 of block
 * state_block_table[b][p / 128].  Sequence b's chunk (tokens cu_seqlens[b] ..
 * cu_seqlens[b+1]-1, n of them) sits at positions seq_lens[b]-n ..
 * seq_lens[b]-1; its convolution reads positions seq_lens[b]-n-3 ..
 * seq_lens[b]-n-1 from the state cache (zero before position 0), then writes
 * the chunk's own input rows there.  The outputs go to k_cache/v_cache at
 * slot_mapping[t] exactly as inkattn_sconv writes them.  Sequences may share
 * state blocks of their common prefix (read only); the blocks a call writes
 * must not be read by another sequence in the same call.
 *   state_block_table int32 [num_seqs][max_state_blocks]
 * num_tokens == 0 or num_seqs == 0 is a no-op returning INKATTN_OK; other
 * errors as inkattn_sconv. */
inkattn_status_t inkattn_sconv_paged(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t num_seqs, int32_t num_tokens,
                                     int32_t max_chunk_len, const void* k_in, const void* v_in,
                                     const void* conv_w, const int32_t* cu_seqlens,
                                     const int32_t* seq_lens, const int32_t* state_block_table,
                                     int32_t max_state_blocks, void* k_state, void* v_state,
                                     const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                     void* stream);

/* Short convolution of a plain activation tensor: the attention output and
 * the MoE output each pass through a sconv of their own ([A] Model
 * Architecture / Sconv: four per layer, on keys, values, attention output and
 * MoE output), with the same taps and three-token state as inkattn_sconv but
 * no KV-cache write:
 *   y[t][c] = sum_{k=0..3} conv_w[c][k] * xp[t+k][c],  xp = [state; chunk]
 * and the state becomes the last three rows of xp.
 *   x, y        [num_tokens][channels]  sequences packed back to back; y must
 *                                       not overlap x
 *   conv_w      [channels][4]           conv_w[c][3] weights the current token
 *   conv_state  [num_slots][3][channels] read, then updated in place
 *   state_slot  int32 [num_seqs]        distinct within one call
 *   cu_seqlens  int32 [num_seqs+1]
 *   max_chunk_len: host upper bound of cu_seqlens[b+1]-cu_seqlens[b].
 * channels: a multiple of 8 (EINVAL otherwise), at most 8192 (ENOTSUP).
 * Pointers 16-byte aligned.  num_tokens == 0 or num_seqs == 0 is a no-op
 * returning INKATTN_OK. */
inkattn_status_t inkattn_sconv_out(int32_t dtype, int32_t channels, int32_t num_seqs,
                                   int32_t num_tokens, int32_t max_chunk_len, const void* x,
                                   const void* conv_w, void* conv_state,
                                   const int32_t* state_slot, const int32_t* cu_seqlens, void* y,
                                   void* stream);

/* Relative-position GQA attention over a chunk of new tokens per sequence
 * ([A] Attention; [A] FA4 with sheared bias):
 *   logit[h,i,j] = q_i . k_j / sqrt(128) + bias[h][min(i-j, R-1)]
 * over keys j <= i (and i-j <= W-1 when W > 0), softmax, times V.  Query
 * head h reads KV head h / (Hq/Hkv).  The chunk of sequence b
 * (tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1, q_len = their count)
 * occupies positions seq_lens[b]-q_len .. seq_lens[b]-1; its keys and values
 * must already be in the cache (inkattn_sconv).
 *
 *   q     [num_tokens][Hq][128]
 *   block_table int32 [num_seqs][max_blocks_per_seq]
 *   cu_seqlens_q int32 [num_seqs+1], seq_lens int32 [num_seqs]
 *   bias  [Hq][R]
 *   out   [num_tokens][Hq][128]
 *   lse   float [num_tokens][Hq] = log(sum_j exp(logit_j)), or NULL
 *   max_q_len: host upper bound of the per-sequence q_len.
 * INKATTN_ENOTSUP if the bias table (Hq * R elements) reaches 2 GiB. */
inkattn_status_t inkattn_relattn_prefill(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                         int32_t num_tokens, int32_t max_q_len,
                                         const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* block_table,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                         const void* bias, void* out, float* lse,
                                         void* stream);

/* Prefill over an E4M3 (OCP FP8) KV cache written by inkattn_sconv_fp8
 * ([A] Roadmap: FP8 for the global-attention layers): the same logits and
 * outputs as inkattn_relattn_prefill over a cache whose keys are
 * code * k_scale and whose values are code * v_scale.  bf16 queries only.
 * The blocks each sequence's chunk attends are first converted to bf16
 * codes (exact) in `workspace`, which also holds a block table of its own;
 * the prefill kernel then reads that copy and applies the scales.
 *   k_cache, v_cache: uint8 codes, [num_blocks][Hkv][128][128] and
 *                     [num_blocks][Hkv][128 dims][128 tokens].
 *   workspace: device, 16-byte aligned, caller-owned scratch of at least
 *              inkattn_relattn_prefill_fp8_workspace_size(...) bytes (two
 *              bf16 page copies per (sequence, block) plus an int32 table);
 *              its contents need no initialisation and are overwritten.
 * Other arguments as inkattn_relattn_prefill.  INKATTN_ENOTSUP for an fp32
 * desc, more than 65535 sequences or 2^31 (sequence, block) pages;
 * INKATTN_EINVAL for a scale that is not positive and finite or a workspace
 * that is too small. */
size_t inkattn_relattn_prefill_fp8_workspace_size(const inkattn_attn_desc_t* desc,
                                                  int32_t num_seqs, int32_t max_blocks_per_seq);
inkattn_status_t inkattn_relattn_prefill_fp8(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                             int32_t num_tokens, int32_t max_q_len,
                                             const void* q, const void* k_cache,
                                             const void* v_cache, float k_scale, float v_scale,
                                             const int32_t* block_table,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* cu_seqlens_q,
                                             const int32_t* seq_lens, const void* bias,
                                             void* out, float* lse, void* workspace,
                                             size_t workspace_bytes, void* stream);

/* Prefill over an E4M3 cache with FP8 matrix products, for the global
 * (full-causal) attention layers ([A] Roadmap: FP8 for global attention,
 * whose cost is compute as well as KV capacity).  The same logits as
 * inkattn_relattn_prefill_fp8, computed with both products in E4M3:
 *   - Q is quantised per tile of 256 query rows of one q-head (rows
 *     256t .. 256t+255 of each sequence's chunk): s_q = amax / 448 over the
 *     tile's |q| (1 for an all-zero tile), codes = RNE_E4M3(q * (448 / amax))
 *     computed in fp32; the logits use code * s_q.
 *   - The softmax probabilities (each <= 256) are rounded to E4M3 before the
 *     P V product, and the row sums add the rounded values.
 * K and V are read as codes straight from the pages (no workspace).  Outputs
 * differ from the exact attention over (code * s_q, k codes * k_scale,
 * v codes * v_scale) only through the rounding of the probabilities: each
 * weight of the output's weighted mean moves by a relative 2^-4 at most.
 *   k_cache, v_cache: uint8 codes, [num_blocks][Hkv][128][128] and
 *                     [num_blocks][Hkv][128 dims][128 tokens].
 * Other arguments as inkattn_relattn_prefill.  INKATTN_ENOTSUP for an fp32
 * desc or a bias table of 2 GiB or more; INKATTN_EINVAL for a scale that is
 * not positive and finite or a pointer that is not 16-byte aligned. */
inkattn_status_t inkattn_relattn_prefill_fp8_mma(const inkattn_attn_desc_t* desc,
                                                 int32_t num_seqs, int32_t num_tokens,
                                                 int32_t max_q_len, const void* q,
                                                 const void* k_cache, const void* v_cache,
                                                 float k_scale, float v_scale,
                                                 const int32_t* block_table,
                                                 int32_t max_blocks_per_seq,
                                                 const int32_t* cu_seqlens_q,
                                                 const int32_t* seq_lens, const void* bias,
                                                 void* out, float* lse, void* stream);

/* Number of KV splits inkattn_relattn_decode uses for num_splits = 0 (auto):
 * enough (sequence, kv-head, split) work-groups to fill the GPU, never more
 * splits than 128-token blocks in the attended range ([A] FA4 with sheared
 * bias: the split count is chosen from batch size and KV length). */
int32_t inkattn_relattn_decode_num_splits(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                          int32_t max_seq_len);

/* Workspace bytes inkattn_relattn_decode needs for this shape and split
 * count (0 = auto): per (sequence, q-head, split) 128 floats of partial
 * output plus one float of log-sum-exp.  Returns 0 for an invalid desc. */
size_t inkattn_relattn_decode_workspace_size(const inkattn_attn_desc_t* desc,
                                             int32_t num_seqs, int32_t max_seq_len,
                                             int32_t num_splits);

/* One decode step: the query of each sequence sits at position
 * seq_lens[b]-1, whose key and value are already in the cache
 * (inkattn_sconv with one token per sequence, same stream, earlier).
 * Same logits as inkattn_relattn_prefill.  Split-K: each (sequence, kv-head,
 * split) work-group attends over its share of the key blocks with all
 * Hq/Hkv query heads of the group, writes a partial output and
 * log-sum-exp to `workspace`, and a second kernel merges the splits (with
 * one split the work-group writes out/lse itself and no merge runs).
 *
 *   q     [num_seqs][Hq][128]
 *   out   [num_seqs][Hq][128], lse float [num_seqs][Hq] or NULL
 *   max_seq_len: host upper bound of seq_lens[b].
 *   num_splits : 0 = auto (inkattn_relattn_decode_num_splits), else >= 1.
 *   workspace  : device memory of at least
 *                inkattn_relattn_decode_workspace_size(...) bytes, 16 B aligned.
 * INKATTN_ENOTSUP if the bias table (Hq * R elements) reaches 2 GiB, or if
 * num_splits * Hkv * num_seqs work-groups exceed 2^31. */
inkattn_status_t inkattn_relattn_decode(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                        int32_t max_seq_len, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                        const void* bias, void* out, float* lse,
                                        int32_t num_splits, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* inkattn_relattn_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments (minus workspace
 * and workspace_bytes), same computation and kernels, same result.
 *   The split partials live in a static device array of
 *   INKATTN_NOALLOC_SCRATCH_BYTES (8 MiB) inside the library, which every GPU
 *   the library runs on holds until the process ends; the call itself
 *   allocates nothing.  They take inkattn_relattn_decode_workspace_size(...)
 *   bytes for the split count used (none with one split): at 8 MiB about
 *   16,000 (sequence, q-head, split) rows, e.g. 4 x 1M-key sequences with
 *   Hq = 32 at the automatic 16 splits use 1 MiB.
 *   Every call on one GPU shares that GPU's array: calls that overlap in
 *   time on one GPU (other streams, other host threads) race and may return
 *   wrong results.  Calls ordered on one stream are safe; nothing in the
 *   array needs clearing between calls (each call writes every partial it
 *   reads).
 * Errors as inkattn_relattn_decode; INKATTN_ESCRATCH when the partials of
 * the split count used exceed the array (pass fewer splits); INKATTN_EHIP
 * when the runtime cannot give the array's device address. */
inkattn_status_t inkattn_relattn_decode_noalloc(const inkattn_attn_desc_t* desc,
                                                int32_t num_seqs, int32_t max_seq_len,
                                                const void* q, const void* k_cache,
                                                const void* v_cache, const int32_t* block_table,
                                                int32_t max_blocks_per_seq,
                                                const int32_t* seq_lens, const void* bias,
                                                void* out, float* lse, int32_t num_splits,
                                                void* stream);

/* Decode of several query tokens per sequence at once: the verification
 * step of multi-token prediction, where a sequence's last accepted token and
 * its draft tokens are checked together ([A] Model Architecture / MTP: up to
 * 9 tokens per forward step; [A] Performance: MTP8 with a mean acceptance
 * length of 4.5).  Sequence b has q_len = cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] query tokens (1 <= q_len <= max_q_len <= 16) at positions
 * seq_lens[b]-q_len .. seq_lens[b]-1, whose keys and values are already in
 * the cache (inkattn_sconv); each attends causally (and within the window)
 * with the logit of inkattn_relattn_prefill, so the result equals prefill
 * of those tokens with the sequence's earlier tokens as context.  With bf16
 * queries and 17 .. 128 (token, q-head) pairs per kv-head group, K and V are
 * read once per (sequence, kv-head, split) for all of them (staged through
 * LDS); otherwise once per 16 such pairs (fp32) or per 48 (bf16, larger
 * groups).
 *   q    [num_tokens][Hq][128]        out [num_tokens][Hq][128]
 *   lse  float [num_tokens][Hq], or NULL
 *   cu_seqlens_q int32 [num_seqs+1], cu_seqlens_q[num_seqs] = num_tokens
 *   workspace: device, 16-byte aligned, >= inkattn_relattn_decode_mq_
 *              workspace_size(...) bytes; caller-owned scratch.
 *   num_splits: 0 = automatic (inkattn_relattn_decode_mq_num_splits).
 * Errors as inkattn_relattn_decode; INKATTN_ENOTSUP for max_q_len > 16. */
int32_t inkattn_relattn_decode_mq_num_splits(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                             int32_t max_q_len, int32_t max_seq_len);
size_t inkattn_relattn_decode_mq_workspace_size(const inkattn_attn_desc_t* desc,
                                                int32_t num_seqs, int32_t num_tokens,
                                                int32_t max_q_len, int32_t max_seq_len,
                                                int32_t num_splits);
inkattn_status_t inkattn_relattn_decode_mq(const inkattn_attn_desc_t* desc, int32_t num_seqs,
                                           int32_t num_tokens, int32_t max_q_len,
                                           int32_t max_seq_len, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_table,
                                           int32_t max_blocks_per_seq,
                                           const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                           const void* bias, void* out, float* lse,
                                           int32_t num_splits, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* ---- FP8 KV cache ---------------------------------------------------------
 * [A] Roadmap: FP8 for the global-attention layers, which are bound by
 * compute and by KV-cache capacity.  An FP8 cache has the layout above with
 * one byte per element (a 16 KiB tile per (block, kv-head)); each byte is the
 * OCP E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinity; largest finite value 448) of the key divided by k_scale, or of
 * the value divided by v_scale: one positive finite float scale per cache,
 * chosen by the caller (for example max |x| / 448 over a calibration set).
 * A cached element reads back as value(code) * scale.
 *
 * inkattn_sconv_fp8: inkattn_sconv writing an FP8 cache.  Each output is
 * divided by its cache's scale (as a product with the fp32 reciprocal),
 * clamped to +-448 and rounded to the nearest E4M3 value, ties to even.
 * Inputs, taps and the sconv state keep the dtype (fp32 or bf16).  Errors as
 * inkattn_sconv, plus INKATTN_EINVAL for a scale that is not positive and
 * finite or whose reciprocal overflows. */
inkattn_status_t inkattn_sconv_fp8(int32_t dtype, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_chunk_len,
                                   const void* k_in, const void* v_in, const void* conv_w,
                                   void* conv_state, const int32_t* state_slot,
                                   const int32_t* cu_seqlens, const int32_t* slot_mapping,
                                   float k_scale, float v_scale, void* k_cache, void* v_cache,
                                   void* stream);

/* inkattn_relattn_decode_mq over an FP8 cache: the same arguments and
 * results, with the keys and values read back from their codes (k_scale,
 * v_scale as written).  Queries, bias and out are bf16 (desc->dtype must be
 * INKATTN_BF16, else INKATTN_ENOTSUP); one query token per sequence is the
 * plain decode.  Split count and workspace size come from
 * inkattn_relattn_decode_mq_num_splits / _workspace_size.  Errors as
 * inkattn_relattn_decode_mq, plus INKATTN_EINVAL for a bad scale. */
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
                                            size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* inkattn_status_string(int32_t status);

/* ---- Diagnostics: measured ceilings for the roofline denominators --------
 * Not part of the attention path.  A benchmark runs them in the same job as
 * the kernels to report each kernel's fraction of what this GPU sustains
 * beside its fraction of the published peaks.  Both are asynchronous on
 * `stream` (a hipStream_t, NULL = default stream). */

#define INKATTN_PROBE_MFMA_WAVES 8
#define INKATTN_PROBE_MFMA_CHAINS 8
#define INKATTN_PROBE_READ_GROUPS 256

/* Dense bf16 MFMA loop: num_groups work-groups of INKATTN_PROBE_MFMA_WAVES
 * waves (two per SIMD), each wave running iters rounds of
 * INKATTN_PROBE_MFMA_CHAINS independent v_mfma_f32_32x32x16_bf16 chains on
 * operands with random mantissas.  Work = num_groups * iters * WAVES * CHAINS
 * * 32768 flop.
 * out: device float[3 * num_groups]; group g writes an accumulator sum (a
 * sink), then the shader-clock cycles and the 100 MHz real-time ticks of its
 * first wave's loop (cycles / ticks * 100 = sclk in MHz).
 * INKATTN_EINVAL if num_groups < 1, iters < 1 or out is NULL. */
inkattn_status_t inkattn_probe_mfma_bf16(int32_t num_groups, int32_t iters, float* out,
                                         void* stream);

/* Streaming read of `bytes` bytes of device memory at `buf` (16-byte words,
 * grid-stride, INKATTN_PROBE_READ_GROUPS work-groups of 256 threads, eight
 * 16-byte loads in flight per thread).  The memory is only read.
 * out: device float[INKATTN_PROBE_READ_GROUPS], a sink that is written only
 * if the XOR of the data read equals one fixed constant.
 * INKATTN_EINVAL if buf or out is NULL, bytes is 0, or buf / bytes are not
 * multiples of 16. */
inkattn_status_t inkattn_probe_stream_read(const void* buf, size_t bytes, float* out,
                                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INKATTN_H_ */
