// Short convolution (window 4, causal, depthwise) of keys and values, fused
// with the write into the paged KV cache and the update of the three-token
// state cache.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Model Architecture /
// Sconv (window-4 short convolution over the attention key and value
// channels) and vLLM Integration & Optimization / Managing the sconv cache
// (the last W-1 tokens are kept).  The cached rows are the pre-convolution
// inputs; tap 3 weights the current token.
//
// Work split: a wave covers 64 tokens x 64 channels of one sequence, lane l
// the tokens 8*(l%8) .. +7 and the channels 8*(l/8) .. +7 of that block
// (one 16-byte bf16 vector of each token, two for fp32).  It loads the 8
// tokens and the 3-token halo before them up front, so all loads are in
// flight together and the halo rows are ones its neighbouring lanes read
// too; the 4-tap window then runs in registers.  With this lane order one
// store instruction of the transposed V cache writes 8 rows x 64 tokens,
// whole 128-byte lines, and a K-cache store 8 tokens x 64 channels.  Work-
// groups are dealt so that those one XCD runs together are neighbours in the
// token order (their halos come from that XCD's L2).  Only the lane that
// handles a sequence's first chunk touches that sequence's state, so the
// in-place state update is race-free.
// Memory-bound: every input byte is read once (plus a 3-row halo per 8
// tokens, mostly from the caches) and every output byte written once.
//
// Paged state (kPaged): the pre-convolution rows of every token are kept in a
// paged cache of their own, [block][128 tokens][Hkv*128 channels], addressed
// through a block table like the K/V cache: the sconv cache as the K/V cache
// of a virtual sliding-window layer of window 3 (vLLM Integration &
// Optimization / Managing the sconv cache: blocks older than the window can
// be evicted, and prefix caching covers the sconv state too).  A chunk at
// positions ctx .. ctx+n-1 reads its halo ctx-3 .. ctx-1 from there (zero
// before position 0) and writes its own rows there.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace inkattn {

constexpr int kSconvTok = 8;          // tokens per thread
// 256 threads per work-group: a thread holds 11 rows of 8 channels and 64
// fp32 outputs, more than the 128 VGPRs a 1024-thread bound leaves.
constexpr int kSconvThreads = 256;
// K/V cache write: a work-group covers 128 tokens x one head (128 channels)
// of K or V, waves (token half, channel half).  Output sconv: 64 tokens x 256
// channels, waves side by side in channels.
constexpr int kWriteTok = 128;
constexpr int kOutTok = 64;
constexpr int kOutCh = 256;

// Work-group id -> linear work index.  The dispatcher deals ids round-robin
// over the 8 XCDs; index (id % 8) * per + id / 8 gives each XCD a contiguous
// range of the work, token blocks fastest.
__device__ __forceinline__ int xcd_work_index(int id, int per) { return (id & 7) * per + (id >> 3); }

// Paged-state arguments (unused by the dense-state kernel).
struct SconvPaged {
  const int32_t* seq_lens;        // chunk of sequence b ends at position seq_lens[b]-1
  const int32_t* block_table;     // [num_seqs][max_blocks] blocks of the state cache
  int max_blocks;
  void* k_state;                  // [blocks][128][C] pre-convolution keys
  void* v_state;                  // [blocks][128][C] pre-convolution values
};

// FP8 cache (TC = fp8e4): the outputs are stored as E4M3 codes of y / scale;
// inv_scale[0|1] = 1 / scale of the key | value cache.
template <typename T, typename TC, bool kPaged>
__global__ __launch_bounds__(kSconvThreads) void sconv_cache_write_kernel(
    int C, int Hkv, const T* __restrict__ k_in, const T* __restrict__ v_in,
    const T* __restrict__ conv_w, T* __restrict__ conv_state,
    const int32_t* __restrict__ state_slot, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ slot_mapping, TC* __restrict__ k_cache,
    TC* __restrict__ v_cache, SconvPaged pg, float inv_scale_k, float inv_scale_v, int ntb,
    int num_seqs, int per) {
  constexpr bool kFp8 = std::is_same<TC, fp8e4>::value;
  // work index -> (token block, sequence, K|V and head)
  const int wi = xcd_work_index(blockIdx.x, per);
  if (wi >= ntb * num_seqs * 2 * Hkv) return;
  const int tb = wi % ntb;
  const int b = (wi / ntb) % num_seqs;
  const int z = wi / (ntb * num_seqs);
  const int which = z / Hkv;                 // 0 = keys, 1 = values
  const int head = z % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = kWriteTok * tb + 64 * (wave >> 1) + kSconvTok * (lane & 7);   // first token (relative)
  const int c0 = kHeadDim * head + 64 * (wave & 1) + 8 * (lane >> 3);
  const int t_begin = cu_seqlens[b];
  const int n = cu_seqlens[b + 1] - t_begin;
  if (r0 >= n || c0 >= C) return;

  const T* x = (which ? v_in : k_in) + (size_t)t_begin * C + c0;
  const T* wp = conv_w + ((size_t)which * C + c0) * 4;
  T* st = kPaged ? nullptr : conv_state + ((size_t)state_slot[b] * 2 + which) * 3 * C + c0;
  // Paged state: position of the chunk's first token, and the slot of a
  // position in the state cache.
  const int ctx = kPaged ? pg.seq_lens[b] - n : 0;
  T* pst = kPaged ? static_cast<T*>(which ? pg.v_state : pg.k_state) + c0 : nullptr;
  auto state_row = [&](int p) {
    const int32_t blk = pg.block_table[(size_t)b * pg.max_blocks + (p >> 7)];
    return pst + ((size_t)blk * kPage + (p & (kPage - 1))) * C;
  };

  // All inputs of the chunk and its 3-token halo are loaded up front (the
  // halo before the chunk comes from the cached state).
  Frag8<T> xs[kSconvTok + 3];
#pragma unroll
  for (int k = 0; k < kSconvTok + 3; ++k) {
    const int rel = r0 - 3 + k;
    if (rel >= 0)
      xs[k] = rel < n ? Frag8<T>::load(x + (size_t)rel * C) : Frag8<T>::zero();
    else if (!kPaged)
      xs[k] = Frag8<T>::load(st + (size_t)(rel + 3) * C);
    else
      xs[k] = ctx + rel >= 0 ? Frag8<T>::load(state_row(ctx + rel)) : Frag8<T>::zero();
  }
  int slot[kSconvTok];
#pragma unroll
  for (int t = 0; t < kSconvTok; ++t)
    slot[t] = r0 + t < n ? slot_mapping[t_begin + r0 + t] : -1;

  float w[8][4];
  {
    const Frag8<T> f0 = Frag8<T>::load(wp), f1 = Frag8<T>::load(wp + 8),
                   f2 = Frag8<T>::load(wp + 16), f3 = Frag8<T>::load(wp + 24);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const Frag8<T>& f = e < 2 ? f0 : e < 4 ? f1 : e < 6 ? f2 : f3;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[e][k] = f.get((e & 1) * 4 + k);
    }
  }

  float y[kSconvTok][8];
#pragma unroll
  for (int t = 0; t < kSconvTok; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      y[t][e] = w[e][0] * xs[t].get(e) + w[e][1] * xs[t + 1].get(e) +
                w[e][2] * xs[t + 2].get(e) + w[e][3] * xs[t + 3].get(e);

  const int kvh = c0 / kHeadDim;
  const int dd = c0 % kHeadDim;
  // 8 outputs -> 8 cache elements at p (one 16-byte bf16 / 32-byte fp32
  // store, or 8 E4M3 codes in one 8-byte store).  Single elements (the V^T
  // column of a token that is not part of an aligned run of 8, as in a
  // decode step) are stored nontemporally in bf16 and E4M3: they are 2-byte
  // pieces of many lines, and the decode right after the step reads those
  // lines faster when they do not sit partly dirty in the caches (16K SWA
  // decode after its sconv: 0.096 -> 0.095 ms).  Whole 8-element stores stay
  // ordinary: nontemporal, they slowed an 8K-token prefill write by 40%.
  const float inv = which ? inv_scale_v : inv_scale_k;
  auto store8 = [&](TC* p, const float* v8) {
    if constexpr (kFp8) {
      *reinterpret_cast<u32x2*>(p) =
          u32x2{fp8x4_from_f32(v8[0] * inv, v8[1] * inv, v8[2] * inv, v8[3] * inv),
                fp8x4_from_f32(v8[4] * inv, v8[5] * inv, v8[6] * inv, v8[7] * inv)};
    } else {
      Frag8<T>::pack(v8).store(p);
    }
  };
  auto store1 = [&](TC* p, float v) {
    if constexpr (kFp8)
      __builtin_nontemporal_store(
          (uint8_t)(fp8x4_from_f32(v * inv, 0.0f, 0.0f, 0.0f) & 0xffu), &p->bits);
    else if constexpr (std::is_same<T, bf16>::value)
      __builtin_nontemporal_store(from_f32<T>(v).bits, &p->bits);
    else
      *p = from_f32<T>(v);
  };
  if (which == 0) {
#pragma unroll
    for (int t = 0; t < kSconvTok; ++t) {
      if (slot[t] < 0) continue;
      const size_t tile = (size_t)(slot[t] >> 7) * Hkv + kvh;
      store8(k_cache + (tile * kPage + (slot[t] & (kPage - 1))) * kHeadDim + dd, y[t]);
    }
  } else {
    // V is stored transposed per page.  When the 8 tokens occupy 8
    // consecutive slots starting at a multiple of 8 (always the case for a
    // fresh prefill), each channel's 8 values are one 16-byte store;
    // otherwise they are scattered element by element.
    bool run = slot[0] >= 0 && (slot[0] & 7) == 0;
#pragma unroll
    for (int t = 1; t < kSconvTok; ++t) run = run && slot[t] == slot[0] + t;
    if (run) {
      const size_t tile = (size_t)(slot[0] >> 7) * Hkv + kvh;
      TC* vt = v_cache + (tile * kHeadDim + dd) * kPage + (slot[0] & (kPage - 1));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float col[kSconvTok];
#pragma unroll
        for (int t = 0; t < kSconvTok; ++t) col[t] = y[t][e];
        store8(vt + (size_t)e * kPage, col);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kSconvTok; ++t) {
        if (slot[t] < 0) continue;
        const size_t tile = (size_t)(slot[t] >> 7) * Hkv + kvh;
        TC* vt = v_cache + (tile * kHeadDim + dd) * kPage + (slot[t] & (kPage - 1));
#pragma unroll
        for (int e = 0; e < 8; ++e) store1(vt + (size_t)e * kPage, y[t][e]);
      }
    }
  }

  if constexpr (kPaged) {
    // This thread's tokens' inputs go to the state cache (rows the halo
    // reads of this call are all before the chunk, so nothing read here is
    // written here).
#pragma unroll
    for (int t = 0; t < kSconvTok; ++t)
      if (r0 + t < n) xs[t + 3].store(state_row(ctx + r0 + t));
  } else if (r0 == 0) {
    // New state = last three rows of [old state; sequence inputs].  Only the
    // thread that owns the first chunk touches the state.
    Frag8<T> ns[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int rel = n - 3 + k;
      ns[k] = rel >= 0 ? Frag8<T>::load(x + (size_t)rel * C)
                       : Frag8<T>::load(st + (size_t)(rel + 3) * C);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) ns[k].store(st + (size_t)k * C);
  }
}

// Short convolution of a plain activation tensor [tokens][C] (the attention
// output or the MoE output: Model Architecture / Sconv names four sconv
// modules per layer, on keys, values, attention output and MoE output), with
// the dense three-token state [slots][3][C].  Same work split as above: each
// thread owns 8 channels and kSconvTok tokens of one sequence.
template <typename T>
__global__ __launch_bounds__(kSconvThreads) void sconv_out_kernel(
    int C, const T* __restrict__ x_in, const T* __restrict__ conv_w, T* __restrict__ conv_state,
    const int32_t* __restrict__ state_slot, const int32_t* __restrict__ cu_seqlens,
    T* __restrict__ y_out, int ntb, int num_seqs, int per) {
  // work index -> (token block, sequence, channel block)
  const int wi = xcd_work_index(blockIdx.x, per);
  const int ncb = (C + kOutCh - 1) / kOutCh;
  if (wi >= ntb * num_seqs * ncb) return;
  const int tb = wi % ntb;
  const int b = (wi / ntb) % num_seqs;
  const int cb = wi / (ntb * num_seqs);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = kOutTok * tb + kSconvTok * (lane & 7);                 // first token (relative)
  const int c0 = kOutCh * cb + 64 * wave + 8 * (lane >> 3);
  const int t_begin = cu_seqlens[b];
  const int n = cu_seqlens[b + 1] - t_begin;
  if (r0 >= n || c0 >= C) return;
  const T* x = x_in + (size_t)t_begin * C + c0;
  T* y = y_out + (size_t)t_begin * C + c0;
  T* st = conv_state + (size_t)state_slot[b] * 3 * C + c0;

  Frag8<T> xs[kSconvTok + 3];
#pragma unroll
  for (int k = 0; k < kSconvTok + 3; ++k) {
    const int rel = r0 - 3 + k;
    xs[k] = rel < 0 ? Frag8<T>::load(st + (size_t)(rel + 3) * C)
                    : (rel < n ? Frag8<T>::load(x + (size_t)rel * C) : Frag8<T>::zero());
  }
  float w[8][4];
  {
    const T* wp = conv_w + (size_t)c0 * 4;
    const Frag8<T> f0 = Frag8<T>::load(wp), f1 = Frag8<T>::load(wp + 8),
                   f2 = Frag8<T>::load(wp + 16), f3 = Frag8<T>::load(wp + 24);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const Frag8<T>& f = e < 2 ? f0 : e < 4 ? f1 : e < 6 ? f2 : f3;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[e][k] = f.get((e & 1) * 4 + k);
    }
  }
#pragma unroll
  for (int t = 0; t < kSconvTok; ++t) {
    if (r0 + t >= n) break;
    float yt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      yt[e] = w[e][0] * xs[t].get(e) + w[e][1] * xs[t + 1].get(e) +
              w[e][2] * xs[t + 2].get(e) + w[e][3] * xs[t + 3].get(e);
    Frag8<T>::pack(yt).store(y + (size_t)(r0 + t) * C);
  }
  if (r0 == 0) {
    // New state = last three rows of [old state; inputs]; only the thread
    // that owns the first chunk touches the state.
    Frag8<T> ns[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int rel = n - 3 + k;
      ns[k] = rel >= 0 ? Frag8<T>::load(x + (size_t)rel * C)
                       : Frag8<T>::load(st + (size_t)(rel + 3) * C);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) ns[k].store(st + (size_t)k * C);
  }
}

hipError_t launch_sconv_out(int dtype, int C, int num_seqs, int max_chunk_len, const void* x,
                            const void* conv_w, void* conv_state, const int32_t* state_slot,
                            const int32_t* cu_seqlens, void* y, hipStream_t stream) {
  const int ntb = (max_chunk_len + kOutTok - 1) / kOutTok;
  const long work = (long)ntb * num_seqs * ((C + kOutCh - 1) / kOutCh);
  if (work > 0x7ffffff0L) return hipErrorInvalidConfiguration;
  const int per = (int)((work + 7) / 8);
  const dim3 grid((unsigned)(8L * per)), block(kSconvThreads);
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL(sconv_out_kernel<bf16>, grid, block, 0, stream, C, (const bf16*)x,
                       (const bf16*)conv_w, (bf16*)conv_state, state_slot, cu_seqlens, (bf16*)y,
                       ntb, num_seqs, per);
  else
    hipLaunchKernelGGL(sconv_out_kernel<float>, grid, block, 0, stream, C, (const float*)x,
                       (const float*)conv_w, (float*)conv_state, state_slot, cu_seqlens,
                       (float*)y, ntb, num_seqs, per);
  return hipGetLastError();
}

template <bool kPaged>
hipError_t launch_sconv_any(int dtype, int Hkv, int num_seqs, int max_chunk_len,
                            const void* k_in, const void* v_in, const void* conv_w,
                            void* conv_state, const int32_t* state_slot,
                            const int32_t* cu_seqlens, const int32_t* slot_mapping,
                            void* k_cache, void* v_cache, const SconvPaged& pg,
                            const float* fp8_scales, hipStream_t stream) {
  const int C = Hkv * kHeadDim;
  const int ntb = (max_chunk_len + kWriteTok - 1) / kWriteTok;
  const long work = (long)ntb * num_seqs * 2 * Hkv;
  if (work > 0x7ffffff0L) return hipErrorInvalidConfiguration;
  const int per = (int)((work + 7) / 8);
  const dim3 grid((unsigned)(8L * per)), block(kSconvThreads);
  auto go = [&](auto t_tag, auto c_tag) {
    using T = decltype(t_tag);
    using TC = decltype(c_tag);
    const float ik = fp8_scales ? 1.0f / fp8_scales[0] : 1.0f;
    const float iv = fp8_scales ? 1.0f / fp8_scales[1] : 1.0f;
    hipLaunchKernelGGL((sconv_cache_write_kernel<T, TC, kPaged>), grid, block, 0, stream, C,
                       Hkv, (const T*)k_in, (const T*)v_in, (const T*)conv_w, (T*)conv_state,
                       state_slot, cu_seqlens, slot_mapping, (TC*)k_cache, (TC*)v_cache, pg,
                       ik, iv, ntb, num_seqs, per);
  };
  if constexpr (!kPaged) {
    if (fp8_scales != nullptr) {
      if (dtype == kDtypeBf16) go(bf16{}, fp8e4{});
      else go(0.0f, fp8e4{});
      return hipGetLastError();
    }
  }
  if (dtype == kDtypeBf16) go(bf16{}, bf16{});
  else go(0.0f, 0.0f);
  return hipGetLastError();
}

hipError_t launch_sconv(int dtype, int Hkv, int num_seqs, int max_chunk_len,
                        const void* k_in, const void* v_in, const void* conv_w,
                        void* conv_state, const int32_t* state_slot,
                        const int32_t* cu_seqlens, const int32_t* slot_mapping,
                        void* k_cache, void* v_cache, const float* fp8_scales,
                        hipStream_t stream) {
  return launch_sconv_any<false>(dtype, Hkv, num_seqs, max_chunk_len, k_in, v_in, conv_w,
                                 conv_state, state_slot, cu_seqlens, slot_mapping, k_cache,
                                 v_cache, SconvPaged{nullptr, nullptr, 0, nullptr, nullptr},
                                 fp8_scales, stream);
}

hipError_t launch_sconv_paged(int dtype, int Hkv, int num_seqs, int max_chunk_len,
                              const void* k_in, const void* v_in, const void* conv_w,
                              const int32_t* cu_seqlens, const int32_t* seq_lens,
                              const int32_t* state_block_table, int max_state_blocks,
                              void* k_state, void* v_state, const int32_t* slot_mapping,
                              void* k_cache, void* v_cache, hipStream_t stream) {
  return launch_sconv_any<true>(dtype, Hkv, num_seqs, max_chunk_len, k_in, v_in, conv_w,
                                nullptr, nullptr, cu_seqlens, slot_mapping, k_cache, v_cache,
                                SconvPaged{seq_lens, state_block_table, max_state_blocks,
                                           k_state, v_state},
                                nullptr, stream);
}

}  // namespace inkattn
