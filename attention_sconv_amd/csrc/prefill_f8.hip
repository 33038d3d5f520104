// Prefill attention over an E4M3 (OCP FP8) KV cache with FP8 matrix
// products: the global-attention layers' prefill in FP8.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Roadmap (FP8 for
// the global-attention layers, whose attention is a bottleneck in compute as
// well as in KV capacity), Model Architecture / Attention and vLLM
// Integration & Optimization / FA4 with sheared bias.  The logit is the one
// of the bf16 prefill,  q_i.k_j / sqrt(128) + bias[h][min(i-j, R-1)],  over
// keys k_j = code * k_scale and values v_j = code * v_scale.
//
// Quantisation (the products run on v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3):
// * Q: one scale per work-group tile (256 query rows of one q-head): the
//   largest |q| of the tile's rows maps to 448.  s_q = amax / 448, codes
//   RNE(q * (448 / amax)) in fp32; a tile of zeros keeps s_q = 1.  The factor
//   s_q * k_scale enters the base-2 logit multiplier, and the bias band is
//   divided by it, so the MFMA accumulates  q8.k8 + bias * sqrt(128) /
//   (s_q * k_scale).
// * P: the probabilities of the online softmax (<= 2^8 under the lazy
//   rescale) are rounded to E4M3 for the PV product, and the row sums add
//   the rounded values (a product with a matrix of ones), so the output is a
//   weighted mean with exactly the weights the product used.
//
// Schedule: as the bf16 prefill (prefill.hip): 8 waves, 32 query rows each,
// ping-pong matrix and softmax phases between the two waves of a SIMD, K and
// V^T tiles of 64 keys by LDS-DMA two phases ahead, the sheared band in LDS
// loaded as the S^T accumulators' start value, lazy rescale.  What differs:
// * K and V^T stay E4M3 in LDS: 144-byte K rows and 80-byte V^T rows (9 and
//   5 slots of 16 bytes: odd, so the 32 rows a half-wave reads land on 32
//   distinct slots mod 32, which ds_read_b128 serves in one pass).
// * A matrix phase is 4 QK^T products (2 key blocks x 2 64-dim steps) and 4
//   PV products (4 dim tiles, one 64-key step) of 64 cycles each, and every
//   fragment it reads from LDS is issued at its start.
// * K rows are permuted in LDS: row 32t + 8a + 4g + c holds key
//   32g + 16t + 4a + c, so that accumulator register j of S^T block t in lane
//   group g is key 32g + 16t + j: each lane group ends with the 32
//   consecutive keys that its bytes of the P^T operand carry.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "prefill_common.h"

namespace inkattn {

namespace {

constexpr int kF8Waves = 8;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8BQ = 32 * kF8Waves;          // query rows per work-group
constexpr int kF8BK = 64;                     // keys per KV tile
constexpr int kF8Band = kF8BQ + kF8BK - 1;    // 319 distances per tile
constexpr int kF8BandPad = 336;               // band copy stride (floats)
constexpr int kF8Xcds = 8;
constexpr float kF8Slack = 8.0f;              // lazy-rescale threshold, log2 units
constexpr int kF8KRow = kHeadDim + 16;        // LDS K row, bytes (9 slots)
constexpr int kF8VRow = kF8BK + 16;           // LDS V^T row, bytes (5 slots)
constexpr int kF8KSlots = kF8KRow / 16, kF8KData = kHeadDim / 16;
constexpr int kF8VSlots = kF8VRow / 16, kF8VData = kF8BK / 16;
constexpr int kF8KLoads = kF8BK * kF8KSlots / 64;      // 9 wave loads per K tile
constexpr int kF8VLoads = kHeadDim * kF8VSlots / 64;   // 10 per V^T tile
constexpr int kF8Loaders = kF8Waves / 2;
// Tile blocks per loader: loaders 0-2 take runs of three consecutive 1 KiB
// blocks of K and of V^T (one M0 value per run: rewriting M0 costs the
// issuing wave ~110 cycles per load); loader 3 takes V^T block 9.
constexpr int kF8Run = 3;
static_assert(kF8KLoads == 3 * kF8Run && kF8VLoads == 3 * kF8Run + 1, "run layout of the tiles");
constexpr int kF8BandRaw = ((kF8Band + 2) / 2 + 63) / 64 * 64;  // dwords of a raw bf16 slice
constexpr int kF8BandLoads = kF8BandRaw / 64;
constexpr int kF8BandPer = (kF8BandLoads + kF8Loaders - 1) / kF8Loaders;
static_assert(kF8BandPad >= kF8Band + 1, "band copy stride");
static_assert(kF8BK * kF8KSlots % 64 == 0 && kHeadDim * kF8VSlots % 64 == 0,
              "tile buffers are whole wave loads");

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct alignas(16) PrefillF8Smem {
  uint8_t k[2][kF8BK * kF8KRow];              // [permuted key row][d]
  uint8_t vt[2][kHeadDim * kF8VRow];          // [d][key]
  float band[2][4][kF8BandPad];               // copy s holds band[v + s]
  uint32_t braw[2][kF8BandRaw];               // raw bf16 bias slice of a stage
  int32_t pages[2][2];                        // physical pages of a stage's K and V tiles
  float amax[kF8Waves];                       // per-wave max |q| of the tile
};

struct PrefillF8Args {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const void* bias;
  void* out;
  float* lse;
  int Hq, Hkv, G, window, R, max_blocks, num_seqs, total_groups;
  float k_scale, v_scale;
};

// Key held by LDS row r (0..63) of a K tile: r = 32t + 8a + 4g + c holds
// 32g + 16t + 4a + c (a bijection on 0..63).
__device__ __forceinline__ int f8_row_key(int r) {
  const int t = r >> 5, a = (r >> 3) & 3, g = (r >> 2) & 1, c = r & 3;
  return 32 * g + 16 * t + 4 * a + c;
}

// 32x32 output, contracts 64 E4M3 values: lane l supplies row (A) or column
// (B) l % 32 and the 32 consecutive k-values 32 (l / 32) .. +31.
__device__ __forceinline__ f32x16 mfma32_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ i32x8 lds_read32(const uint8_t* p) {   // 16-byte aligned
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// Zero the bytes of a 16-byte slot from byte n on.
__device__ __forceinline__ u32x4 keep_first_bytes(u32x4 v, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int k = n - 4 * w;                  // bytes of this word to keep
    const uint32_t mask = k >= 4 ? 0xffffffffu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
    v[w] &= mask;
  }
  return v;
}
// Four probabilities (in [0, 256], so no saturation is needed) -> E4M3 codes,
// rounded to nearest even; byte e holds value e.
__device__ __forceinline__ uint32_t f8x4_probs(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
__global__ __launch_bounds__(kF8Threads) void prefill_f8_kernel(PrefillF8Args A) {
  __shared__ PrefillF8Smem sm;

  // ---- which (sequence, q-tile, head): as the bf16 prefill
  const int id = blockIdx.x;
  const int xcd = id % kF8Xcds;
  const int local = id / kF8Xcds;
  const int e_head = local % A.G;
  const int gi = (local / A.G) * kF8Xcds + xcd;
  if (gi >= A.total_groups) return;
  const int per_rank = A.num_seqs * A.Hkv;
  const int rank = gi / per_rank;
  const int b = (gi % per_rank) / A.Hkv;
  const int kvg = gi % A.Hkv;
  const int tok0 = A.cu_q[b];
  const int q_len = A.cu_q[b + 1] - tok0;
  const int nqt = (q_len + kF8BQ - 1) / kF8BQ;
  const int qt = nqt - 1 - rank;
  if (qt < 0) return;
  const int h = kvg * A.G + e_head;
  const int seq_len = A.seq_lens[b];
  const int row0 = qt * kF8BQ;
  const int P0 = seq_len - q_len + row0;
  const int P_last = seq_len - q_len + min(row0 + kF8BQ, q_len) - 1;
  const int key_lo = A.window > 0 ? max(0, P0 - A.window + 1) : 0;
  const int jt_lo = key_lo / kF8BK;
  const int jt_hi = P_last / kF8BK;
  const int n_t = jt_hi - jt_lo + 1;
  const int n_tail = seq_len - jt_hi * kF8BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2;
  const int lq = lane & 31;
  const int lg = lane >> 5;
  const int a_row = 32 * wave + lq;
  const bool row_ok = row0 + a_row < q_len;

  const bf16* qp = static_cast<const bf16*>(A.q);
  const uint8_t* kc = static_cast<const uint8_t*>(A.k_cache);
  const uint8_t* vc = static_cast<const uint8_t*>(A.v_cache);
  const bf16* bias_h = static_cast<const bf16*>(A.bias) + (size_t)h * A.R;
  const int32_t* btab = A.block_table + (size_t)b * A.max_blocks;

  // ---- staging (the bf16 prefill's scheme, in E4M3 bytes)
  constexpr uint32_t kPageBytes = kPage * kHeadDim;
  const uint32_t bias_bytes = (uint32_t)A.Hq * (uint32_t)A.R * 2u;
  const u32x4 bias_rsrc = make_buf_rsrc(A.bias, bias_bytes);
  const u32x4 btab_rsrc = make_buf_rsrc(btab, (uint32_t)A.max_blocks * 4u);
  const int lw = wave - kF8Loaders;           // loader index (waves 4-7)
  auto page_rsrc = [&](const uint8_t* cache, int phys) {
    return make_buf_rsrc(cache + ((size_t)phys * A.Hkv + kvg) * (size_t)kPageBytes, kPageBytes);
  };
  auto page_rsrc_early = [&](const uint8_t* cache, int phys) {   // starts 4 KiB before the page
    return make_buf_rsrc(cache + ((size_t)phys * A.Hkv + kvg) * (size_t)kPageBytes - 4096,
                         kPageBytes + 4096u);
  };
  // Block j (0 .. kF8Run-1) of this loader's share, or -1.
  auto k_block = [&](int j) { return lw < 3 ? kF8Run * lw + j : -1; };
  auto v_block = [&](int j) { return lw < 3 ? kF8Run * lw + j : (j == 0 ? kF8VLoads - 1 : -1); };
  auto lds_addr = [](const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
  };
  auto band_e0 = [&](int x) {                 // first (even) bias element of stage x's slice
    const int d_lo = P0 - (jt_lo + x) * kF8BK - kF8BK + 1;
    const int e0 = h * A.R + d_lo;
    return e0 - (((e0 % 2) + 2) % 2);
  };
  auto dma_ahead = [&](int x) {
    if (lw < 0) return;
    if (x < n_t) {
#pragma unroll
      for (int j = 0; j < kF8BandPer; ++j) {
        const int n = lw + kF8Loaders * j;
        if (n < kF8BandLoads) {
          const uint32_t voff = (uint32_t)(band_e0(x) * 2) + 4u * (64 * n + lane);
          lds_dma4(bias_rsrc, lds_addr(&sm.braw[x & 1][64 * n]), voff, 0u);
        }
      }
    }
    if (x <= n_t && wave == kF8Waves - 1 && lane < 2) {
      const int jt = min(max(jt_lo + x - lane, jt_lo), jt_hi);
      lds_dma4(btab_rsrc, lds_addr(&sm.pages[x & 1][0]), (uint32_t)(jt * kF8BK / kPage) * 4u, 0u);
    }
  };
  // Byte offset in the page of the 16-byte chunk an LDS slot holds (padding
  // slots take a harmless copy of the row's last chunk).
  auto k_src = [&](int slot) {
    const int row = slot / kF8KSlots, ch = min(slot % kF8KSlots, kF8KData - 1);
    return (uint32_t)(f8_row_key(row) * kHeadDim + 16 * ch);
  };
  auto v_src = [&](int slot) {
    const int row = slot / kF8VSlots, ch = min(slot % kF8VSlots, kF8VData - 1);
    return (uint32_t)(row * kPage + 16 * ch);
  };
  auto dma_tiles = [&](int x, int k_phys, int v_phys) {
    if (lw < 0) return;
    const int ln = lane;
    if (x < n_t && lw < 3) {                  // K of tile x: one run of three blocks
      const int jt = jt_lo + x;
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kF8BK % kPage) * kHeadDim);
      const int n0 = kF8Run * lw;
      lds_dma16x3(page_rsrc_early(kc, k_phys), lds_addr(&sm.k[x & 1][0]) + 1024u * n0,
                  k_src(64 * n0 + ln) + 4096u, k_src(64 * (n0 + 1) + ln) + 3072u,
                  k_src(64 * (n0 + 2) + ln) + 2048u, soff);
    }
    if (x >= 1) {                             // V of tile x-1
      const int jt = jt_lo + x - 1;
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kF8BK % kPage));
      const uint32_t lds = lds_addr(&sm.vt[(x - 1) & 1][0]);
      if (lw < 3) {
        const int n0 = kF8Run * lw;
        lds_dma16x3(page_rsrc_early(vc, v_phys), lds + 1024u * n0, v_src(64 * n0 + ln) + 4096u,
                    v_src(64 * (n0 + 1) + ln) + 3072u, v_src(64 * (n0 + 2) + ln) + 2048u, soff);
      } else {
        const int n = kF8VLoads - 1;
        lds_dma16(page_rsrc(vc, v_phys), lds + 1024u * n, v_src(64 * n + ln), soff);
      }
    }
  };
  auto stage_pages = [&](int x, int& k_phys, int& v_phys) {
    k_phys = __builtin_amdgcn_readfirstlane(sm.pages[x & 1][0]);
    v_phys = __builtin_amdgcn_readfirstlane(sm.pages[x & 1][1]);
  };
  // Keys >= seq_len (last tile only) may hold any bits: each loader zeroes
  // them in its own slots once its loads have landed.
  auto fix_tail = [&](int x) {
    if (lw < 0 || n_tail >= kF8BK) return;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (x < n_t && jt_lo + x == jt_hi) {
      u32x4* buf = reinterpret_cast<u32x4*>(&sm.k[x & 1][0]);
#pragma unroll
      for (int j = 0; j < kF8Run; ++j) {
        const int n = k_block(j);
        const int slot = 64 * n + ln;
        if (n >= 0 && f8_row_key(slot / kF8KSlots) >= n_tail) buf[slot] = u32x4{0, 0, 0, 0};
      }
    }
    if (x >= 1 && jt_lo + x - 1 == jt_hi) {
      u32x4* buf = reinterpret_cast<u32x4*>(&sm.vt[(x - 1) & 1][0]);
#pragma unroll
      for (int j = 0; j < kF8Run; ++j) {
        const int n = v_block(j);
        const int slot = 64 * n + ln;
        const int ch = slot % kF8VSlots;
        if (n >= 0 && ch < kF8VData && 16 * (ch + 1) > n_tail)
          buf[slot] = keep_first_bytes(buf[slot], n_tail - 16 * ch);
      }
    }
  };
  float bias_last;
  float band_mul = 0.0f;                      // sqrt(128) / (s_q k_scale), set in the prologue
  // Band of stage x, written by waves 0-3 (256 threads, entries tid and
  // tid + 256): the raw bias entries are read from LDS at the start of the
  // softmax phase (band_fetch) and the four shifted copies written at its
  // end (band_write), so the LDS latency overlaps the softmax.
  constexpr int kBandPerThread = (kF8Band + kF8Threads / 2 - 1) / (kF8Threads / 2);
  auto band_dist = [&](int x, int k) {
    return P0 - (jt_lo + x) * kF8BK + (kF8BQ - 1) - (tid + (kF8Threads / 2) * k);
  };
  auto band_fetch = [&](int x, float (&bv)[kBandPerThread]) {
    const bf16* raw = reinterpret_cast<const bf16*>(&sm.braw[x & 1][0]);
    const int e0 = band_e0(x);
#pragma unroll
    for (int k = 0; k < kBandPerThread; ++k) {
      const int dist = band_dist(x, k);
      // (an index inside the slice for every lane; entries past R-1 use bias_last)
      const int idx = min(max(h * A.R + min(dist, A.R - 1) - e0, 0), 2 * kF8BandRaw - 1);
      bv[k] = to_f32(raw[idx]);
    }
  };
  auto band_write = [&](int x, const float (&bv)[kBandPerThread]) {
    if (x >= n_t) return;
#pragma unroll
    for (int k = 0; k < kBandPerThread; ++k) {
      const int v = tid + (kF8Threads / 2) * k;
      if (v < kF8Band) {
        const int dist = band_dist(x, k);
        const bool vis = dist >= 0 && (A.window == 0 || dist < A.window);
        const float b = dist > A.R - 1 ? bias_last : bv[k];
        const float band_v = vis ? b * band_mul : -INFINITY;
#pragma unroll
        for (int sh = 0; sh < 4; ++sh)            // (entries before a copy's start: a spare slot)
          sm.band[x & 1][sh][v - sh >= 0 ? v - sh : kF8BandPad - 1] = band_v;
      }
    }
  };
  auto band_store = [&](int x) {
    float bv[kBandPerThread];
    band_fetch(x, bv);
    band_write(x, bv);
  };

  // ---- running softmax state
  float m_used = -INFINITY;
  f32x16 o[4];
  // Row sums as one more product: a matrix of E4M3 ones times P^T puts the
  // sum of the rounded probabilities of a query row in every register of its
  // column, and rescales with O.  (On the vector ALU the decode and the adds
  // cost ~40 instructions per tile in the softmax phase, which is the longer
  // of the two phases.)
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
  const i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  f32x16 acc[2];
  bool rescale = false;
  float alpha = 1.0f;
  i32x8 pf;                                   // P^T (E4M3) between softmax and matrix phase
  i32x8 qf[2];                                // Q^T (E4M3): dims 64 ks + 32 lg .. +31
  float c = 0.0f;                             // log2(e) s_q k_scale / sqrt(128)
  const int band_shift = (3 - (lane & 3)) & 3;

  // Matrix phase of tile i: S^T_i = K_i Q^T from the band, and O^T +=
  // V^T_{i-1} P^T_{i-1}.  The first phase multiplies a zero P^T with a zeroed
  // V buffer.
  // kQK false: the closing phase (i = n_t), PV of the last tile only (there
  // is no tile n_t whose S^T would be computed).
  auto matrix_phase = [&](int i, auto qk_tag) {
    constexpr bool kQK = decltype(qk_tag)::value;
    const int kb = i & 1, vb = (i - 1) & 1;
    // LDS reads in the order the products need them (they return in order):
    // block t's band and K fragments, then V^T.
    i32x8 kf[2][2], vf[4];
#pragma unroll
    for (int t = 0; t < 2 && kQK; ++t) {
      const int v0 = (kF8BQ - 1) - a_row + 32 * lg + 16 * t;
      const float* bp = &sm.band[kb][band_shift][v0 - band_shift];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(bp + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][4 * q4 + e] = x[e];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kf[t][ks] = lds_read32(&sm.k[kb][(32 * t + lq) * kF8KRow + 64 * ks + 32 * lg]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) vf[dt] = lds_read32(&sm.vt[vb][(32 * dt + lq) * kF8VRow + 32 * lg]);
    if (rescale) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) asm("v_mul_f32 %0, %1, %0" : "+v"(o[dt][r]) : "v"(alpha));
#pragma unroll
      for (int r = 0; r < 16; ++r) asm("v_mul_f32 %0, %1, %0" : "+v"(lacc[r]) : "v"(alpha));
      rescale = false;
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kQK) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) acc[t] = mfma32_f8(kf[t][ks], qf[ks], acc[t]);
    }
    lacc = mfma32_f8(ones, pf, lacc);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32_f8(vf[dt], pf, o[dt]);
  };

  // Softmax phase: online softmax in base 2 with a lazy rescale; P rounded
  // to E4M3 (its row sum follows in the next matrix phase).
  auto softmax_phase = [&]() {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[t][r]);
    mx = pair_max(mx);
    const float m_tile = mx * c;
    const bool need = m_tile > m_used + kF8Slack;
    rescale = __any(need);
    if (rescale) {
      alpha = need ? fast_exp2(m_used - m_tile) : 1.0f;
      m_used = need ? m_tile : m_used;
    }
    const float msub = m_used == -INFINITY ? 0.0f : m_used;
#pragma unroll
    for (int w = 0; w < 8; ++w) {             // word w: keys 32 lg + 4w .. +3
      const int t = w >> 2, r0 = 4 * (w & 3);
      pf[w] = (int)f8x4_probs(fast_exp2(acc[t][r0] * c - msub),
                              fast_exp2(acc[t][r0 + 1] * c - msub),
                              fast_exp2(acc[t][r0 + 2] * c - msub),
                              fast_exp2(acc[t][r0 + 3] * c - msub));
    }
  };

  // V buffer 1 is read (times P^T = 0) by the first matrix phase.
  {
    u32x4* vz = reinterpret_cast<u32x4*>(&sm.vt[1][0]);
    constexpr int kVBufSlots = kHeadDim * kF8VRow / 16;
    for (int i = tid; i < kVBufSlots; i += kF8Threads) vz[i] = u32x4{0, 0, 0, 0};
  }
  pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

  // ---- prologue: Q (bf16) of this lane's 64 dims, the first stages.
  Frag8<bf16> qb[2][4];                       // dims 64 ks + 32 lg + 8 j .. +7
  {
    int k0 = 0;
    if (half == 1) k0 = __builtin_amdgcn_readfirstlane(btab[jt_lo * kF8BK / kPage]);
    bias_last = to_f32(bias_h[A.R - 1]);
    const bf16* qrow = qp + ((size_t)(tok0 + row0 + a_row) * A.Hq + h) * kHeadDim + 32 * lg;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        qb[ks][j] = row_ok ? Frag8<bf16>::load(qrow + 64 * ks + 8 * j) : Frag8<bf16>::zero();
    if (half == 1) {
      keep_live(k0);
      dma_ahead(0);
      dma_ahead(1);
      dma_tiles(0, k0, 0);
    }
  }
  wait_all_loads();
  keep_live(bias_last);
  {
    float am = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(qb[ks][j].get(e)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, wave_shfl_xor(am, off));
    if (lane == 0) sm.amax[wave] = am;
  }
  __syncthreads();                            // slices 0-1, pages of stage 1, amax
  {
    float am = 0.0f;
#pragma unroll
    for (int w = 0; w < kF8Waves; ++w) am = fmaxf(am, sm.amax[w]);
    const float inv = am > 0.0f ? kFp8Max / am : 1.0f;
    const float s_q = am > 0.0f ? am / kFp8Max : 1.0f;
    const float sqrt_d = 11.313708498984761f;
    c = kLog2e / sqrt_d * A.k_scale * s_q;
    band_mul = sqrt_d / (A.k_scale * s_q);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const Frag8<bf16>& f = qb[ks][j];
        qf[ks][2 * j] = (int)fp8x4_from_f32(f.get(0) * inv, f.get(1) * inv, f.get(2) * inv,
                                            f.get(3) * inv);
        qf[ks][2 * j + 1] = (int)fp8x4_from_f32(f.get(4) * inv, f.get(5) * inv, f.get(6) * inv,
                                                f.get(7) * inv);
      }
  }
  if (half == 1) fix_tail(0); else band_store(0);
  __syncthreads();                            // stage 0 published
  if (half == 1) {
    int kp1, vp1;
    stage_pages(1, kp1, vp1);
    dma_ahead(2);
    dma_tiles(1, kp1, vp1);
  }

  // ---- phase loop (the bf16 prefill's ping-pong)
  if (half == 1) __syncthreads();
  for (int i = 0;; ++i) {
    if (i == n_t) {
      matrix_phase(i, std::false_type{});
      break;
    }
    matrix_phase(i, std::true_type{});
    if (half == 0) {
      __syncthreads();
      float bv[kBandPerThread];
      band_fetch(i + 1, bv);
      softmax_phase();
      band_write(i + 1, bv);
      __syncthreads();
    } else {
      wait_all_loads();
      fix_tail(i + 1);
      __syncthreads();
      if (i + 1 < n_t) {
        int kp, vp;
        stage_pages(i + 2, kp, vp);
        dma_ahead(i + 3);
        dma_tiles(i + 2, kp, vp);
      }
      softmax_phase();
      __syncthreads();
    }
  }
  if (half == 0) __syncthreads();

  // ---- epilogue: O^T register r of tile dt is dim 32dt + 8(r/4) + 4lg + r%4
  const float lt = lacc[0];                   // (every register holds the row sum)
  if (!row_ok) return;
  const float inv = A.v_scale / lt;
  bf16* op = static_cast<bf16*>(A.out) + ((size_t)(tok0 + row0 + a_row) * A.Hq + h) * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      store4(op + 32 * dt + 8 * q4 + 4 * lg, o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv,
             o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
  if (A.lse != nullptr && lg == 0)
    A.lse[(size_t)(tok0 + row0 + a_row) * A.Hq + h] = (m_used + fast_log2(lt)) * kLn2;
}

}  // namespace

hipError_t launch_prefill_f8(const AttnShape& s, int num_seqs, int max_q_len, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int max_blocks_per_seq,
                             const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                             const void* bias, void* out, float* lse, hipStream_t stream,
                             float k_scale, float v_scale) {
  PrefillF8Args a;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
  a.cu_q = cu_seqlens_q; a.seq_lens = seq_lens; a.bias = bias; a.out = out; a.lse = lse;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.Hq / s.Hkv; a.window = s.window; a.R = s.bias_len;
  a.max_blocks = max_blocks_per_seq; a.num_seqs = num_seqs;
  const int nqt = (max_q_len + kF8BQ - 1) / kF8BQ;
  a.total_groups = nqt * num_seqs * s.Hkv;
  const long padded = ((long)a.total_groups + kF8Xcds - 1) / kF8Xcds * kF8Xcds;
  const long blocks = padded * a.G;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_f8_kernel, dim3((unsigned)blocks), dim3(kF8Threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace inkattn
