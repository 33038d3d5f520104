// Prefill attention with a sheared (Toeplitz) relative-position bias.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Model Architecture /
// Attention (GQA with head size 128; sliding-window and full causal layers;
// a learned relative-position term added to the pre-softmax logits instead of
// RoPE) and vLLM Integration & Optimization / FA4 with sheared bias (the
// relative term disturbs the attention kernel's memory access; the fix is a
// "sheared" bias that follows the diagonal structure).  The logit used here
// is  q_i.k_j / sqrt(128) + bias[h][min(i-j, R-1)].
//
// Design (gfx950, one work-group = 8 waves = 256 query rows of one q-head):
// * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (fp32 storage:
//   v_mfma_f32_32x32x2_f32 on the same fragments).  Wave w owns query rows
//   32w .. 32w+31 as the 32 MFMA columns, so every softmax row statistic is
//   one lane plus its partner 32 lanes away.
// * Ping-pong phases: a wave alternates matrix phases (QK^T of tile i with
//   the PV of tile i-1) and softmax phases (tile i).  Waves 4-7 run one phase
//   behind waves 0-3 and a barrier closes every phase, so the two waves that
//   share a SIMD are always in opposite phases and the matrix cores and the
//   vector ALU work at the same time.
// * K and V^T tiles of 64 keys go global -> LDS by buffer loads with the
//   LDS-DMA flag (no staging registers) into padded rows (conflict-free
//   fragment reads at fixed offsets), double-buffered; a tile's loads have
//   two phases to land.
// * Sheared bias: for a (256-query, 64-key) tile the relative distances form
//   a band of 319 values.  The band, pre-multiplied by sqrt(128) and holding
//   -inf where the key is outside the causal window, is written to LDS once
//   per tile (four copies shifted by one entry so every lane's eight
//   consecutive distances are one aligned 32-byte read) and loaded straight
//   into the S^T accumulators before the QK^T MFMAs.  The MFMA then returns
//   q.k + sqrt(128)*bias (or -inf), and a single FMA with log2(e)/sqrt(128)
//   gives the base-2 logit: bias add and masking cost no extra ALU work.
// * Window tile skipping: only KV tiles intersecting
//   [first_query - W + 1, last_query] are visited.
// * Online softmax in base 2 with a lazy rescale: the running max only moves
//   (and O is only rescaled) when a tile's max exceeds it by more than 8, so
//   probabilities stay <= 2^8.
// * Work order: work-groups are numbered longest-first (q-tiles counted from
//   the end of each sequence) and the 8 q-heads of one GQA group land on the
//   same XCD (hardware dispatches work-group ids round-robin over the 8
//   XCDs), so they share K/V in that XCD's L2.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "prefill_common.h"

namespace inkattn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;         // query rows per work-group (32 per wave)
constexpr int kBK = 64;                  // keys per KV tile
constexpr int kBand = kBQ + kBK - 1;     // 319 distinct distances per tile
// Copy stride of the band in LDS: 336 words = 16 (mod 64), so the four
// copies start 4 bank groups apart (the band reads count no bank conflicts).
constexpr int kBandPad = 336;
static_assert(kBandPad >= kBand + 1 && kBandPad % 64 == 16, "band copy stride");
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;    // log2 units
static_assert((kBQ - 1) % 4 == 3, "band copy selection assumes kBQ % 4 == 0");
static_assert(kBand <= kThreads, "one band entry per thread");

// LDS rows are padded by one 16-byte bf16 fragment: a K row is 272 B, a V^T
// row 144 B.  A half-wave reads one fragment column from 32 distinct rows,
// which start at 16-byte slot 17r (K) or 9r (V^T): 32 distinct slots mod 32,
// a pattern a probe of ds_read_b128 times at full rate (rows of an even slot
// count run at two thirds of it).  The bank-conflict counter reads 0 for
// this kernel.  Unlike an XOR swizzle, padding keeps every fragment read at
// (per-lane base + compile-time offset), so the LDS reads cost no address
// arithmetic.
constexpr int kKStride = kHeadDim + 8;   // elements per K row in LDS
constexpr int kVStride = kBK + 8;        // elements per V^T row in LDS

// Raw bias slice of one stage: the kBand distances of a tile, fetched as
// whole dwords (from a dword-aligned start) by whole wave loads.
template <typename T>
constexpr int band_raw_dwords() {
  constexpr int epd = 4 / (int)sizeof(T);                       // elements per dword
  constexpr int dwords = (kBand + epd - 1 + epd - 1) / epd;     // + alignment slack
  return (dwords + 63) / 64 * 64;
}

template <typename T>
struct PrefillSmem {
  T k[2][kBK * kKStride];                // [key][d]
  T vt[2][kHeadDim * kVStride];          // [d][key]
  float band[2][4][kBandPad];            // copy s holds band[v + s]
  uint32_t braw[2][band_raw_dwords<T>()];  // raw bias slice of a stage
  int32_t pages[2][2];                   // physical pages of a stage's K and V tiles
};

struct PrefillArgs {
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
  // Cache scales (read by the kScaled instance only): the cache holds
  // keys / k_scale and values / v_scale.
  float k_scale, v_scale;
};

// Row r of a 32-row S^T tile holds key keyperm(r): accumulator register j of
// lane group g then holds key 16*(j/8) + 8*g + j%8 (see device_common.h for
// the accumulator layout), i.e. each lane owns runs of 8 consecutive keys,
// which is the B-operand layout the P^T V^T product needs.
__device__ __forceinline__ int keyperm(int r) {
  const int a = r >> 3, g = (r >> 2) & 1, c = r & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + c;
}

// Keep the first n elements of a 16-byte slot of T, zero the rest.
template <typename T> __device__ __forceinline__ u32x4 keep_first_elems(u32x4 v, int n);
template <> __device__ __forceinline__ u32x4 keep_first_elems<bf16>(u32x4 v, int n) {
  Frag8<bf16> f; f.v = v; return f.keep_first(n).v;
}
template <> __device__ __forceinline__ u32x4 keep_first_elems<float>(u32x4 v, int n) {
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = e < n ? v[e] : 0u;
  return v;
}

// kScaled: apply the cache scales of A (a separate instance, so that the
// kernel for a cache of the values themselves is compiled exactly without
// them: the runtime factors cost that kernel ~3% through its schedule).
template <typename T, bool kScaled>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs A) {
  __shared__ PrefillSmem<T> sm;

  // ---- which (sequence, q-tile, head) this work-group computes
  const int id = blockIdx.x;
  const int xcd = id % kXcds;
  const int local = id / kXcds;
  const int e_head = local % A.G;
  const int gi = (local / A.G) * kXcds + xcd;
  if (gi >= A.total_groups) return;
  const int per_rank = A.num_seqs * A.Hkv;
  const int rank = gi / per_rank;              // 0 = last q-tile of each sequence
  const int b = (gi % per_rank) / A.Hkv;
  const int kvg = gi % A.Hkv;
  const int tok0 = A.cu_q[b];
  const int q_len = A.cu_q[b + 1] - tok0;
  const int nqt = (q_len + kBQ - 1) / kBQ;
  const int qt = nqt - 1 - rank;
  if (qt < 0) return;
  const int h = kvg * A.G + e_head;
  const int seq_len = A.seq_lens[b];
  const int row0 = qt * kBQ;
  const int P0 = seq_len - q_len + row0;                   // position of row 0 of the tile
  const int P_last = seq_len - q_len + min(row0 + kBQ, q_len) - 1;
  const int key_lo = A.window > 0 ? max(0, P0 - A.window + 1) : 0;
  const int jt_lo = key_lo / kBK;
  const int jt_hi = P_last / kBK;
  const int n_t = jt_hi - jt_lo + 1;                       // KV tiles visited (>= 1)
  const int n_tail = seq_len - jt_hi * kBK;                // valid keys of the last tile

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2;        // 0: waves 0-3; 1: waves 4-7, one phase behind
  const int lq = lane & 31;          // query column within the wave
  const int lg = lane >> 5;          // lane group (k-half)
  const int a_row = 32 * wave + lq;  // query row within the tile
  const bool row_ok = row0 + a_row < q_len;

  const T* qp = static_cast<const T*>(A.q);
  const T* kc = static_cast<const T*>(A.k_cache);
  const T* vc = static_cast<const T*>(A.v_cache);
  const T* bias_h = static_cast<const T*>(A.bias) + (size_t)h * A.R;
  const int32_t* btab = A.block_table + (size_t)b * A.max_blocks;

  // Q^T fragments (B operand): d = 16*ks + 8*lg + e.
  // Loaded in the prologue, together with the first stage.
  Frag8<T> qf[8];

  const float sqrt_d = 11.313708498984761f;               // sqrt(128)
  const float c = kScaled ? kLog2e / sqrt_d * A.k_scale : kLog2e / sqrt_d;
  const float band_mul = kScaled ? sqrt_d / A.k_scale : sqrt_d;   // bias in units of raw q.k

  // ---- staging.  Stage s holds K and the bias band of tile s and V of tile
  // s-1 (stage n_t holds only V of the last tile): V is consumed one tile
  // after K.  Every per-stage read of global memory is a buffer load with
  // the LDS-DMA flag (lane l of a wave's load writes its bytes at slot l of
  // the destination): K and V^T tiles, the raw bias slice and the block-table
  // entries.  No register holds them and the compiler's memory-wait
  // bookkeeping never sees them (it would otherwise wait for them before LDS
  // reads it cannot tell apart, or at loop back edges); they are written as
  // inline assembly and waited for explicitly:
  //   * stage s+1's tiles are issued right after the barrier that closes
  //     phase 2s-1 (their buffers held tiles s-1 and s-2, which nobody reads
  //     any more) and waited for at the end of phase 2s+1, before the barrier
  //     that publishes them: two phases to land;
  //   * the bias slice and the block-table entries of a stage travel one
  //     stage earlier still, so that they are published by a barrier before
  //     other waves read them (the band conversion reads entries fetched by
  //     other waves; the tile loads of a stage need its page numbers).
  // Each lane fetches whichever (row, chunk) the padded tile layout keeps at
  // its slot; padding slots receive a harmless copy.  Keys >= seq_len exist
  // only in the sequence's last tile and hold no data (possibly NaN); once a
  // wave's loads have landed it zeroes those K rows and V^T columns in its
  // own slots, so 0 * garbage cannot reach O and masked logits stay -inf
  // rather than NaN.
  constexpr int kSlotBytes = 16;
  constexpr int kKRowSlots = kKStride * (int)sizeof(T) / kSlotBytes;    // incl. padding
  constexpr int kKDataSlots = kHeadDim * (int)sizeof(T) / kSlotBytes;
  constexpr int kKLoads = kBK * kKRowSlots / 64;                        // wave loads per K tile
  constexpr int kVRowSlots = kVStride * (int)sizeof(T) / kSlotBytes;
  constexpr int kVDataSlots = kBK * (int)sizeof(T) / kSlotBytes;
  constexpr int kVLoads = kHeadDim * kVRowSlots / 64;
  // Tile loads are issued by waves 4-7 only (at the start of their softmax
  // phase); waves 0-3 go straight from the barrier into their matrix phase.
  constexpr int kLoaders = kWaves / 2;
  const int lw = wave - kLoaders;                                       // loader index (>= 0 for waves 4-7)
  constexpr int kKPer = (kKLoads + kLoaders - 1) / kLoaders;
  constexpr int kVPer = (kVLoads + kLoaders - 1) / kLoaders;
  constexpr int kEpd = 4 / (int)sizeof(T);                              // bias elements per dword
  constexpr int kBandLoads = band_raw_dwords<T>() / 64;
  static_assert(kBK * kKRowSlots % 64 == 0 && kHeadDim * kVRowSlots % 64 == 0,
                "tile buffers are whole wave loads");
  constexpr int kBandPer = (kBandLoads + kLoaders - 1) / kLoaders;
  constexpr uint32_t kPageBytes = kPage * kHeadDim * sizeof(T);

  const uint32_t bias_bytes = (uint32_t)A.Hq * (uint32_t)A.R * sizeof(T);
  const u32x4 bias_rsrc = make_buf_rsrc(A.bias, bias_bytes);
  const u32x4 btab_rsrc = make_buf_rsrc(btab, (uint32_t)A.max_blocks * 4u);
  auto page_rsrc = [&](const T* cache, int phys) {
    return make_buf_rsrc(cache + ((size_t)phys * A.Hkv + kvg) * (size_t)(kPage * kHeadDim),
                         kPageBytes);
  };
  auto lds_addr = [](const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
  };
  // First element (absolute, dword-aligned) of the bias slice of stage x.
  auto band_e0 = [&](int x) {
    const int d_lo = P0 - (jt_lo + x) * kBK - kBK + 1;          // smallest distance of the band
    const int e0 = h * A.R + d_lo;
    return e0 - (((e0 % kEpd) + kEpd) % kEpd);
  };
  // Slice of stage x and the block-table entries of stage x (one stage ahead).
  auto dma_ahead = [&](int x) {
    if (lw < 0) return;                           // only waves 4-7 load
    const int ln = lane;
    if (x < n_t) {
#pragma unroll
      for (int j = 0; j < kBandPer; ++j) {
        const int n = lw + kLoaders * j;
        if (n < kBandLoads) {
          const uint32_t voff = (uint32_t)(band_e0(x) * (int)sizeof(T)) + 4u * (64 * n + ln);
          lds_dma4(bias_rsrc, lds_addr(&sm.braw[x & 1][64 * n]), voff, 0u);
        }
      }
    }
    if (x <= n_t && wave == kWaves - 1 && ln < 2) {
      const int jt = min(max(jt_lo + x - ln, jt_lo), jt_hi);    // lane 0: K tile x, lane 1: V tile x-1
      lds_dma4(btab_rsrc, lds_addr(&sm.pages[x & 1][0]), (uint32_t)(jt * kBK / kPage) * 4u, 0u);
    }
  };
  // Which 1 KiB blocks of a tile loader lw fetches.  bf16: a run of four
  // consecutive blocks 4 lw .. 4 lw + 3 under one M0 value, and block
  // 16 + lw when the tile has it (K 17 blocks, V^T 18); fp32: blocks
  // lw, lw + 4, lw + 8, ...
  constexpr bool kRuns = sizeof(T) == 2;
  static_assert(!kRuns || (kKLoads >= 16 && kKLoads <= 20 && kVLoads >= 16 && kVLoads <= 20 &&
                           kKPer == 5 && kVPer == 5),
                "run layout of the bf16 tiles");
  auto my_block = [&](int j) { return kRuns ? (j < 4 ? 4 * lw + j : 16 + lw) : lw + kLoaders * j; };
  auto page_rsrc_early = [&](const T* cache, int phys) {          // starts 4 KiB before the page
    return make_buf_rsrc(reinterpret_cast<const char*>(
                             cache + ((size_t)phys * A.Hkv + kvg) * (size_t)(kPage * kHeadDim)) - 4096,
                         kPageBytes + 4096u);
  };
  // Tile loads of stage x, on page numbers published earlier.
  auto dma_tiles = [&](int x, int k_phys, int v_phys) {
    if (lw < 0) return;                           // only waves 4-7 load
    const int ln = lane;                          // (per-lane offsets are loop-invariant)
    if constexpr (kRuns) {
      auto koff = [&](int n) {
        const int slot = 64 * n + ln;
        const int row = slot / kKRowSlots, ch = min(slot % kKRowSlots, kKDataSlots - 1);
        return (uint32_t)(row * kHeadDim * (int)sizeof(T) + ch * kSlotBytes);
      };
      auto voff = [&](int n) {
        const int slot = 64 * n + ln;
        const int row = slot / kVRowSlots, ch = min(slot % kVRowSlots, kVDataSlots - 1);
        return (uint32_t)(row * kPage * (int)sizeof(T) + ch * kSlotBytes);
      };
      const int n0 = 4 * lw;
      if (x < n_t) {                                 // K of tile x: one run + block 16 + lw
        const int jt = jt_lo + x;
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kBK % kPage) * kHeadDim * sizeof(T));
        const uint32_t lds = lds_addr(&sm.k[x & 1][0]);
        lds_dma16x4(page_rsrc_early(kc, k_phys), lds + 1024u * n0, koff(n0) + 4096u,
                    koff(n0 + 1) + 3072u, koff(n0 + 2) + 2048u, koff(n0 + 3) + 1024u, soff);
        if (16 + lw < kKLoads) lds_dma16(page_rsrc(kc, k_phys), lds + 1024u * (16 + lw), koff(16 + lw), soff);
      }
      if (x >= 1) {                                  // V of tile x-1: the same
        const int jt = jt_lo + x - 1;
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kBK % kPage) * sizeof(T));
        const uint32_t lds = lds_addr(&sm.vt[(x - 1) & 1][0]);
        lds_dma16x4(page_rsrc_early(vc, v_phys), lds + 1024u * n0, voff(n0) + 4096u,
                    voff(n0 + 1) + 3072u, voff(n0 + 2) + 2048u, voff(n0 + 3) + 1024u, soff);
        if (16 + lw < kVLoads) lds_dma16(page_rsrc(vc, v_phys), lds + 1024u * (16 + lw), voff(16 + lw), soff);
      }
      return;
    }
    if (x < n_t) {                                   // K of tile x
      const int jt = jt_lo + x;
      const u32x4 r = page_rsrc(kc, k_phys);
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kBK % kPage) * kHeadDim * sizeof(T));
      const uint32_t lds = lds_addr(&sm.k[x & 1][0]);
#pragma unroll
      for (int j = 0; j < kKPer; ++j) {
        const int n = lw + kLoaders * j;
        if (n < kKLoads) {
          const int slot = 64 * n + ln;
          const int row = slot / kKRowSlots, ch = min(slot % kKRowSlots, kKDataSlots - 1);
          lds_dma16(r, lds + 1024u * n, (uint32_t)(row * kHeadDim * (int)sizeof(T) + ch * kSlotBytes), soff);
        }
      }
    }
    if (x >= 1) {                                    // V of tile x-1
      const int jt = jt_lo + x - 1;
      const u32x4 r = page_rsrc(vc, v_phys);
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(jt * kBK % kPage) * sizeof(T));
      const uint32_t lds = lds_addr(&sm.vt[(x - 1) & 1][0]);
#pragma unroll
      for (int j = 0; j < kVPer; ++j) {
        const int n = lw + kLoaders * j;
        if (n < kVLoads) {
          const int slot = 64 * n + ln;
          const int row = slot / kVRowSlots, ch = min(slot % kVRowSlots, kVDataSlots - 1);
          lds_dma16(r, lds + 1024u * n, (uint32_t)(row * kPage * (int)sizeof(T) + ch * kSlotBytes), soff);
        }
      }
    }
  };
  auto stage_pages = [&](int x, int& k_phys, int& v_phys) {   // published by a barrier
    k_phys = __builtin_amdgcn_readfirstlane(sm.pages[x & 1][0]);
    v_phys = __builtin_amdgcn_readfirstlane(sm.pages[x & 1][1]);
  };
  auto fix_tail = [&](int x) {                       // after this wave's loads landed
    if (lw < 0 || n_tail >= kBK) return;             // the slots of waves 4-7 only
    // An opaque copy of the lane index keeps this once-per-work-group
    // arithmetic here instead of being hoisted out of the phase loop (where
    // its results would hold registers for the whole loop).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (x < n_t && jt_lo + x == jt_hi) {
      char* buf = reinterpret_cast<char*>(&sm.k[x & 1][0]);
#pragma unroll
      for (int j = 0; j < kKPer; ++j) {
        const int n = my_block(j);
        const int slot = 64 * n + ln;
        if (n < kKLoads && slot / kKRowSlots >= n_tail)
          *reinterpret_cast<u32x4*>(buf + kSlotBytes * slot) = u32x4{0, 0, 0, 0};
      }
    }
    if (x >= 1 && jt_lo + x - 1 == jt_hi) {
      char* buf = reinterpret_cast<char*>(&sm.vt[(x - 1) & 1][0]);
      constexpr int kPer = kSlotBytes / (int)sizeof(T);          // keys per 16-byte slot
#pragma unroll
      for (int j = 0; j < kVPer; ++j) {
        const int n = my_block(j);
        const int slot = 64 * n + ln;
        const int ch = slot % kVRowSlots;
        if (n < kVLoads && ch < kVDataSlots && kPer * (ch + 1) > n_tail) {
          u32x4* q16 = reinterpret_cast<u32x4*>(buf + kSlotBytes * slot);
          *q16 = keep_first_elems<T>(*q16, n_tail - kPer * ch);
        }
      }
    }
  };
  // Bias band of stage x from its raw slice (published by an earlier
  // barrier): pre-multiplied by sqrt(128), -inf outside the causal window,
  // distances >= R take bias[R-1].  Four copies shifted by one entry.
  float bias_last;                                  // loaded in the prologue
  // Written by waves 0-3 (256 threads), at the end of their softmax phase.
  auto band_store = [&](int x) {
    if (x >= n_t) return;
    const T* raw = reinterpret_cast<const T*>(&sm.braw[x & 1][0]);
    const int e0 = band_e0(x);
#pragma unroll
    for (int k = 0; k < (kBand + kThreads / 2 - 1) / (kThreads / 2); ++k) {
      const int v = tid + (kThreads / 2) * k;
      if (v < kBand) {
        const int dist = P0 - (jt_lo + x) * kBK + (kBQ - 1) - v;
        const bool vis = dist >= 0 && (A.window == 0 || dist < A.window);
        const float bv = dist > A.R - 1 ? bias_last : to_f32(raw[h * A.R + dist - e0]);
        const float band_v = vis ? bv * band_mul : -INFINITY;
#pragma unroll
        for (int sh = 0; sh < 4; ++sh)
          if (v - sh >= 0) sm.band[x & 1][sh][v - sh] = band_v;
      }
    }
  };

  // ---- running softmax state (per lane: one query row, half of the keys)
  float m_used = -INFINITY;
  float l_sum = 0.0f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  f32x16 acc[2];           // S^T of the tile between its matrix and softmax phases
  bool rescale = false;    // the last softmax phase moved the running max ...
  float alpha = 1.0f;      // ... and O must be scaled by alpha before its P V
  Frag8<T> pf[4];          // P^T of the tile between its softmax and the next matrix phase

  const int kp = keyperm(lq);
  const int band_shift = (3 - (lane & 3)) & 3;

  // Matrix phase of tile i: S^T_i = K_i Q^T (accumulators start as the
  // sheared bias band) and O^T += V^T_{i-1} P^T_{i-1}, interleaved two + two
  // MFMAs per k-step.  In the first phase P^T is zero and V buffer 1 has
  // been zeroed, so O gains exactly +0.
  // LDS fragment reads run ahead of the MFMAs that consume them (K two
  // k-steps ahead, V one) and sched_barrier keeps the compiler from sinking
  // them back next to their uses.
  // kQK false: the closing phase (i = n_t), PV of the last tile only (there
  // is no tile n_t whose S^T would be computed).
  auto matrix_phase = [&](int i, auto qk_tag) {
    constexpr bool kQK = decltype(qk_tag)::value, kPV = true;
    const int kb = i & 1, vb = (i - 1) & 1;
    auto kfrag = [&](int ks, int t) {
      return Frag8<T>::load(&sm.k[kb][(32 * t + kp) * kKStride + 8 * (2 * ks + lg)]);
    };
    auto vfrag = [&](int step, int j) {          // k-step `step` uses slab step/2, dims tile 2(step%2)+j
      const int dr = 32 * (2 * (step & 1) + j) + lq;
      return Frag8<T>::load(&sm.vt[vb][dr * kVStride + 8 * (2 * (step >> 1) + lg)]);
    };
    Frag8<T> kq[3][2], vq[2][2];
    if constexpr (kQK) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 2; ++t) kq[j][t] = kfrag(j, t);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int v0 = (kBQ - 1) - a_row + 32 * t + 16 * hh + 8 * lg;
          const float* bp = &sm.band[kb][band_shift][v0 - band_shift];
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(bp);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(bp + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[t][8 * hh + e] = x0[e];
            acc[t][8 * hh + 4 + e] = x1[e];
          }
        }
    }
    if constexpr (kPV) {
#pragma unroll
      for (int j = 0; j < 2; ++j) vq[0][j] = vfrag(0, j);
      if (rescale) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) asm("v_mul_f32 %0, %1, %0" : "+v"(o[dt][r]) : "v"(alpha));
        rescale = false;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (kQK) {
        if (ks + 2 < 8) {
#pragma unroll
          for (int t = 0; t < 2; ++t) kq[(ks + 2) % 3][t] = kfrag(ks + 2, t);
        }
      }
      if constexpr (kPV) {
        if (ks + 1 < 8) {
#pragma unroll
          for (int j = 0; j < 2; ++j) vq[(ks + 1) & 1][j] = vfrag(ks + 1, j);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kQK) {
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[t] = mfma32(kq[ks % 3][t], qf[ks], acc[t]);
      }
      if constexpr (kPV) {
        const int d0 = 2 * (ks & 1);
#pragma unroll
        for (int j = 0; j < 2; ++j) o[d0 + j] = mfma32(vq[ks & 1][j], pf[ks >> 1], o[d0 + j]);
      }
    }
  };

  // Softmax phase of a tile: online softmax in base 2 with a lazy rescale.
  auto softmax_phase = [&]() {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[t][r]);
    mx = pair_max(mx);
    const float m_tile = mx * c;
    const bool need = m_tile > m_used + kRescaleSlack;
    rescale = __any(need);
    if (rescale) {
      // Lanes that do not need it keep their max (alpha = 1); this also keeps
      // rows that have seen no key yet (m_used = -inf) free of -inf - -inf.
      // O itself is rescaled by the next matrix phase, before it adds this
      // tile's P V: the matrix-phase wave has idle vector-ALU cycles, and O
      // stays out of this phase (touching it here made the compiler copy all
      // 64 O registers on every pass).
      alpha = need ? fast_exp2(m_used - m_tile) : 1.0f;   // -inf -> 0
      l_sum *= alpha;
      m_used = need ? m_tile : m_used;
    }
    const float msub = m_used == -INFINITY ? 0.0f : m_used;
    // The row sum adds the fp32 probabilities on the vector ALU, in four
    // independent chains.  (v_dot2_f32_bf16 over the packed values would
    // take one instruction per pair, but it does not co-issue with the
    // other wave's MFMAs: each one waits for the matrix core, which
    // doubled this phase when it ran beside a matrix phase.)
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(acc[t][8 * hh + e] * c - msub);
        pf[2 * t + hh] = Frag8<T>::pack(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) ls[e & 3] += p[e];
      }
    l_sum += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // V buffer 1 is read (times P^T = 0) by the first matrix phase before any
  // V tile is loaded: zero it so that 0 * garbage cannot produce NaN.
  {
    u32x4* vz = reinterpret_cast<u32x4*>(&sm.vt[1][0]);
    constexpr int kVBufSlots = kHeadDim * kVStride * (int)sizeof(T) / 16;
    for (int i = tid; i < kVBufSlots; i += kThreads) vz[i] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) pf[j] = Frag8<T>::zero();

  // Prologue: stage 0 (its page from the block table directly), the slices
  // and page numbers of stages 0 and 1; then stage 1's tiles and the slice
  // and page numbers of stage 2.
  // The plain loads (the first page number, bias[R-1], the Q fragments) are
  // issued first and the first stage's DMA right behind them, so their
  // latencies overlap; all of them are consumed after the wait below, so the
  // compiler's own memory-wait bookkeeping sees them finished before the
  // phase loop and never waits there (such a wait would also stall on the
  // in-flight tile loads, which the bookkeeping cannot see).
  {
    int k0 = 0;
    if (half == 1) k0 = __builtin_amdgcn_readfirstlane(btab[jt_lo * kBK / kPage]);
    bias_last = to_f32(bias_h[A.R - 1]);
    const T* qrow = qp + ((size_t)(tok0 + row0 + a_row) * A.Hq + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = row_ok ? Frag8<T>::load(qrow + 16 * ks) : Frag8<T>::zero();
    if (half == 1) {
      keep_live(k0);
      dma_ahead(0);
      dma_ahead(1);
      dma_tiles(0, k0, 0);
    }
  }
  wait_all_loads();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) keep_live(qf[ks]);
  keep_live(bias_last);
  __syncthreads();                                 // slices 0-1, pages of stage 1
  if (half == 1) fix_tail(0); else band_store(0);
  __syncthreads();                                 // stage 0 published
  if (half == 1) {
    int kp1, vp1;
    stage_pages(1, kp1, vp1);
    dma_ahead(2);
    dma_tiles(1, kp1, vp1);
  }

  // ---- phase loop.  Waves 4-7 run one phase behind waves 0-3, and a barrier
  // closes every phase, so the two waves sharing a SIMD are always in
  // opposite phases: one issues MFMAs while the other runs the softmax on the
  // vector ALU, and the two overlap.  A wave's own sequence is
  //   M(0) S(0) M(1) S(1) ... M(n-1) S(n-1) M(n)
  // (M = matrix phase, S = softmax phase, M(n) = PV of the last tile only);
  // waves 0-3 run step p in phase p, waves 4-7 step p-1.  K_i and band_i live
  // in LDS buffer i%2 through phases 2i and 2i+1, V_i in buffer i%2 through
  // phases 2i+2 and 2i+3.  The barrier closing phase 2i+1 also publishes
  // stage i+1 and, right after it, issues stage i+2 into the buffers of
  // tiles i and i-1, which nobody reads any more.  The loop follows a wave's
  // own steps, so the matrix and softmax code each appear once in it, in
  // order (O flows straight from one to the next).  Waves 0-3 reach that
  // barrier from their softmax phase and write the band before it; waves
  // 4-7 reach it from their matrix phase, wait for and fix up their own tile
  // loads before it and issue the next ones after it, before their softmax
  // phase.  So the waves that must start MFMAs after the barrier do no
  // staging work at all.
  if (half == 1) __syncthreads();                  // waves 4-7 sit out phase 0
  for (int i = 0;; ++i) {
    if (i == n_t) {
      matrix_phase(i, std::false_type{});
      break;
    }
    matrix_phase(i, std::true_type{});
    if (half == 0) {
      __syncthreads();                             // closes phase 2i
      softmax_phase();
      band_store(i + 1);
      __syncthreads();                             // closes phase 2i+1
    } else {
      wait_all_loads();
      fix_tail(i + 1);
      __syncthreads();                             // closes phase 2i+1
      if (i + 1 < n_t) {
        int kp, vp;
        stage_pages(i + 2, kp, vp);
        dma_ahead(i + 3);
        dma_tiles(i + 2, kp, vp);
      }
      softmax_phase();
      __syncthreads();                             // closes phase 2i+2
    }
  }
  if (half == 0) __syncthreads();                  // closes phase 2n (M(n) of waves 0-3)

  // ---- epilogue: O^T register r of tile dt is dim 32dt + 8(r/4) + 4lg + r%4
  const float lt = pair_sum(l_sum);
  if (!row_ok) return;
  const float inv = kScaled ? A.v_scale / lt : 1.0f / lt;
  T* op = static_cast<T*>(A.out) + ((size_t)(tok0 + row0 + a_row) * A.Hq + h) * kHeadDim;
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

hipError_t launch_prefill(const AttnShape& s, int num_seqs, int max_q_len, const void* q,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                          const void* bias, void* out, float* lse, hipStream_t stream,
                          float k_scale, float v_scale) {
  PrefillArgs a;
  a.k_scale = k_scale; a.v_scale = v_scale;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
  a.cu_q = cu_seqlens_q; a.seq_lens = seq_lens; a.bias = bias; a.out = out; a.lse = lse;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.Hq / s.Hkv; a.window = s.window; a.R = s.bias_len;
  a.max_blocks = max_blocks_per_seq; a.num_seqs = num_seqs;
  const int nqt = (max_q_len + kBQ - 1) / kBQ;
  a.total_groups = nqt * num_seqs * s.Hkv;
  const long padded = ((long)a.total_groups + kXcds - 1) / kXcds * kXcds;
  const long blocks = padded * a.G;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const bool scaled = k_scale != 1.0f || v_scale != 1.0f;
  if (s.dtype == kDtypeBf16 && scaled)
    hipLaunchKernelGGL((prefill_kernel<bf16, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else if (s.dtype == kDtypeBf16)
    hipLaunchKernelGGL((prefill_kernel<bf16, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<float, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace inkattn
