// Multi-query split-K paged decode: several query tokens per sequence (the
// verification of multi-token-prediction drafts), K/V staged through LDS.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Model Architecture /
// Attention (GQA, head size 128, sliding-window and full layers, a learned
// relative-position term added to the logits), Model Architecture / MTP and
// Performance (draft tokens verified in one step), and vLLM Integration &
// Optimization / FA4 with sheared bias (the key range cut into splits).
// Logit of query head h at position p against key j:
//   q.k_j / sqrt(128) + bias[h][min(p - j, R - 1)].
//
// With n query tokens a kv-head group has n * Hq/Hkv (token, head) columns,
// e.g. 72 for 9 tokens and 8 heads.  A kernel that keeps every column in
// each wave's registers must read the K/V range once per few columns; here
// one work-group of 8 waves per (split, kv-head, sequence) reads each K/V
// byte of its range once:
// * Units of 64 keys (half a page) go HBM -> registers -> LDS, every thread
//   moving 16-byte chunks (coalesced: a wave load covers 1 KiB of a K page or
//   eight 128-byte runs of its V^T rows).  Three units are in flight while a
//   fourth is computed; one barrier per unit.  An E4M3 cache is converted to
//   bf16 on its way into LDS, so both caches share the compute below.
// * Wave t owns column tile t (columns 16t .. 16t+15, token = column / G,
//   head = column % G) and runs, per unit, S^T = K Q^T and O^T += V^T P^T on
//   v_mfma_f32_16x16x32_bf16 with its fragments read from LDS, and the online
//   softmax of its columns over the unit's two 32-key items.  Waves left over
//   (8 - tiles) become partners of tiles 0, 1, ...: the owner then takes the
//   first item of every unit and the partner the second, and the partner
//   hands its (max, sum, O) to the owner through LDS at the end.  With 5
//   tiles (9 tokens x 8 heads) the busiest SIMD runs 3 items per unit
//   instead of 4.
// * Sheared bias: the distances of a unit form, per head, a band of 63 + n
//   entries; the band of every head of the group is staged with the unit
//   (clamped at R - 1, pre-multiplied by log2 e) and read from LDS.  Head e's
//   band starts 81 floats after head e-1's.  A probe of 4-byte reads times
//   this pattern (8 heads, 2 tokens per column tile) at two passes per
//   half-wave, an even stride (80) at four; no head stride, and no second
//   copy read by the odd lane groups, measured better than two.
// * K rows are stored in LDS with bits 2 and 4 of the key index swapped, so
//   the 16 keys a fragment reads are 16 consecutive rows.  ds_read_b128 serves
//   32 lanes a pass over 128 banks and is conflict-free when the 32 lanes hit
//   32 distinct 16-byte slots mod 32 (measured with a probe of read patterns):
//   K rows of 18 slots (72 dwords) and V^T rows of 10 (40 dwords) put the 16
//   rows of a half-wave on 16 distinct even slots and its two lane groups on
//   the even and the odd ones.  (Rows of 17 and 9 slots, which suit a model
//   of 16 lanes over 64 banks, conflict in half of the passes.)
// Keys past the sequence end exist only in its last page and may hold any
// bits: their V^T columns are zeroed on the way into LDS and their logits are
// masked, so 0 * NaN never reaches O.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace inkattn {

namespace {

constexpr int kMqWaves = 8;
constexpr int kMqThreads = 64 * kMqWaves;
constexpr int kUnit = 64;                   // keys per staged unit (half a page)
constexpr int kKRow = kHeadDim + 16;        // LDS K row, elements (72 dwords, 18 slots)
constexpr int kVRow = kUnit + 16;           // LDS V^T row, elements (40 dwords, 10 slots)
constexpr int kMaxG = 16;                   // q-heads per kv-head
constexpr int kBandW = 81;                  // >= 63 + 16 distances per head and unit; odd
constexpr int kBandSlots = kMaxG * kBandW;  // staged bias entries per unit
constexpr int kBandPer = (kBandSlots + kMqThreads - 1) / kMqThreads;
constexpr int kSets = 3;                    // units staged in registers / LDS buffers
constexpr float kSlack = 8.0f;              // lazy-rescale threshold, log2 units

struct MqSmem {
  bf16 k[kSets][kUnit * kKRow];             // [key (permuted)][d]
  bf16 vt[kSets][kHeadDim * kVRow];         // [d][key]
  float band[kSets][kBandSlots];            // [head in group][distance - d_min]
};

// LDS row, within its 32-key item, of key k (0 .. 31): bits 2 and 4 swapped.
__device__ __forceinline__ int krow(int k) {
  return (k & 0x0b) | ((k & 0x04) << 2) | ((k & 0x10) >> 2);
}

// Max over the lane pair (l, l ^ 16) with v_permlane16_swap (a VALU op, no
// LDS round trip): after the swap the two result registers hold lane l's
// value and its partner's.
__device__ __forceinline__ float row_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A unit's raw chunks in flight: 16-byte chunks of K and of V^T per thread
// (two each for bf16, one each for E4M3), and the thread's bias entries.
template <typename TKV> struct MqStage {
  static constexpr int kChunks = (int)sizeof(TKV);
  u32x4 k[kChunks], v[kChunks];
  bf16 bias[kBandPer];
};

// Barrier that publishes this wave's LDS writes but leaves its global loads
// in flight (a fenced barrier would wait for those as well).  One asm
// statement with a memory clobber, so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Empty asms that consume a value: whatever computes it runs
// unconditionally, and has completed, at this point.
__device__ __forceinline__ void keep_live_f(float x) { asm volatile("" :: "v"(x)); }
__device__ __forceinline__ void keep_live_frag(const Frag8<bf16>& f) { asm volatile("" :: "v"(f.v)); }

// Sixteen E4M3 codes -> two bf16 fragments (elements 0-7 and 8-15), exactly.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& w, Frag8<bf16>& lo, Frag8<bf16>& hi) {
  lo = fp8x8_to_bf16(w[0], w[1]);
  hi = fp8x8_to_bf16(w[2], w[3]);
}

template <typename TKV>
__global__ __launch_bounds__(kMqThreads) void decode_mq_kernel(
    int Hq, int Hkv, int window, int R, int S, int B, const bf16* __restrict__ q,
    const TKV* __restrict__ k_cache, const TKV* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const bf16* __restrict__ bias,
    float* __restrict__ part_o, float* __restrict__ part_lse, bf16* __restrict__ out,
    float* __restrict__ lse, float k_scale, float v_scale) {
  constexpr bool kFp8 = std::is_same<TKV, fp8e4>::value;
  constexpr int kSz = (int)sizeof(TKV);
  constexpr int kKChunksPerRow = kHeadDim * kSz / 16;   // 16-byte chunks per K row
  constexpr int kVChunksPerRow = kUnit * kSz / 16;      // ... per V^T row of a unit
  static_assert(kKChunksPerRow == (kFp8 ? 8 : 16) && kVChunksPerRow == (kFp8 ? 4 : 8),
                "chunk maps of k_chunk / v_chunk");
  constexpr int kEpc = 16 / kSz;                        // elements per chunk
  constexpr uint32_t kPageBytes = kPage * kHeadDim * kSz;
  __shared__ MqSmem sm;

  const int id = blockIdx.x;
  if (id >= S * Hkv * B) return;
  const int split = id % S;
  const int kvh = (id / S) % Hkv;
  const int b = id / (S * Hkv);
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int tok0 = cu_q[b];
  const int q_len = cu_q[b + 1] - tok0;
  const int n_cols = G * q_len;
  const int L = seq_lens[b];
  const int pos0 = L - q_len;                    // position of the first query token
  const int kstart = window > 0 ? max(0, pos0 - window + 1) : 0;
  const int blk_first = kstart >> 7;
  const int blk_last = (L - 1) >> 7;
  const int nblk = blk_last - blk_first + 1;
  const int bps = (nblk + S - 1) / S;
  const int my_lo = blk_first + split * bps;
  const int my_hi = min(my_lo + bps, blk_last + 1);
  const int n_units = 2 * max(my_hi - my_lo, 0);

  // This wave's role (wave-uniform): its column tile and which items of
  // every unit it computes (bit ii: item ii).
  const int n_ct = (n_cols + 15) / 16;           // <= 8 (checked by the host)
  const int n_pair = max(0, min(kMqWaves - n_ct, n_ct));
  const bool partner = wave >= n_ct;
  const int tile = partner ? wave - n_ct : wave;
  const bool active = wave < n_ct + n_pair;
  const int item_mask = tile >= n_pair ? 3 : (partner ? 2 : 1);
  const int gc = 16 * tile + col;
  const bool head_ok = gc < n_cols;
  const int token = head_ok ? gc / G : 0;
  const int hl = head_ok ? gc % G : 0;           // head within the group
  const int h = kvh * G + hl;
  const int pos = pos0 + token;
  const int k_lo = window > 0 ? max(0, pos - window + 1) : 0;
  // Keys that every valid column of this wave sees: units inside
  // [w_lo, w_hi] skip the per-key window mask (columns past n_cols then
  // compute finite values nobody stores).
  int w_lo = head_ok ? k_lo : 0, w_hi = head_ok ? pos : 0x7fffffff;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    w_lo = max(w_lo, __shfl_xor(w_lo, off, 64));
    w_hi = min(w_hi, __shfl_xor(w_hi, off, 64));
  }
  w_lo = __builtin_amdgcn_readfirstlane(w_lo);
  w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  const float c = 0.08838834764831845f * kLog2e * k_scale;   // log2(e) / sqrt(128)

  // Q^T fragments (B operand): k-step ds of lane group grp holds dims
  // 32ds + 8grp .. +7.
  Frag8<bf16> qf[4];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds)
    qf[ds] = head_ok ? Frag8<bf16>::load(q + ((size_t)(tok0 + token) * Hq + h) * kHeadDim +
                                         32 * ds + 8 * grp)
                     : Frag8<bf16>::zero();
  // (waited for here, once: a wait inside the unit loop would also drain the
  // K/V loads in flight)
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) keep_live_frag(qf[ds]);

  // ---- staging.  Unit u is page my_hi-1 - u/2, keys 64(u%2) .. +63 of it.
  // Every load is unconditional (a unit index past the end re-reads the last
  // unit) so that each wait the compiler places covers exactly the loads it
  // needs and the next units stay in flight.
  const rsrc_t bias_r = make_rsrc(bias, (uint32_t)((size_t)Hq * R * sizeof(bf16)));
  // Pages are taken newest first (the page the step's sconv has just written
  // is fetched early, while the rest of the range still streams).
  auto unit_key0 = [&](int u) { return (my_hi - 1 - (u >> 1)) * kPage + kUnit * (u & 1); };
  // Chunk i of this thread: its K row in LDS (and the key it holds) and
  // 16-byte column, its V^T row and key chunk.  The chunks of a half-wave
  // are chosen so that its LDS writes fall on 32 distinct 16-byte slots mod
  // 32.  bf16: K rows r and r+8 (starts 18r, 18r+144: 16 slots apart), V^T
  // rows d, d+4, d+8, d+12 (8 slots apart).  E4M3 chunks become 32 bytes in
  // LDS, written as two halves: half of the rows write their high half first
  // (odd slots) while the others write their low half (even slots).
  struct KChunk { int row, key, kc; bool hi_first; };
  struct VChunk { int d, vc; bool hi_first; };
  auto k_chunk = [&](int i) {
    const int hw = (tid >> 5) + (kMqThreads / 32) * i;
    const int l = tid & 31;
    KChunk r;
    if constexpr (!kFp8) {
      r.row = 16 * (hw >> 3) + (hw & 7) + 8 * (l >> 4);
      r.kc = l & 15;
      r.hi_first = false;
    } else {
      const int j = l >> 3;
      r.row = 32 * (hw >> 3) + (hw & 7) + 8 * (j >> 1) + 16 * (j & 1);
      r.kc = l & 7;
      r.hi_first = (j & 1) != 0;
    }
    r.key = 32 * (r.row >> 5) + krow(r.row & 31);   // (krow is its own inverse)
    return r;
  };
  auto v_chunk = [&](int i) {
    const int hw = (tid >> 5) + (kMqThreads / 32) * i;
    const int l = tid & 31;
    VChunk r;
    if constexpr (!kFp8) {
      r.d = 16 * (hw >> 2) + (hw & 3) + 4 * (l >> 3);
      r.vc = l & 7;
      r.hi_first = false;
    } else {
      const int j = l >> 2;
      r.d = 16 * (hw >> 1) + 2 * (hw & 1) + (j & 1) + 4 * (j >> 1);
      r.vc = l & 3;
      r.hi_first = (j & 1) != 0;
    }
    return r;
  };
  auto stage_load = [&](int u, MqStage<TKV>& st) {
    u = min(u, n_units - 1);
    const int blk = my_hi - 1 - (u >> 1);
    const int phys = block_table[(size_t)b * max_blocks + blk];
    const size_t base = ((size_t)phys * Hkv + kvh) * (size_t)(kPage * kHeadDim);
    const rsrc_t kr = make_rsrc(k_cache + base, kPageBytes);
    const rsrc_t vr = make_rsrc(v_cache + base, kPageBytes);
    const uint32_t k_soff = (uint32_t)(kUnit * (u & 1) * kHeadDim * kSz);
    const uint32_t v_soff = (uint32_t)(kUnit * (u & 1) * kSz);
#pragma unroll
    for (int i = 0; i < MqStage<TKV>::kChunks; ++i) {
      const KChunk kq = k_chunk(i);
      st.k[i] = buf_load16(kr, (uint32_t)(kq.key * kHeadDim * kSz + 16 * kq.kc), k_soff);
      const VChunk vq = v_chunk(i);
      st.v[i] = buf_load16(vr, (uint32_t)(vq.d * kPage * kSz + 16 * vq.vc), v_soff);
    }
    // Band of head e at offset v: distance d_min + v, d_min = pos0 - key0 - 63.
    const int d_min = pos0 - unit_key0(u) - (kUnit - 1);
#pragma unroll
    for (int i = 0; i < kBandPer; ++i) {
      const int s = min(tid + kMqThreads * i, G * kBandW - 1);
      const int e = s / kBandW, v = s % kBandW;
      const int dist = min(max(d_min + v, 0), R - 1);
      st.bias[i] = buf_load_elem<bf16>(
          bias_r, (uint32_t)(((kvh * G + e) * R + dist) * (int)sizeof(bf16)));
    }
    // Keep a unit's loads together and in this order: the waits placed for
    // a unit then count only the units issued after it (the scheduler would
    // otherwise gather the bias loads of several units behind their K/V).
    __builtin_amdgcn_sched_barrier(0);
  };
  auto stage_store = [&](int u, const MqStage<TKV>& st, int buf) {
    const int key0 = unit_key0(u);
    const bool tail = key0 + kUnit > L;          // (wave-uniform) keys past L in this unit
#pragma unroll
    for (int i = 0; i < MqStage<TKV>::kChunks; ++i) {
      const KChunk kq = k_chunk(i);
      bf16* kd = &sm.k[buf][kq.row * kKRow + kEpc * kq.kc];
      const VChunk vq = v_chunk(i);
      bf16* vd = &sm.vt[buf][vq.d * kVRow + kEpc * vq.vc];
      const int nvalid = L - (key0 + kEpc * vq.vc);  // valid keys of this V^T chunk
      if constexpr (kFp8) {
        Frag8<bf16> lo, hi;
        fp8x16_to_bf16(st.k[i], lo, hi);
        (kq.hi_first ? hi : lo).store(kd + (kq.hi_first ? 8 : 0));
        (kq.hi_first ? lo : hi).store(kd + (kq.hi_first ? 0 : 8));
        fp8x16_to_bf16(st.v[i], lo, hi);
        if (tail) {
          lo = lo.keep_first(nvalid);
          hi = hi.keep_first(nvalid - 8);
        }
        (vq.hi_first ? hi : lo).store(vd + (vq.hi_first ? 8 : 0));
        (vq.hi_first ? lo : hi).store(vd + (vq.hi_first ? 0 : 8));
      } else {
        *reinterpret_cast<u32x4*>(kd) = st.k[i];
        Frag8<bf16> f;
        f.v = st.v[i];
        if (tail) f = f.keep_first(nvalid);
        f.store(vd);
      }
    }
#pragma unroll
    for (int i = 0; i < kBandPer; ++i) {
      const int s = tid + kMqThreads * i;
      if (s < G * kBandW) sm.band[buf][s] = to_f32(st.bias[i]) * kLog2e;
    }
  };

  // ---- per-lane fragment offsets (elements).  S^T tile t of item ii: row r
  // is key 32ii + 8(r/4) + 4t + r%4, so accumulator register r of lane group
  // grp holds key 32ii + 8grp + 4t + r: each lane group ends up with 8
  // consecutive keys, the B-operand layout of P^T.
  int k_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) k_off[t] = krow(8 * (col >> 2) + (col & 3) + 4 * t) * kKRow + 8 * grp;
  const int v_off = col * kVRow + 8 * grp;
  const int band_off = hl * kBandW + token + (kUnit - 1) - 8 * grp;   // offset of key 8grp, ii = 0

  float m = -INFINITY, l = 0.0f;                 // running max (log2 units), this lane's sum
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0, 0, 0, 0};

  // Fragment reads are issued in batches of eight and consumed by an empty
  // asm before their MFMAs, so each batch waits for LDS once rather than
  // once per fragment.  kMask: the items of the unit this wave computes.
  auto compute_items = [&](int u, int buf, auto mask_tag) {
    constexpr int kMask = decltype(mask_tag)::value;
    constexpr int kN = kMask == 3 ? 2 : 1;        // items
    constexpr int kI0 = kMask == 2 ? 1 : 0;       // first item
    const int key0 = unit_key0(u);
    f32x4 sacc[kN][2];
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ii = kI0 + n;
      Frag8<bf16> kf[8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          kf[4 * t + ds] = Frag8<bf16>::load(&sm.k[buf][32 * ii * kKRow + k_off[t] + 32 * ds]);
#pragma unroll
      for (int f = 0; f < 8; ++f) keep_live_frag(kf[f]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[n][t] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) sacc[n][t] = mfma16(kf[4 * t + ds], qf[ds], sacc[n][t]);
      }
    }
    // Band entries are read for every key and consumed by an empty asm: left
    // to itself the compiler reads only the visible ones, each behind a
    // branch of its own.
    float bv[8 * kN];
#pragma unroll
    for (int n = 0; n < kN; ++n)
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[8 * n + e] = sm.band[buf][band_off - 32 * (kI0 + n) - e];
#pragma unroll
    for (int e = 0; e < 8 * kN; ++e) keep_live_f(bv[e]);
    float x[8 * kN];
    float mx = -INFINITY;
    const int j_first = key0 + 32 * kI0;         // this wave's keys: j_first .. j_first + 32kN - 1
    if (j_first >= w_lo && j_first + 32 * kN - 1 <= w_hi) {
#pragma unroll
      for (int e = 0; e < 8 * kN; ++e) {
        x[e] = sacc[e >> 3][(e >> 2) & 1][e & 3] * c + bv[e];
        mx = fmaxf(mx, x[e]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < kN; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j_first + 32 * n + 8 * grp + e;
          const bool ok = head_ok && j >= k_lo && j <= pos;
          x[8 * n + e] = ok ? sacc[n][e >> 2][e & 3] * c + bv[8 * n + e] : -INFINITY;
          mx = fmaxf(mx, x[8 * n + e]);
        }
    }
    mx = row_pair_max(mx);
    mx = pair_max(mx);
    // Lazy rescale: the running max (and O with it) only moves when a
    // column's max exceeds it by more than kSlack, so probabilities stay
    // <= 2^kSlack; lanes that need no move keep alpha = 1 (and a column
    // that has seen no key yet stays at -inf without -inf - -inf).
    const bool need = mx > m + kSlack;
    if (__any(need)) {
      const float alpha = need ? fast_exp2(m - mx) : 1.0f;   // m = -inf -> 0
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      m = need ? mx : m;
    }
    const float m_sub = m == -INFINITY ? 0.0f : m;
    float p[8 * kN];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8 * kN; ++e) {
      p[e] = fast_exp2(x[e] - m_sub);
      psum += p[e];
    }
    l += psum;
    Frag8<bf16> pf[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) pf[n] = Frag8<bf16>::pack(p + 8 * n);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const int ii = kI0 + n;
      Frag8<bf16> vf[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        vf[dt] = Frag8<bf16>::load(&sm.vt[buf][16 * dt * kVRow + v_off + 32 * ii]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) keep_live_frag(vf[dt]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] = mfma16(vf[dt], pf[n], o[dt]);
    }
  };
  auto compute = [&](int u, int buf) {
    if (!active) return;
    if (item_mask == 3) compute_items(u, buf, std::integral_constant<int, 3>{});
    else if (item_mask == 1) compute_items(u, buf, std::integral_constant<int, 1>{});
    else compute_items(u, buf, std::integral_constant<int, 2>{});
  };

  // ---- unit loop: unit v sits in register set v % kSets until it is stored
  // to LDS buffer v % kSets, right after the compute of unit v-1.  Unit v is
  // computed while units v+1 and v+2 (issued two and one iterations earlier)
  // and v+3 (issued just before) are in flight, so a unit's loads have two
  // whole iterations to land.  The loop starts at v = -kSets so that the
  // first units are loaded by the same code, into the same registers, as
  // all later ones (a separate prologue made the compiler drain every load
  // at the loop head); it is unrolled by kSets so that every register set
  // and buffer index is static.
  if (n_units > 0) {
    MqStage<TKV> st[kSets];
    for (int v0 = -kSets;; v0 += kSets) {
      bool last = false;
#pragma unroll
      for (int r = 0; r < kSets; ++r) {
        const int v = v0 + r;                      // v % kSets == r
        stage_load(v + kSets, st[r]);              // set r was stored to LDS last iteration
        if (v >= 0) compute(v, r);
        if (v + 1 >= n_units) {
          last = true;
          break;
        }
        if (v + 1 >= 0) {
          stage_store(v + 1, st[(r + 1) % kSets], (r + 1) % kSets);
          lds_barrier();
        }
      }
      if (last) break;
    }
  }

  // ---- partners hand (max, this lane's sum, O) to their owners: lane l of
  // the owner holds the same (column, dims) as lane l of its partner.  The
  // exchange reuses the K buffers once every wave is done with them.
  if (n_pair > 0) {
    constexpr int kX = 34;                       // floats per lane: m, l, 32 of O
    float* xch = reinterpret_cast<float*>(&sm.k[0][0]);
    static_assert(4 * kX * 64 * 4 <= (int)sizeof(sm.k), "exchange fits the K buffers");
    lds_barrier();
    if (active && partner) {
      float* w = xch + tile * kX * 64 + lane;
      w[0] = m;
      w[64] = l;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) w[64 * (2 + 4 * dt + r)] = o[dt][r];
    }
    lds_barrier();
    if (active && !partner && tile < n_pair) {
      const float* w = xch + tile * kX * 64 + lane;
      const float mp = w[0];
      const float mt = fmaxf(m, mp);
      if (mt != -INFINITY) {
        const float a = fast_exp2(m - mt), bp = fast_exp2(mp - mt);
        l = l * a + w[64] * bp;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[dt][r] = o[dt][r] * a + w[64 * (2 + 4 * dt + r)] * bp;
        m = mt;
      }
    }
  }

  // ---- epilogue: O^T register r of dim tile dt is dim 16dt + 4grp + r.
  if (!active || partner) return;
  float lt = l + wave_shfl_xor(l, 16);
  lt = pair_sum(lt);
  if (!head_ok) return;
  const size_t orow = (size_t)(tok0 + token) * Hq + h;
  const size_t prow = orow * S + split;
  if (m == -INFINITY) {                          // no visible key in this split
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      store4(part_o + prow * kHeadDim + 16 * dt + 4 * grp, 0.0f, 0.0f, 0.0f, 0.0f);
    if (grp == 0) part_lse[prow] = -INFINITY;
    return;
  }
  const float sc = v_scale / lt;
  const float row_lse = (m + fast_log2(lt)) * kLn2;
  if (S == 1) {
    // One split is the whole key range: the result goes straight out.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      store4(out + orow * kHeadDim + 16 * dt + 4 * grp, o[dt][0] * sc, o[dt][1] * sc,
             o[dt][2] * sc, o[dt][3] * sc);
    if (lse != nullptr && grp == 0) lse[orow] = row_lse;
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      store4(part_o + prow * kHeadDim + 16 * dt + 4 * grp, o[dt][0] * sc, o[dt][1] * sc,
             o[dt][2] * sc, o[dt][3] * sc);
    if (grp == 0) part_lse[prow] = row_lse;
  }
}

}  // namespace

void launch_decode_mq_lds(const AttnShape& s, int num_seqs, int num_splits, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          int max_blocks_per_seq, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens, const void* bias, void* out, float* lse,
                          float* part_o, float* part_lse, const float* fp8_scales,
                          hipStream_t stream) {
  const unsigned groups = (unsigned)((long)num_splits * s.Hkv * num_seqs);
  if (fp8_scales != nullptr)
    hipLaunchKernelGGL(decode_mq_kernel<fp8e4>, dim3(groups), dim3(kMqThreads), 0, stream, s.Hq,
                       s.Hkv, s.window, s.bias_len, num_splits, num_seqs, (const bf16*)q,
                       (const fp8e4*)k_cache, (const fp8e4*)v_cache, block_table,
                       max_blocks_per_seq, cu_seqlens_q, seq_lens, (const bf16*)bias, part_o,
                       part_lse, (bf16*)out, lse, fp8_scales[0], fp8_scales[1]);
  else
    hipLaunchKernelGGL(decode_mq_kernel<bf16>, dim3(groups), dim3(kMqThreads), 0, stream, s.Hq,
                       s.Hkv, s.window, s.bias_len, num_splits, num_seqs, (const bf16*)q,
                       (const bf16*)k_cache, (const bf16*)v_cache, block_table,
                       max_blocks_per_seq, cu_seqlens_q, seq_lens, (const bf16*)bias, part_o,
                       part_lse, (bf16*)out, lse, 1.0f, 1.0f);
}

}  // namespace inkattn
