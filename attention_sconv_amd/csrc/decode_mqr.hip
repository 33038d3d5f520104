// Multi-query split-K paged decode with every key's K/V held in the registers
// of one wave: several query tokens per sequence (the verification of
// multi-token-prediction drafts), 17 .. 80 (token, head) columns per kv-head
// group.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Model Architecture /
// Attention (GQA, head size 128, sliding-window and full layers, a learned
// relative-position term added to the logits), Model Architecture / MTP and
// Performance (draft tokens verified in one step), and vLLM Integration &
// Optimization / FA4 with sheared bias (the key range cut into splits).
// Logit of query head h at position p against key j:
//   q.k_j / sqrt(128) + bias[h][min(p - j, R - 1)].
//
// One work-group of four waves per (split, kv-head, sequence): one wave per
// SIMD, each with up to 512 registers.  Every wave computes all columns of
// the group over a quarter of the keys: wave w takes keys 32w .. 32w+31 (an
// "item") of every page of the split's range.  Each K/V byte is therefore
// read once, by one wave, straight from HBM into the registers that feed its
// matrix products, and the waves meet only at the end, where their (max,
// sum, O) are merged through LDS.  (The LDS-staged kernel, which shares each
// unit between 8 waves behind a barrier per unit, serves 81 .. 128 columns.)
// * S^T = K Q^T on v_mfma_f32_16x16x32_bf16.  Lane l loads 16 bytes of dims
//   of key row l%16 (A operand).  The two 16-row tiles t of an item hold keys
//   8(r/4) + 4t + r%4 in row r, so accumulator register r of lane group g
//   holds key 8g + 4t + r: each lane group ends up with 8 consecutive keys,
//   the B-operand layout of P^T.
// * O^T += V^T P^T: lane l loads 8 keys of the V^T row of dim l%16 (the cache
//   holds V transposed within each page).
// * Q^T fragments (B operand) are staged in LDS once, in fragment order, and
//   read per item: held in registers they would crowd out the loads in
//   flight.
// * Register sets: one item in flight while one is computed (bf16; two over
//   an E4M3 cache, half the bytes).  Items past the range, or wholly outside
//   every column's window, load through a zero-length buffer descriptor: the
//   load returns zeros and moves no bytes.
// * Sheared bias and mask: per item each wave stages into its own LDS band
//   the 31 + q_len distances that each head of the group sees there, clamped
//   at R - 1 and pre-multiplied by log2 e, or -inf where the distance is
//   negative (a key after the token) or reaches the window: the causal and
//   window mask is a function of the distance alone, so it costs the softmax
//   nothing.  Head e's band starts at 66e, plus 8 when bit 2 of e is set, so
//   the 32 lanes of a half-wave that read one key for 8 heads x 2 tokens fall
//   on 32 distinct banks.
// * One wave issues its matrix products and its vector instructions one
//   after the other (measured: a pipeline step of 16 products and ~75 vector
//   instructions takes the sum of the two), so this kernel's time is the sum
//   of its products, softmax and load issue; it wins over the LDS-staged one
//   by dropping the staging, the barriers and the per-16-column re-reads of
//   each K/V byte, most of all over an E4M3 cache.
// * Softmax per column tile against a fixed reference: the column's max in
//   the first item where it sees a key.  Probabilities may exceed 1 (up to
//   2^32; the bf16 P and fp32 sums keep their relative precision), and a
//   column whose logits pass the reference by more makes the wave run its
//   range again from the exact column max.  O is thus never rescaled inside
//   the loop and stays in the accumulator registers.
// Keys past the sequence end exist only in its last page and may hold any
// bits: their K rows and V^T elements are zeroed before the products, so
// their logits are exactly -inf and 0 * NaN never reaches O.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace inkattn {

namespace {

constexpr int kRWaves = 4;
constexpr int kRThreads = 64 * kRWaves;
constexpr int kItem = 32;                               // keys per item: a quarter page
constexpr int kHeadBand = 66;                           // band floats per head (2 mod 32)
constexpr int kBandSlots = kRegMqBandEntries / 64;      // staged entries per lane and item
constexpr int kBandFloats = (kMaxRegMqG - 1) * kHeadBand + 8 + kItem + kMaxMqTokens;
constexpr float kBail = 32.0f;                          // largest logit over the reference, log2 units

__device__ __forceinline__ int band_base(int e) { return kHeadBand * e + ((e & 4) ? 8 : 0); }

template <int NCT> struct MqrSmem {
  u32x4 q[NCT * 4 * 64];                                // Q^T fragments [ct][ds][lane]
  float band[kRWaves][(kBandFloats + 4) & ~3];          // each wave's bias band (+ a spare)
  f32x4 xch[kRWaves][kRWaves - 1][NCT][64];             // epilogue: O^T [owner][source][ct][lane]
  float ml[kRWaves][NCT * 16][2];                       // epilogue: (max, sum) per column
};

// One item's loads: K fragments [t][ds], V^T fragments [dt] and the lane's
// bias entries.  bf16: the 16-byte fragments themselves.  E4M3: K as 16 codes
// per pair of k-steps [t][ds/2], V^T as 8 codes per fragment.
template <typename TKV> struct MqrSet;
template <> struct MqrSet<bf16> {
  u32x4 k[2][4], v[8];
  bf16 bias[kBandSlots];
};
template <> struct MqrSet<fp8e4> {
  u32x4 k[2][2];
  u32x2 v[8];
  bf16 bias[kBandSlots];
};

// Max over the lane pairs (l, l ^ 16) and (l, l ^ 32), i.e. over the four
// lane groups of a column.  v_permlane16_swap / v_permlane32_swap exchange
// the two registers between the lane pair, so after each swap one register
// holds lane l's value and the other its partner's.  Written as one asm
// block: fmaxf would first quiet possibly signalling NaNs of the swapped
// values, four more instructions per column tile (the logits here are
// finite or -inf).  The two wait states before each swap cover its read of
// a register the previous instruction wrote.
__device__ __forceinline__ float col_max(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane16_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1\n\t"
      "v_mov_b32 %1, %0\n\t"
      "s_nop 1\n\t"
      "v_permlane32_swap_b32 %0, %1\n\t"
      "v_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

__device__ __forceinline__ Frag8<bf16> as_frag(const u32x4& w) {
  Frag8<bf16> f;
  f.v = w;
  return f;
}
__device__ __forceinline__ Frag8<bf16> as_frag(const u32x2& w) { return fp8x8_to_bf16(w[0], w[1]); }

template <typename TKV, int NCT>
__global__ __launch_bounds__(kRThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mqr_kernel(int Hq, int Hkv, int window, int R, int S, int B,
                       const bf16* __restrict__ q, const TKV* __restrict__ k_cache,
                       const TKV* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                       int max_blocks, const int32_t* __restrict__ cu_q,
                       const int32_t* __restrict__ seq_lens, const bf16* __restrict__ bias,
                       float* __restrict__ part_o, float* __restrict__ part_lse,
                       bf16* __restrict__ out, float* __restrict__ lse, float k_scale,
                       float v_scale) {
  constexpr bool kFp8 = std::is_same<TKV, fp8e4>::value;
  constexpr int kSz = (int)sizeof(TKV);
  constexpr int kSets = 3;
  constexpr uint32_t kPageBytes = kPage * kHeadDim * kSz;
  __shared__ MqrSmem<NCT> sm;

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
  const int n_items = max(my_hi - my_lo, 0);
  const float c = 0.08838834764831845f * kLog2e * k_scale;   // log2(e) / sqrt(128)

  // ---- Q^T fragments to LDS: fragment (ct, ds), lane ln holds column
  // 16ct + ln%16 (token = column / G, head = column % G) and the 8 dims of
  // lane group g = ln/16 in k-step ds: 32ds + 8g .. +7 (bf16 cache), or
  // 64(ds/2) + 16g + 8(ds%2) .. +7 (E4M3 cache).  The dot product may take
  // the dims in any order that Q and K share; the E4M3 order gives each lane
  // 16 consecutive K codes per pair of k-steps, one 16-byte load.  Columns
  // past n_cols are zero.
#pragma unroll
  for (int i = tid; i < NCT * 4 * 64; i += kRThreads) {
    const int ct = i >> 8, ds = (i >> 6) & 3, ln = i & 63;
    const int cc = 16 * ct + (ln & 15);
    u32x4 w = u32x4{0, 0, 0, 0};
    if (cc < n_cols) {
      const int token = cc / G, hh = kvh * G + cc % G;
      const int d0 = kFp8 ? 64 * (ds >> 1) + 16 * (ln >> 4) + 8 * (ds & 1) : 32 * ds + 8 * (ln >> 4);
      w = *reinterpret_cast<const u32x4*>(q + ((size_t)(tok0 + token) * Hq + hh) * kHeadDim + d0);
    }
    sm.q[i] = w;
  }

  // ---- per-lane column data: band offset of key 8grp + 0 of the item (the
  // lane's keys 8grp + e read offset - e).  Columns past n_cols read the
  // band of token 0, head 0: finite or -inf values nobody stores.
  int boff[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int cc = 16 * ct + col;
    const bool ok = cc < n_cols;
    const int token = ok ? cc / G : 0, hl = ok ? cc % G : 0;
    boff[ct] = band_base(hl) + token + (kItem - 1) - 8 * grp;
  }
  // Band staging: slot i of this lane is entry s = lane + 64i of the item's
  // band, head e = s / BW, offset v = s % BW (distance d_min + v).
  const int bw = (kItem - 1) + q_len;
  int bdst[kBandSlots], bsrc[kBandSlots];
#pragma unroll
  for (int i = 0; i < kBandSlots; ++i) {
    const int s = lane + 64 * i;
    const int e = s / bw, v = s - e * bw;
    const bool ok = s < G * bw;
    bdst[i] = ok ? band_base(e) + v : kBandFloats;   // (a spare float)
    bsrc[i] = ((kvh * G + (ok ? e : 0)) << 8) | v;          // bias row, offset v < 48
  }
  float* const band = sm.band[wave];
  // Each tile's band reads through an LDS pointer the compiler cannot see
  // into: its 8 reads then take small immediate offsets from one register
  // (the band array itself starts further into LDS than a ds_read2 offset
  // reaches, and each pair of reads would add it anew).
  typedef __attribute__((address_space(3))) const float lds_cfloat;
  lds_cfloat* bptr[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    bptr[ct] = (lds_cfloat*)(band + boff[ct] - 7);
    asm volatile("" : "+v"(bptr[ct]));
  }

  // ---- loads of item u (page my_hi - 1 - u, keys 32 wave .. +31 of it).
  const rsrc_t bias_r = make_rsrc(bias, (uint32_t)((size_t)Hq * R * sizeof(bf16)));
  auto item_key0 = [&](int u) { return (my_hi - 1 - u) * kPage + kItem * wave; };
  auto item_live = [&](int u) {
    const int key0 = item_key0(u);
    return u < n_items && key0 + kItem - 1 >= kstart && key0 < L;
  };
  auto page_base = [&](int u) {
    const int blk = my_hi - 1 - min(u, n_items - 1);
    const int phys = block_table[(size_t)b * max_blocks + blk];
    return ((size_t)phys * Hkv + kvh) * (size_t)(kPage * kHeadDim);
  };
  // K fragment (t, ds) of lane l: key 8(r/4) + 4t + r%4 (r = l%16), the
  // dims of lane group grp in k-step ds (the Q^T order above).
  const uint32_t k_voff =
      (uint32_t)(((kItem * wave + 8 * (col >> 2) + (col & 3)) * kHeadDim + (kFp8 ? 16 : 8) * grp) * kSz);
  // V^T fragment dt of lane l: dim 16dt + l%16, keys 8grp .. +7 of the item.
  const uint32_t v_voff = (uint32_t)((col * kPage + kItem * wave + 8 * grp) * kSz);
  // Item u's loads: K, the bias entries of its band, V^T.  Items past the
  // range, or outside every column's window, load through zero-length
  // descriptors (zeros, no bytes moved).
  auto load_item = [&](int u, MqrSet<TKV>& st) {
    const size_t base = page_base(u);
    const uint32_t bytes = item_live(u) ? kPageBytes : 0u;
    const rsrc_t kr = make_rsrc(k_cache + base, bytes);
    const rsrc_t vr = make_rsrc(v_cache + base, bytes);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (kFp8) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          st.k[t][j] = buf_load16(kr, k_voff, (uint32_t)(4 * t * kHeadDim + 64 * j));
      } else {
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          st.k[t][ds] = buf_load16(kr, k_voff, (uint32_t)((4 * t * kHeadDim + 32 * ds) * kSz));
      }
    }
    const int d_min = pos0 - item_key0(u) - (kItem - 1);
#pragma unroll
    for (int i = 0; i < kBandSlots; ++i) {
      const int dist = min(max(d_min + (bsrc[i] & 0xff), 0), R - 1);
      // Row start as a 24-bit product (R < 2^24, host check); the whole
      // table stays under 2^32 bytes, the buffer's offset range.
      const uint32_t elem = __umul24((uint32_t)bsrc[i] >> 8, (uint32_t)R) + (uint32_t)dist;
      st.bias[i] = buf_load_elem<bf16>(bias_r, elem * (uint32_t)sizeof(bf16));
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint32_t soff = (uint32_t)(16 * dt * kPage * kSz);
      if constexpr (kFp8) st.v[dt] = buf_load8(vr, v_voff, soff);
      else st.v[dt] = buf_load16(vr, v_voff, soff);
    }
    // Keep the item's loads together and in this order, so that each wait
    // the compiler places counts exactly the loads issued after them.
    __builtin_amdgcn_sched_barrier(0);
  };

  // Softmax reference per column: the max of the first item with a visible
  // key (O and the sum are still zero then, so nothing is rescaled), never
  // moved afterwards.  Probabilities may then exceed 1, up to 2^kBail; a
  // column whose later logits pass its reference by more than that sets
  // `over_lane`, and the wave runs its range a second time from the exact
  // column max (tracked in `m_all`).  O is only ever written by the matrix
  // products, so it stays in the accumulator registers for the whole loop.
  float m[NCT], l[NCT], m_all[NCT];
  bool over_lane = false;
  f32x4 o[NCT][8];                               // O^T: register r = dim 16dt + 4grp + r
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) m_all[ct] = -INFINITY;

  __syncthreads();                               // Q^T fragments staged

  // Item u: band to LDS, then a software pipeline over the column tiles.
  // Step i issues the S^T products of tile i+1, the PV products of tile i-1
  // and the softmax of tile i, which are independent, and reads the band
  // entries of tile i+1 for the next step; scheduling groups interleave the
  // matrix products with the vector instructions, so that the one wave of
  // each SIMD keeps the matrix core busy while it computes the softmax.
  auto item = [&](int u, const MqrSet<TKV>& st) {
    const int key0 = item_key0(u);
    // Band entry v is distance d_min + v; distances outside [0, window - 1]
    // (d < 0: a key after the token) hold -inf, which masks the key.
    const int d_min = pos0 - key0 - (kItem - 1);
#pragma unroll
    for (int i = 0; i < kBandSlots; ++i) {
      const int d = d_min + (bsrc[i] & 0xff);
      const bool vis = d >= 0 && (window == 0 || d < window);
      band[bdst[i]] = vis ? to_f32(st.bias[i]) * kLog2e : -INFINITY;
    }
    Frag8<bf16> kf[2][4], vf[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (kFp8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          kf[t][2 * j] = fp8x8_to_bf16(st.k[t][j][0], st.k[t][j][1]);
          kf[t][2 * j + 1] = fp8x8_to_bf16(st.k[t][j][2], st.k[t][j][3]);
        }
      } else {
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) kf[t][ds] = as_frag(st.k[t][ds]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vf[dt] = as_frag(st.v[dt]);
    if (key0 + kItem > L) {                      // (wave-uniform) keys past L in this item
      // Their K rows and V elements may hold any bits: zeroed, so that the
      // masked logits are exactly -inf and 0 * NaN never reaches O.
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool krow_ok = key0 + 8 * (col >> 2) + 4 * t + (col & 3) < L;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) kf[t][ds] = kf[t][ds].keep_first(krow_ok ? 8 : 0);
      }
      const int nvalid = L - (key0 + 8 * grp);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) vf[dt] = vf[dt].keep_first(nvalid);
    }
    // S^T of column tile ct.  An opaque offset keeps each tile's Q^T reads
    // next to its products (hoisted, the reads of all tiles would hold up to
    // 80 registers).
    int qi = lane;
    auto s_tile = [&](int ct, f32x4 (&a)[2]) {
      asm volatile("" : "+v"(qi));
      Frag8<bf16> qf[4];
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[ds].v = sm.q[qi + 64 * (4 * ct + ds)];
      a[0] = f32x4{0, 0, 0, 0};
      a[1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        a[0] = mfma16(kf[0][ds], qf[ds], a[0]);
        a[1] = mfma16(kf[1][ds], qf[ds], a[1]);
      }
    };
    auto band_read = [&](int ct, float (&bv)[8]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = bptr[ct][7 - e];
    };
    auto softmax = [&](int ct, const f32x4 (&sa)[2], const float (&bv)[8]) {
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = sa[e >> 2][e & 3] * c + bv[e];
        mx = fmaxf(mx, x[e]);
      }
      mx = col_max(mx);
      m_all[ct] = m_all[ct] > mx ? m_all[ct] : mx;
      m[ct] = m[ct] == -INFINITY ? mx : m[ct];
      over_lane = over_lane || mx > m[ct] + kBail;
      const float m_sub = m[ct] == -INFINITY ? 0.0f : m[ct];
      float p[8];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(x[e] - m_sub);
        psum += p[e];
      }
      l[ct] += psum;
      return Frag8<bf16>::pack(p);
    };
    f32x4 sacc[2][2];
    float bv[2][8];
    Frag8<bf16> pf;
    s_tile(0, sacc[0]);
    band_read(0, bv[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int step = 0; step <= NCT; ++step) {
      if (step + 1 < NCT) {
        s_tile(step + 1, sacc[(step + 1) & 1]);
        band_read(step + 1, bv[(step + 1) & 1]);
      }
      if (step >= 1) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[step - 1][dt] = mfma16(vf[dt], pf, o[step - 1][dt]);
      }
      if (step < NCT) pf = softmax(step, sacc[step & 1], bv[step & 1]);
      // LDS reads first, then one matrix product per three vector
      // instructions (2, 3, 5 and 8 measured within 1-2% of each other).
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- item loop: item v sits in register set v % kSets, loaded in the
  // iteration of item v - kSets right after that item's products, so kSets - 1
  // items are in flight while one is computed.  The loop starts at v = -kSets
  // so that the first items load through the same code, into the same
  // registers, as all later ones; it is unrolled by kSets so that every set
  // index is static.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      m[ct] = pass == 0 ? -INFINITY : m_all[ct];
      l[ct] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[ct][dt] = f32x4{0, 0, 0, 0};
    }
    over_lane = false;
    // Nothing of an earlier pass stays in flight: the wait analysis then
    // starts the item loop from an empty queue.
    __builtin_amdgcn_s_waitcnt(0);
    if (n_items > 0) {
      MqrSet<TKV> st[kSets];
      // One exit, at the end of the unrolled body: an exit after an inner
      // block would reach the loop head with that block's set loaded last,
      // and the wait analysis would then drain every set at the head.
      // Blocks past the last item skip their products and load nothing.
      for (int v0 = -kSets; v0 < n_items; v0 += kSets) {
#pragma unroll
        for (int r = 0; r < kSets; ++r) {
          const int v = v0 + r;                  // v % kSets == r
          if (v >= 0 && item_live(v)) item(v, st[r]);
          load_item(v + kSets, st[r]);
        }
      }
    }
    if (!__any(over_lane)) break;
  }

  // ---- merge the four waves' (max, sum, O) per column.
  float lt[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    lt[ct] = l[ct] + wave_shfl_xor(l[ct], 16);
    lt[ct] = pair_sum(lt[ct]);
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      sm.ml[wave][16 * ct + col][0] = m[ct];
      sm.ml[wave][16 * ct + col][1] = lt[ct];
    }
  }
  __syncthreads();
  float col_lse[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    float mw[kRWaves], lw[kRWaves];
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRWaves; ++w) {
      mw[w] = sm.ml[w][16 * ct + col][0];
      lw[w] = sm.ml[w][16 * ct + col][1];
      mt = fmaxf(mt, mw[w]);
    }
    float f = 0.0f;
    col_lse[ct] = -INFINITY;
    if (mt != -INFINITY) {                       // some key of this split is visible
      float ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kRWaves; ++w) ls += lw[w] * fast_exp2(mw[w] - mt);
      f = fast_exp2(m[ct] - mt) * (v_scale / ls);
      col_lse[ct] = (mt + fast_log2(ls)) * kLn2;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ct][dt] *= f;
  }

  // Each wave owns dims 32 wave .. +31 (dim tiles 2 wave, 2 wave + 1), one
  // dim tile per round: the other three waves hand it their share through
  // LDS, the owner adds them and stores.
  size_t orow[NCT], prow[NCT];
  bool cok[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int cc = 16 * ct + col;
    cok[ct] = cc < n_cols;
    const int token = cok[ct] ? cc / G : 0, hh = kvh * G + (cok[ct] ? cc % G : 0);
    orow[ct] = (size_t)(tok0 + token) * Hq + hh;
    prow[ct] = orow[ct] * S + split;
  }
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
#pragma unroll
    for (int w2 = 0; w2 < kRWaves; ++w2) {
      if (w2 == wave) continue;
      const int slot = wave < w2 ? wave : wave - 1;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) sm.xch[w2][slot][ct][lane] = o[ct][2 * w2 + rd];
    }
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < kRWaves; ++w2) {
      if (w2 != wave) continue;
      const int dt = 2 * w2 + rd;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 a = o[ct][dt];
#pragma unroll
        for (int sl = 0; sl < kRWaves - 1; ++sl) a += sm.xch[w2][sl][ct][lane];
        if (!cok[ct]) continue;
        if (S == 1)
          store4(out + orow[ct] * kHeadDim + 16 * dt + 4 * grp, a[0], a[1], a[2], a[3]);
        else
          store4(part_o + prow[ct] * kHeadDim + 16 * dt + 4 * grp, a[0], a[1], a[2], a[3]);
      }
    }
    __syncthreads();
  }
  if (wave == 0 && grp == 0) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (!cok[ct]) continue;
      if (S == 1) {
        if (lse != nullptr) lse[orow[ct]] = col_lse[ct];
      } else {
        part_lse[prow[ct]] = col_lse[ct];
      }
    }
  }
}

template <typename TKV, int NCT>
void launch_mqr(const AttnShape& s, int num_seqs, int num_splits, const void* q,
                const void* k_cache, const void* v_cache, const int32_t* block_table,
                int max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                const void* bias, void* out, float* lse, float* part_o, float* part_lse,
                float k_scale, float v_scale, hipStream_t stream) {
  const unsigned groups = (unsigned)((long)num_splits * s.Hkv * num_seqs);
  hipLaunchKernelGGL((decode_mqr_kernel<TKV, NCT>), dim3(groups), dim3(kRThreads), 0, stream,
                     s.Hq, s.Hkv, s.window, s.bias_len, num_splits, num_seqs, (const bf16*)q,
                     (const TKV*)k_cache, (const TKV*)v_cache, block_table, max_blocks_per_seq,
                     cu_seqlens_q, seq_lens, (const bf16*)bias, part_o, part_lse, (bf16*)out,
                     lse, k_scale, v_scale);
}

}  // namespace

void launch_decode_mq_reg(const AttnShape& s, int num_seqs, int num_splits, int max_q_len,
                          const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                          const void* bias, void* out, float* lse, float* part_o,
                          float* part_lse, const float* fp8_scales, hipStream_t stream) {
  const int n_ct = decode_column_tiles(s.Hq / s.Hkv, max_q_len);
  auto go = [&](auto kv_tag, auto ct_tag) {
    using TKV = decltype(kv_tag);
    constexpr int kCT = decltype(ct_tag)::value;
    launch_mqr<TKV, kCT>(s, num_seqs, num_splits, q, k_cache, v_cache, block_table,
                         max_blocks_per_seq, cu_seqlens_q, seq_lens, bias, out, lse, part_o,
                         part_lse, fp8_scales ? fp8_scales[0] : 1.0f,
                         fp8_scales ? fp8_scales[1] : 1.0f, stream);
  };
  auto by_ct = [&](auto kv_tag) {
    static_assert(kMaxRegMqTiles == 5, "instantiations below");
    switch (n_ct) {
      case 2: go(kv_tag, std::integral_constant<int, 2>{}); break;
      case 3: go(kv_tag, std::integral_constant<int, 3>{}); break;
      case 4: go(kv_tag, std::integral_constant<int, 4>{}); break;
      default: go(kv_tag, std::integral_constant<int, 5>{}); break;
    }
  };
  if (fp8_scales != nullptr) by_ct(fp8e4{});
  else by_ct(bf16{});
}

}  // namespace inkattn
