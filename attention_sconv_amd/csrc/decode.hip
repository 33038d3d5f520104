// Split-K paged decode for relative-position GQA attention, plus the
// log-sum-exp merge of the splits.
//
// Source: news article "vLLM, TML Inkling Day-0 support", Model Architecture /
// Attention (GQA, head size 128, sliding-window and full layers, a learned
// relative-position term added to the logits) and vLLM Integration &
// Optimization / FA4 with sheared bias (the KV range is cut into a
// per-configuration number of splits).  Logit of query head h at position
// L-1 against key j:  q.k_j / sqrt(128) + bias[h][min(L-1-j, R-1)].
//
// Split kernel: one work-group of 8 waves per (split, kv-head, sequence),
// sized to fill one compute unit (2 waves per SIMD).  The split owns a
// contiguous run of 128-token pages of the sequence's key range, newest page
// first, cut into items of 32 keys (page, quarter; 64 keys, page and half,
// for an E4M3 cache) dealt round-robin: in round r wave w takes item 8r + w.
// The SIMD arbiter favours the older of its two waves; left alone, the
// favoured waves would finish their share early and leave the rest of the
// run at half occupancy, so the work-group meets at a barrier every four
// rounds (no wave runs more than four items ahead, and the order of every
// sum stays fixed: results are bitwise repeatable).  Measured on the 16K
// decode: no barrier costs 4% over a bf16 cache, a barrier every two rounds
// 3% over an E4M3 cache.  A wave reads its item's K and V straight from HBM
// into MFMA operand registers
// (16 B per lane per load, its next item prefetched while the current one is
// computed, also across the barrier), so the kernel streams each K/V byte of
// the range exactly once.  All Hq/Hkv query heads of the group
// ride along in one 16-wide MFMA column tile:
//   S^T[key][head] = K Q^T    (v_mfma 16x16x32, rows = keys, cols = heads)
//   O^T[d][head]  += V^T P^T  (v_mfma 16x16x32, rows = dims,  cols = heads)
// V is stored transposed per page (v_cache [block][kvh][d][token]) so that
// the A operand of the second product is 8 consecutive tokens of one dim, a
// contiguous 16 B load.  Rows of the first product are ordered so that lane
// group G ends up holding the probabilities of keys 8G .. 8G+7, exactly the
// B-operand layout of the second product (no shuffles).
// The eight waves merge their running (max, sum, O) through LDS and write one
// normalised partial output and its log-sum-exp per (sequence, head, split).
//
// Merge kernel: per (sequence, q-head), lse = log sum_s exp(lse_s) and
// out = sum_s exp(lse_s - lse) o_s; splits that saw no key have lse = -inf.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace inkattn {

namespace {

// Column tiles one 4-wave bf16 work-group carries (three fit its registers
// with the double-buffered K/V: 256 VGPRs and ~226 AGPRs; four spill).
constexpr int kMaxTilesPerGroup = 3;

// kW waves per work-group; kCT column tiles of 16 per work-group.  Plain
// decode and fp32 use <8, 1>.  bf16 with several tiles uses 4 waves (one per
// SIMD, so a wave may hold up to 512 registers) and keeps every tile's state
// in the same wave, so each K/V fragment it loads serves all of its tiles.
// Raw K/V registers of one item: the operand fragments themselves for a
// cache in the activation type (32-key items); for an E4M3 cache the codes,
// 8 per fragment, converted to bf16 fragments when the item is processed.
// With several column tiles an E4M3 item has 32 keys (K: this lane's 32 dims
// of its 2 keys, two 16-byte loads per key; V^T: 8 tokens of one dim, one
// 8-byte load per dim tile).  With one column tile (kWide) it has 64 keys, so
// that it carries the same 16 KB of K and V as a bf16 item and as many bytes
// are in flight per prefetched item: K holds 4 keys per lane (two 16-byte
// loads each), V^T 16 tokens of one dim per dim tile (one 16-byte load that
// feeds both PV k-steps).
template <typename T, typename TKV, bool kWide> struct ItemRegs {
  Frag8<T> k[8], v[8];
};
template <> struct ItemRegs<bf16, fp8e4, false> {
  u32x4 k[4];
  u32x2 v[8];
};
// The 64-key E4M3 item also carries this lane's 16 bias entries, packed two
// to a dword.  Its keys j0 .. j0+15 are distances pos-j0 .. pos-j0-15, 16
// consecutive entries of one bias row: fetched as 18 entries (9 dwords) from
// the even entry at or below the smallest, and aligned by `par` when used.
// Entries past R-1 are replaced by bias[R-1] where they are used; the one
// item per sequence whose distances reach below 15 while still visible (it
// holds the query position) has its entries fetched again one by one there.
template <> struct ItemRegs<bf16, fp8e4, true> {
  u32x4 k[8];
  u32x4 v[8];
  uint32_t bw[9];
  uint32_t par;
};

// TKV: the cache element type, T or fp8e4 (bf16 queries only).  An E4M3 cache
// holds keys / k_scale and values / v_scale: the scores take k_scale with the
// 1/sqrt(128) factor and the output takes v_scale (1 for other caches).
template <typename T, typename TKV, int kW, int kCT>
__global__ __launch_bounds__(64 * kW, 1) void decode_split_kernel(
    int Hq, int Hkv, int window, int R, int S, int n_cg, int B, const T* __restrict__ q,
    const TKV* __restrict__ k_cache, const TKV* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ seq_lens, const T* __restrict__ bias,
    float* __restrict__ part_o, float* __restrict__ part_lse, T* __restrict__ out,
    float* __restrict__ lse, float k_scale, float v_scale) {
  constexpr bool kFp8 = std::is_same<TKV, fp8e4>::value;
  static_assert(!kFp8 || std::is_same<T, bf16>::value, "E4M3 cache with bf16 queries");
  constexpr int kThr = 64 * kW;
  __shared__ float sm_m[kW][16];
  __shared__ float sm_l[kW][16];
  __shared__ float sm_o[kW][16][kHeadDim + 4];

  // Work-group id -> (split, kv-head, sequence, column group).  The column
  // groups of one (split, kv-head, sequence) get ids 8 apart: the hardware
  // deals ids round-robin over the 8 XCDs, so they run side by side on one
  // XCD and all but the first read the K/V range from its L2.  With one
  // column group this is the plain order (split fastest).
  const int id = blockIdx.x;
  const int cgi = (id >> 3) % n_cg;  // column group: tiles kCT*cgi .. kCT*cgi+kCT-1
  const int rest = (id & 7) + 8 * ((id >> 3) / n_cg);
  if (rest >= S * Hkv * B) return;               // (padding of the last group of 8)
  const int split = rest % S;
  const int kvh = (rest / S) % Hkv;
  const int b = rest / (S * Hkv);
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int col = lane & 15;      // MFMA column / row index for A loads
  const int grp = lane >> 4;      // lane group 0..3

  // The query tokens of sequence b (one for plain decode; up to a few draft
  // tokens when several positions are verified at once) sit at positions
  // L-q_len .. L-1.  Column c of a kv-head group is (token c / G, head
  // c % G); column tile t holds columns 16t .. 16t+15.
  const int tok0 = cu_q != nullptr ? cu_q[b] : b;
  const int q_len = cu_q != nullptr ? cu_q[b + 1] - tok0 : 1;
  const int n_cols = G * q_len;
  if (16 * kCT * cgi >= n_cols) return;          // (wave-uniform: the whole work-group)
  const int L = seq_lens[b];
  const int pos0 = L - q_len;                    // position of the first query token
  const int kstart = window > 0 ? max(0, pos0 - window + 1) : 0;
  const int blk_first = kstart >> 7;
  const int blk_last = (L - 1) >> 7;
  const int nblk = blk_last - blk_first + 1;
  const int bps = (nblk + S - 1) / S;
  const int my_lo = blk_first + split * bps;
  const int my_hi = min(my_lo + bps, blk_last + 1);
  // Items: kIK keys each, 2^kIL per page.  Item i is page my_hi-1 - i / 2^kIL,
  // keys kIK (i % 2^kIL) .. of it; lane group G holds kKL consecutive keys.
  // Pages are taken newest first: the page that the step's sconv has just
  // written (lines partly dirty in the caches, slower to read) is then
  // fetched while the rest of the range is still streaming, not at the end
  // (a one-token step over 16K keys: 0.098 -> 0.096 ms after its sconv).
  constexpr bool kWide = kFp8 && kCT == 1;
  constexpr int kIK = kWide ? 64 : 32;           // keys per item
  constexpr int kIL = kWide ? 1 : 2;             // log2(items per page)
  constexpr int kKL = kIK / 4;                   // keys per lane group
  constexpr int kRT = kIK / 16;                  // S^T row tiles per item
  const int n_items = (max(my_hi - my_lo, 0)) << kIL;

  // Per column tile u of this work-group: this lane's column, its query
  // position and visible keys k_lo .. pos, its bias row (an element index
  // into the whole table, which the entry point keeps under 2 GiB), its Q^T
  // fragments and running softmax state.
  const rsrc_t bias_r = make_rsrc(bias, (uint32_t)((size_t)Hq * R * sizeof(T)));
  bool head_ok[kCT];
  int pos[kCT], k_lo[kCT];
  uint32_t bias_row[kCT];
  Frag8<T> qf[kCT][4];
  float m[kCT], l[kCT];                          // running max (log2 units), this lane's sum
  f32x4 o[kCT][8];
#pragma unroll
  for (int u = 0; u < kCT; ++u) {
    const int gc = 16 * (kCT * cgi + u) + col;
    head_ok[u] = gc < n_cols;
    const int token = head_ok[u] ? gc / G : 0;
    const int h = kvh * G + (head_ok[u] ? gc % G : 0);
    pos[u] = pos0 + token;
    k_lo[u] = window > 0 ? max(0, pos[u] - window + 1) : 0;
    bias_row[u] = (uint32_t)h * (uint32_t)R;
    // k-step ds of lane group grp contracts dims 32ds+8grp .. +7; with an
    // E4M3 cache the dims are dealt 32grp+8ds .. +7 instead, so that a lane's
    // four k-steps are 32 consecutive bytes of a key row.
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qf[u][ds] = head_ok[u] ? Frag8<T>::load(q + ((size_t)(tok0 + token) * Hq + h) * kHeadDim +
                                              (kFp8 ? 32 * grp + 8 * ds : 32 * ds + 8 * grp))
                             : Frag8<T>::zero();
    m[u] = -INFINITY;
    l[u] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[u][dt] = f32x4{0, 0, 0, 0};
  }
  const float c = 0.08838834764831845f * kLog2e * k_scale;   // log2(e) / sqrt(128)
  // bias[h][R-1] of this lane's head (the entry every distance past the
  // table takes), for the E4M3 items' bias runs
  const float bias_last = kWide ? to_f32(buf_load_elem<T>(bias_r, (bias_row[0] + R - 1) * sizeof(T)))
                                : 0.0f;

  auto page_base = [&](int blk) -> size_t {
    const int phys = block_table[(size_t)b * max_blocks + blk];
    return ((size_t)phys * Hkv + kvh) * (size_t)(kPage * kHeadDim);
  };
  // Row r of the S^T tile t of item i is key kKL*(r/4) + 4t + r%4 of the
  // item, so accumulator register r of lane group G in tile t holds key
  // kKL*G + 4t + r: lane group G ends up with keys kKL*G .. kKL*G + kKL-1,
  // the B-operand layout of P^T (8 keys per PV k-step).
  // Everything an item needs is loaded in one batch, one item ahead: K and
  // V^T fragments and, per column tile, the 8 bias entries of this lane's
  // keys.  Bias indices are clamped into the table (masked keys are dropped
  // later by a select), so no load sits behind a branch and no wait drains
  // the prefetch.
  // Each page is read through a buffer descriptor of its own; the quarter
  // and the dim tile are wave-uniform offsets, so the only per-lane address
  // state is one fixed byte offset for K and one for V^T.
  constexpr uint32_t kPageBytes = kPage * kHeadDim * sizeof(TKV);
  const uint32_t k_lane =
      ((kKL * (col >> 2) + (col & 3)) * kHeadDim + (kFp8 ? 32 : 8) * grp) * sizeof(TKV);
  const uint32_t v_lane = (col * kPage + kKL * grp) * sizeof(TKV);
  using Regs = ItemRegs<T, TKV, kWide>;
  auto load_item = [&](int item, Regs& ir, T (*bb)[kKL]) {
    const int blk = my_hi - 1 - (item >> kIL);
    const int qu = item & ((1 << kIL) - 1);
    const int j0 = blk * kPage + kIK * qu + kKL * grp;
    if constexpr (kWide) {
      // (a run that starts before the table, in the newest item of head 0,
      // reads as zeros: such items are fetched again where they are used)
      const int first = (int)bias_row[0] + pos[0] - j0 - (kKL - 1);
      ir.par = (uint32_t)first & 1u;
      const uint32_t off = ((uint32_t)first & ~1u) * (uint32_t)sizeof(T);
      const u32x4 w0 = buf_load16(bias_r, off, 0);
      const u32x4 w1 = buf_load16(bias_r, off + 16, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ir.bw[i] = w0[i];
        ir.bw[4 + i] = w1[i];
      }
      ir.bw[8] = __builtin_amdgcn_raw_buffer_load_b32(bias_r, off + 32, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < kCT; ++u)
#pragma unroll
        for (int e = 0; e < kKL; ++e)
          bb[u][e] = buf_load_elem<T>(
              bias_r, (bias_row[u] + min(max(pos[u] - (j0 + e), 0), R - 1)) * sizeof(T));
    }
    const size_t base = page_base(blk);
    const rsrc_t kr = make_rsrc(k_cache + base, kPageBytes);
    const rsrc_t vr = make_rsrc(v_cache + base, kPageBytes);
    if constexpr (kWide) {
#pragma unroll
      for (int t = 0; t < kRT; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          ir.k[t * 2 + hh] = buf_load16(kr, k_lane + 4 * t * kHeadDim + 16 * hh,
                                        kIK * qu * kHeadDim);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        ir.v[dt] = buf_load16(vr, v_lane, kIK * qu + 16 * dt * kPage);
    } else if constexpr (kFp8) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          ir.k[t * 2 + hh] = buf_load16(kr, k_lane + 4 * t * kHeadDim + 16 * hh,
                                        32 * qu * kHeadDim);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        ir.v[dt] = buf_load8(vr, v_lane, 32 * qu + 16 * dt * kPage);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          ir.k[t * 4 + ds] = Frag8<T>::load(kr, k_lane + (4 * t * kHeadDim + 32 * ds) * sizeof(T),
                                            32 * qu * kHeadDim * sizeof(T));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        ir.v[dt] = Frag8<T>::load(vr, v_lane, (32 * qu + 16 * dt * kPage) * sizeof(T));
    }
  };
  // Operand fragment (t, ds) of K and dim tile dt of V^T.
  auto k_frag = [&](const Regs& ir, int t, int ds) -> Frag8<T> {
    if constexpr (kFp8) {
      const u32x4& w = ir.k[t * 2 + (ds >> 1)];
      return fp8x8_to_bf16(w[2 * (ds & 1)], w[2 * (ds & 1) + 1]);
    } else {
      return ir.k[t * 4 + ds];
    }
  };
  auto v_frag = [&](const Regs& ir, int dt) -> Frag8<T> {
    if constexpr (kWide) return Frag8<T>::zero();   // (kWide items use v_frag_wide)
    else if constexpr (kFp8) return fp8x8_to_bf16(ir.v[dt][0], ir.v[dt][1]);
    else return ir.v[dt];
  };
  // PV k-step s of a 64-key item: tokens kKL*G + 8s .. +7 of dim tile dt.
  auto v_frag_wide = [&](const Regs& ir, int dt, int s) -> Frag8<T> {
    if constexpr (kWide) return fp8x8_to_bf16(ir.v[dt][2 * s], ir.v[dt][2 * s + 1]);
    else return Frag8<T>::zero();
  };

  // One 64-key E4M3 item, one column tile: scores, online softmax over the
  // lane's 16 keys, O^T += V^T P^T in two k-steps.  The K and V fragments are
  // converted right where the MFMAs consume them.
  auto process_item_wide = [&](int item, Regs& ir, const T (*bb)[kKL]) {
    const int blk = my_hi - 1 - (item >> kIL);
    const int j0 = blk * kPage + kIK * (item & ((1 << kIL) - 1)) + kKL * grp;
    f32x4 sacc[kRT];
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      sacc[t] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) sacc[t] = mfma16(k_frag(ir, t, ds), qf[0][ds], sacc[t]);
    }
    // Bias of key j0 + e: entry t = 15 - e of the aligned run, the low half
    // of dword t/2 for even t, the high half for odd t.  The shift goes
    // through an empty asm so that the alignment stays here, after the
    // item's loads have been waited for, and is not moved up to them.
    float bf[kKL];
    if constexpr (kWide) {
      uint32_t sh = 16u * ir.par;
      asm volatile("" : "+v"(sh));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t a = __builtin_amdgcn_alignbit(ir.bw[i + 1], ir.bw[i], sh);
        bf[15 - 2 * i] = __uint_as_float(a << 16);
        bf[14 - 2 * i] = __uint_as_float(a & 0xffff0000u);
      }
      const int top = pos[0] - j0;                 // distance of key j0
      if (__any(top > R - 1)) {                    // distances past the table: bias[R-1]
#pragma unroll
        for (int e = 0; e < kKL; ++e) bf[e] = top - e > R - 1 ? bias_last : bf[e];
      }
      if (__any(top < kKL - 1 && top >= 0)) {      // the item that holds the query position
#pragma unroll
        for (int e = 0; e < kKL; ++e) {
          const float v = to_f32(buf_load_elem<T>(
              bias_r, (bias_row[0] + min(max(top - e, 0), R - 1)) * sizeof(T)));
          bf[e] = top < kKL - 1 ? v : bf[e];
        }
      }
    }
    float x[kKL];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < kKL; ++e) {
      const int j = j0 + e;
      const bool ok = head_ok[0] && j >= k_lo[0] && j <= pos[0];
      x[e] = ok ? sacc[e >> 2][e & 3] * c + bf[e] * kLog2e : -INFINITY;
      mx = fmaxf(mx, x[e]);
    }
    mx = fmaxf(mx, wave_shfl_xor(mx, 16));
    mx = pair_max(mx);
    const float m_new = fmaxf(m[0], mx);
    const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m[0] - m_sub);        // m = -inf -> 0
    float p[kKL];
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < kKL; ++e) {
      p[e] = fast_exp2(x[e] - m_sub);
      psum += p[e];
    }
    l[0] = l[0] * alpha + psum;
    m[0] = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[0][dt] *= alpha;
    // Keys >= L of the last page may hold any bits: zeroed in V (wave-uniform
    // branch, per-lane select) so that 0 * garbage cannot reach O.
    const bool tail = blk == blk_last && (L & (kPage - 1)) != 0;
    const int nvalid = L - j0;
#pragma unroll
    for (int s = 0; s < kIK / 32; ++s) {
      const Frag8<T> pf = Frag8<T>::pack(p + 8 * s);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        Frag8<T> vf = v_frag_wide(ir, dt, s);
        if (tail) vf = vf.keep_first(nvalid - 8 * s);
        o[0][dt] = mfma16(vf, pf, o[0][dt]);
      }
    }
  };

  // One item (32 keys, or 64 for kWide), for every column tile: scores,
  // online softmax, O^T += V^T P^T.
  auto process_item = [&](int item, Regs& ir, const T (*bb)[kKL]) {
    if constexpr (kWide) {
      process_item_wide(item, ir, bb);
      return;
    }
    const int blk = my_hi - 1 - (item >> kIL);
    const int j0 = blk * kPage + kIK * (item & ((1 << kIL) - 1)) + kKL * grp;
    Frag8<T> kf[8], vf[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[t * 4 + ds] = k_frag(ir, t, ds);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vf[dt] = v_frag(ir, dt);
#pragma unroll
    for (int u = 0; u < kCT; ++u) {
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) sacc[t] = mfma16(kf[t * 4 + ds], qf[u][ds], sacc[t]);
      }

      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const bool ok = head_ok[u] && j >= k_lo[u] && j <= pos[u];
        x[e] = ok ? sacc[e >> 2][e & 3] * c + to_f32(bb[u][e]) * kLog2e : -INFINITY;
        mx = fmaxf(mx, x[e]);
      }
      mx = fmaxf(mx, wave_shfl_xor(mx, 16));
      mx = pair_max(mx);
      const float m_new = fmaxf(m[u], mx);
      const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = fast_exp2(m[u] - m_sub);       // m = -inf -> 0
      float p[8];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(x[e] - m_sub);
        psum += p[e];
      }
      l[u] = l[u] * alpha + psum;
      m[u] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[u][dt] *= alpha;

      const Frag8<T> pf = Frag8<T>::pack(p);
      // Keys >= L of the last page hold no data (possibly NaN): zero them in
      // V (once, before the first tile's product) so that 0 * garbage cannot
      // reach O.  The branch is wave-uniform; the per-lane part is a select,
      // never a divergent branch around the MFMA (matrix instructions must
      // run with every lane active).
      if (u == 0 && blk == blk_last && (L & (kPage - 1)) != 0) {
        const int nvalid = L - j0;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vf[dt] = vf[dt].keep_first(nvalid);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[u][dt] = mfma16(vf[dt], pf, o[u][dt]);
    }
  };

  // A wave's items alternate between two register sets, so the next item's
  // loads are in flight while the current one is computed and no register
  // copy (which would wait for those loads) is needed between rounds.
  // Inside the main loop every load is unconditional (a wave without an item
  // in the last round re-reads the split's last item, an L2 hit) so the
  // memory-wait bookkeeping stays exact and each item only waits for its own
  // loads; the last one or two rounds are peeled so that no load is issued
  // for a round that does not exist.  The barrier carries no memory fence:
  // it only holds waves together, it does not wait for their loads.
  Regs ra, rb;
  T ba[kCT][kKL], bbb[kCT][kKL];
  const int rounds = (n_items + kW - 1) / kW;
  auto item_of = [&](int r) { return min(r * kW + wave, n_items - 1); };
  auto has_item = [&](int r) { return r * kW + wave < n_items; };
  if (rounds > 0) load_item(item_of(0), ra, ba);
  int r = 0;
  for (; r + 2 < rounds; r += 2) {
    load_item(item_of(r + 1), rb, bbb);
    process_item(item_of(r), ra, ba);          // rounds before the last are full
    load_item(item_of(r + 2), ra, ba);
    process_item(item_of(r + 1), rb, bbb);
    if (r & 2) __builtin_amdgcn_s_barrier();     // every fourth round
  }
  if (r + 1 < rounds) {
    load_item(item_of(r + 1), rb, bbb);
    process_item(item_of(r), ra, ba);
    if (has_item(r + 1)) process_item(item_of(r + 1), rb, bbb);
  } else if (r < rounds && has_item(r)) {
    process_item(item_of(r), ra, ba);
  }

  // Merge the waves, one column tile at a time.  O^T register r of tile dt
  // is dim 16dt + 4G + r.
#pragma unroll
  for (int u = 0; u < kCT; ++u) {
    const int ct = kCT * cgi + u;
    if (16 * ct >= n_cols) break;                // (wave-uniform)
    if (u > 0) __syncthreads();                  // the previous tile's merge is done with LDS
    float lt = l[u] + wave_shfl_xor(l[u], 16);
    lt = pair_sum(lt);
    if (grp == 0) {
      sm_m[wave][col] = m[u];
      sm_l[wave][col] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sm_o[wave][col][16 * dt + 4 * grp + rr] = o[u][dt][rr];
    __syncthreads();

    const int tile_cols = min(16, n_cols - 16 * ct);
    for (int idx = threadIdx.x; idx < tile_cols * kHeadDim; idx += kThr) {
      const int hh = idx / kHeadDim;             // column within the tile
      const int d = idx % kHeadDim;
      const int cg = 16 * ct + hh;
      const size_t orow = (size_t)(tok0 + cg / G) * Hq + kvh * G + cg % G;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kW; ++w) M = fmaxf(M, sm_m[w][hh]);
      const size_t row = orow * S + split;
      if (M == -INFINITY) {
        part_o[row * kHeadDim + d] = 0.0f;
        if (d == 0) part_lse[row] = -INFINITY;
        continue;
      }
      float num = 0.0f, den = 0.0f;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float sc = fast_exp2(sm_m[w][hh] - M);
        num += sc * sm_o[w][hh][d];
        den += sc * sm_l[w][hh];
      }
      if (S == 1) {
        // A single split is the whole key range: write the result directly
        // (no merge pass).
        out[orow * kHeadDim + d] = from_f32<T>(num / den * v_scale);
        if (lse != nullptr && d == 0) lse[orow] = (M + fast_log2(den)) * kLn2;
      } else {
        part_o[row * kHeadDim + d] = num / den * v_scale;
        if (d == 0) part_lse[row] = (M + fast_log2(den)) * kLn2;
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kHeadDim) void decode_merge_kernel(
    int Hq, int S, const float* __restrict__ part_o, const float* __restrict__ part_lse,
    T* __restrict__ out, float* __restrict__ lse) {
  // one work-group per (query token, q-head) on a 1-D grid (token counts
  // beyond the 65535 a grid's y dimension holds)
  const int h = blockIdx.x % Hq;
  const int t = blockIdx.x / Hq;                 // query token
  const int d = threadIdx.x;
  const size_t row0 = ((size_t)t * Hq + h) * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_lse[row0 + s]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float ls = part_lse[row0 + s];
    if (ls == -INFINITY) continue;
    const float w = fast_exp2((ls - M) * kLog2e);
    num += w * part_o[(row0 + s) * kHeadDim + d];
    den += w;
  }
  out[((size_t)t * Hq + h) * kHeadDim + d] = from_f32<T>(num / den);
  if (lse != nullptr && d == 0) lse[(size_t)t * Hq + h] = M + fast_log2(den) * kLn2;
}

}  // namespace

template <typename T, typename TKV, int kW, int kCT>
void launch_split(const AttnShape& s, int num_seqs, int num_splits, int n_cg, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  int max_blocks_per_seq, const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                  const void* bias, void* out, float* lse, float* part_o, float* part_lse,
                  float k_scale, float v_scale, hipStream_t stream) {
  // One work-group per (split, kv-head, sequence) x column group, in groups
  // of 8 (see the kernel's id mapping).
  const long rest = (long)num_splits * s.Hkv * num_seqs;
  hipLaunchKernelGGL((decode_split_kernel<T, TKV, kW, kCT>),
                     dim3((unsigned)((rest + 7) / 8 * 8 * n_cg)), dim3(64 * kW), 0, stream, s.Hq,
                     s.Hkv, s.window, s.bias_len, num_splits, n_cg, num_seqs, (const T*)q,
                     (const TKV*)k_cache, (const TKV*)v_cache, block_table, max_blocks_per_seq,
                     cu_seqlens_q, seq_lens, (const T*)bias, part_o, part_lse, (T*)out, lse,
                     k_scale, v_scale);
}

template <typename T>
void launch_merge(const AttnShape& s, int num_tokens, int num_splits, float* part_o,
                  float* part_lse, void* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(decode_merge_kernel<T>, dim3((unsigned)((long)s.Hq * num_tokens)),
                     dim3(kHeadDim), 0, stream,
                     s.Hq, num_splits, part_o, part_lse, (T*)out, lse);
}

hipError_t launch_decode(const AttnShape& s, int num_seqs, int num_tokens, int max_q_len,
                         int num_splits, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         int max_blocks_per_seq, const int32_t* cu_seqlens_q,
                         const int32_t* seq_lens, const void* bias, void* out, float* lse,
                         float* part_o, float* part_lse, const float* fp8_scales,
                         hipStream_t stream) {
  const int n_ct = decode_column_tiles(s.Hq / s.Hkv, max_q_len);
  const float ks = fp8_scales ? fp8_scales[0] : 1.0f;
  const float vs = fp8_scales ? fp8_scales[1] : 1.0f;
  if (decode_uses_reg_mq(s.dtype, s.Hq / s.Hkv, max_q_len, s.Hq, s.bias_len)) {
    launch_decode_mq_reg(s, num_seqs, num_splits, max_q_len, q, k_cache, v_cache, block_table,
                         max_blocks_per_seq, cu_seqlens_q, seq_lens, bias, out, lse, part_o,
                         part_lse, fp8_scales, stream);
    if (num_splits > 1) launch_merge<bf16>(s, num_tokens, num_splits, part_o, part_lse, out, lse, stream);
  } else if (decode_uses_lds_mq(s.dtype, s.Hq / s.Hkv, max_q_len)) {
    launch_decode_mq_lds(s, num_seqs, num_splits, q, k_cache, v_cache, block_table,
                         max_blocks_per_seq, cu_seqlens_q, seq_lens, bias, out, lse, part_o,
                         part_lse, fp8_scales, stream);
    if (num_splits > 1) launch_merge<bf16>(s, num_tokens, num_splits, part_o, part_lse, out, lse, stream);
  } else if (s.dtype == kDtypeBf16) {
    auto bf16_path = [&](auto kv_tag) {
      using TKV = decltype(kv_tag);
      if (n_ct == 1) {
        launch_split<bf16, TKV, 8, 1>(s, num_seqs, num_splits, 1, q, k_cache, v_cache,
                                      block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens,
                                      bias, out, lse, part_o, part_lse, ks, vs, stream);
      } else {
        // Several column tiles: up to kMaxTilesPerGroup per work-group, spread
        // evenly over the fewest groups.
        const int n_cg = (n_ct + kMaxTilesPerGroup - 1) / kMaxTilesPerGroup;
        const int per = (n_ct + n_cg - 1) / n_cg;
        auto go = [&](auto tag) {
          constexpr int kCT = decltype(tag)::value;
          launch_split<bf16, TKV, 4, kCT>(s, num_seqs, num_splits, n_cg, q, k_cache, v_cache,
                                          block_table, max_blocks_per_seq, cu_seqlens_q,
                                          seq_lens, bias, out, lse, part_o, part_lse, ks, vs,
                                          stream);
        };
        static_assert(kMaxTilesPerGroup == 3, "instantiations below");
        if (per == 2) go(std::integral_constant<int, 2>{});
        else go(std::integral_constant<int, 3>{});
      }
    };
    if (fp8_scales != nullptr) bf16_path(fp8e4{});
    else bf16_path(bf16{});
    if (num_splits > 1) launch_merge<bf16>(s, num_tokens, num_splits, part_o, part_lse, out, lse, stream);
  } else {
    launch_split<float, float, 8, 1>(s, num_seqs, num_splits, n_ct, q, k_cache, v_cache,
                                     block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens,
                                     bias, out, lse, part_o, part_lse, 1.0f, 1.0f, stream);
    if (num_splits > 1) launch_merge<float>(s, num_tokens, num_splits, part_o, part_lse, out, lse, stream);
  }
  return hipGetLastError();
}

}  // namespace inkattn
