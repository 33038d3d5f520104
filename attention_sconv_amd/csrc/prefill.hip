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
// * K and V^T tiles of 64 keys are staged global -> registers -> LDS in
//   padded rows (conflict-free fragment reads at fixed offsets),
//   double-buffered with one barrier per tile; the next tile's loads are in
//   flight while the current tile is computed.
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
#include "device_common.h"
#include "launch.h"

namespace inkattn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;         // query rows per work-group (32 per wave)
constexpr int kBK = 64;                  // keys per KV tile
constexpr int kBand = kBQ + kBK - 1;     // 319 distinct distances per tile
// Copy stride of the band in LDS: 336 words = 16 (mod 64), so the four
// copies start 4 bank groups apart and the 16 lanes of a quarter-wave
// (4 copies x 4 consecutive 16-byte groups) hit 16 distinct bank groups.
constexpr int kBandPad = 336;
static_assert(kBandPad >= kBand + 1 && kBandPad % 64 == 16, "band copy stride");
constexpr int kStageFrags = kBK * kHeadDim / 8 / kThreads;   // fragments per thread per tile
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;    // log2 units
static_assert(kStageFrags * kThreads * 8 == kBK * kHeadDim, "staging covers one tile");
static_assert((kBQ - 1) % 4 == 3, "band copy selection assumes kBQ % 4 == 0");
static_assert(kBand <= kThreads, "one band entry per thread");

// LDS rows are padded by one 16-byte bf16 fragment: a K row is 272 B, a V^T
// row 144 B.  ds_read_b128 is served a quarter-wave (16 lanes) at a time over
// 64 banks; a quarter reads one fragment column from 16 distinct rows, and
// with these strides row r starts 17r (K) or 9r (V^T) bank groups in, which
// is 16 distinct groups mod 16.  Unlike an XOR swizzle, padding keeps every
// fragment read at (per-lane base + compile-time offset), so the LDS reads
// cost no address arithmetic.
constexpr int kKStride = kHeadDim + 8;   // elements per K row in LDS
constexpr int kVStride = kBK + 8;        // elements per V^T row in LDS

template <typename T>
struct PrefillSmem {
  T k[2][kBK * kKStride];                // [key][d]
  T vt[2][kHeadDim * kVStride];          // [d][key]
  float band[2][4][kBandPad];            // copy s holds band[v + s]
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
};

// Row r of a 32-row S^T tile holds key keyperm(r): accumulator register j of
// lane group g then holds key 16*(j/8) + 8*g + j%8 (see device_common.h for
// the accumulator layout), i.e. each lane owns runs of 8 consecutive keys,
// which is the B-operand layout the P^T V^T product needs.
__device__ __forceinline__ int keyperm(int r) {
  const int a = r >> 3, g = (r >> 2) & 1, c = r & 3;
  return 16 * (a >> 1) + 8 * g + 4 * (a & 1) + c;
}

template <typename T>
struct Stage {
  Frag8<T> k[kStageFrags], v[kStageFrags];
  float band;
};

template <typename T>
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  Frag8<T> qf[8];
  {
    const T* qrow = qp + ((size_t)(tok0 + row0 + a_row) * A.Hq + h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = row_ok ? Frag8<T>::load(qrow + 16 * ks) : Frag8<T>::zero();
  }

  const float sqrt_d = 11.313708498984761f;               // sqrt(128)
  const float c = kLog2e / sqrt_d;

  // ---- staging of one KV tile
  auto stage_load = [&](int jt, Stage<T>& s) {
    const int J0 = jt * kBK;
    const int phys = btab[J0 / kPage];
    const int koff = J0 % kPage;
    const size_t tile = ((size_t)phys * A.Hkv + kvg) * (size_t)(kPage * kHeadDim);
    // The whole 64-key slice lies inside one allocated page, so every load is
    // in bounds (keys >= seq_len of the last tile are cleaned up in LDS).
#pragma unroll
    for (int p = 0; p < kStageFrags; ++p) {
      const int F = tid + kThreads * p;
      const int r = F >> 4, f = F & 15;                   // K: 64 rows x 16 fragments
      s.k[p] = Frag8<T>::load(kc + tile + (size_t)(koff + r) * kHeadDim + 8 * f);
      const int d = F >> 3, fv = F & 7;                   // V^T: 128 rows x 8 fragments
      s.v[p] = Frag8<T>::load(vc + tile + (size_t)d * kPage + koff + 8 * fv);
    }
    if (tid < kBand) {
      const int dist = P0 - J0 + (kBQ - 1) - tid;
      const bool vis = dist >= 0 && (A.window == 0 || dist < A.window);
      s.band = vis ? to_f32(bias_h[min(dist, A.R - 1)]) * sqrt_d : -INFINITY;
    }
  };
  auto stage_store = [&](int buf, const Stage<T>& s) {
#pragma unroll
    for (int p = 0; p < kStageFrags; ++p) {
      const int F = tid + kThreads * p;
      const int r = F >> 4, f = F & 15;
      s.k[p].store(&sm.k[buf][r * kKStride + 8 * f]);
      const int d = F >> 3, fv = F & 7;
      s.v[p].store(&sm.vt[buf][d * kVStride + 8 * fv]);
    }
    if (tid < kBand) {
#pragma unroll
      for (int sh = 0; sh < 4; ++sh)
        if (tid - sh >= 0) sm.band[buf][sh][tid - sh] = s.band;
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

  const int kp = keyperm(lq);
  const int band_shift = (3 - (lane & 3)) & 3;

  Stage<T> st;
  stage_load(jt_lo, st);
  stage_store(0, st);
  __syncthreads();

  // Keys >= seq_len exist only in the sequence's last tile.  They hold no
  // data (possibly NaN), so before that tile is used its K rows and V^T
  // columns past seq_len are zeroed in LDS: 0 * garbage must not reach O,
  // and the masked logits must stay -inf rather than NaN.
  const int n_tail = seq_len - jt_hi * kBK;               // valid keys of the last tile
  auto clean_tail = [&](int buf) {
#pragma unroll
    for (int p = 0; p < kStageFrags; ++p) {
      const int F = tid + kThreads * p;
      const int r = F >> 4, f = F & 15;
      if (r >= n_tail) Frag8<T>::zero().store(&sm.k[buf][r * kKStride + 8 * f]);
      const int d = F >> 3, fv = F & 7;
      if (8 * fv + 8 > n_tail) {
        T* q8 = &sm.vt[buf][d * kVStride + 8 * fv];
        Frag8<T>::load(q8).keep_first(n_tail - 8 * fv).store(q8);
      }
    }
  };

  for (int jt = jt_lo; jt <= jt_hi; ++jt) {
    const int buf = (jt - jt_lo) & 1;
    const bool has_next = jt < jt_hi;
    if (jt == jt_hi && n_tail < kBK) {          // wave-uniform, once per work-group
      clean_tail(buf);
      __syncthreads();
    }
    if (has_next) stage_load(jt + 1, st);

    // LDS fragment reads run ahead of the MFMAs that consume them (K two
    // steps ahead, the first V slab before the softmax, later V slabs one
    // slab ahead) so that LDS latency overlaps matrix work.
    auto kfrag = [&](int ks, int t) {
      const int kr = 32 * t + kp;
      return Frag8<T>::load(&sm.k[buf][kr * kKStride + 8 * (2 * ks + lg)]);
    };
    auto vfrag = [&](int slab, int dt) {
      const int dr = 32 * dt + lq;
      return Frag8<T>::load(&sm.vt[buf][dr * kVStride + 8 * (2 * slab + lg)]);
    };
    Frag8<T> kq[3][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int t = 0; t < 2; ++t) kq[j][t] = kfrag(j, t);

    // S^T accumulators start as the sheared bias band.
    f32x16 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int v0 = (kBQ - 1) - a_row + 32 * t + 16 * hh + 8 * lg;
        const float* bp = &sm.band[buf][band_shift][v0 - band_shift];
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(bp);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(bp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[t][8 * hh + e] = x0[e];
          acc[t][8 * hh + 4 + e] = x1[e];
        }
      }

    // (sched_barrier keeps the compiler from sinking the reads back next to
    // their uses, which would expose the full LDS latency on every MFMA.)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 2 < 8) {
#pragma unroll
        for (int t = 0; t < 2; ++t) kq[(ks + 2) % 3][t] = kfrag(ks + 2, t);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t] = mfma32(kq[ks % 3][t], qf[ks], acc[t]);
    }
    Frag8<T> vq[2][4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) vq[0][dt] = vfrag(0, dt);
    __builtin_amdgcn_sched_barrier(0);

    // ---- online softmax (base 2), lazy rescale
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[t][r]);
    mx = pair_max(mx);
    const float m_tile = mx * c;
    const bool need = m_tile > m_used + kRescaleSlack;
    if (__any(need)) {
      // Lanes that do not need it keep their max (alpha = 1); this also keeps
      // rows that have seen no key yet (m_used = -inf) free of -inf - -inf.
      const float alpha = need ? fast_exp2(m_used - m_tile) : 1.0f;   // -inf -> 0
      l_sum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      m_used = need ? m_tile : m_used;
    }
    const float msub = m_used == -INFINITY ? 0.0f : m_used;
    Frag8<T> pf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = fast_exp2(acc[t][8 * hh + e] * c - msub);
        pf[2 * t + hh] = Frag8<T>::pack(p);
        l_sum = pf[2 * t + hh].sum_into(l_sum);     // sums the values fed to P V
      }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int slab = 0; slab < 4; ++slab) {
      if (slab + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vq[(slab + 1) & 1][dt] = vfrag(slab + 1, dt);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(vq[slab & 1][dt], pf[slab], o[dt]);
    }

    if (has_next) stage_store(buf ^ 1, st);
    __syncthreads();
  }

  // ---- epilogue: O^T register r of tile dt is dim 32dt + 8(r/4) + 4lg + r%4
  const float lt = pair_sum(l_sum);
  if (!row_ok) return;
  const float inv = 1.0f / lt;
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
                          const void* bias, void* out, float* lse, hipStream_t stream) {
  PrefillArgs a;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
  a.cu_q = cu_seqlens_q; a.seq_lens = seq_lens; a.bias = bias; a.out = out; a.lse = lse;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.Hq / s.Hkv; a.window = s.window; a.R = s.bias_len;
  a.max_blocks = max_blocks_per_seq; a.num_seqs = num_seqs;
  const int nqt = (max_q_len + kBQ - 1) / kBQ;
  a.total_groups = nqt * num_seqs * s.Hkv;
  const long padded = ((long)a.total_groups + kXcds - 1) / kXcds * kXcds;
  const long blocks = padded * a.G;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (s.dtype == kDtypeBf16)
    hipLaunchKernelGGL(prefill_kernel<bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace inkattn
