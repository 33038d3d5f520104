// Device-side building blocks shared by the libinkattn kernels (gfx950 only).
//
// Element types: the library stores activations either as fp32 or as bf16
// (bit pattern in a uint16_t).  Arithmetic is always fp32.
//
// MFMA fragments.  Every matrix-core call in this library contracts over a
// run of k-values in which lane group G of the wave (G = lane/32 for the
// 32x32 shapes, lane/16 for the 16x16 shapes) supplies 8 consecutive
// k-values, 8G .. 8G+7, held as one "frag8" (8 elements of the storage type).
//   bf16: one v_mfma_f32_32x32x16_bf16 / v_mfma_f32_16x16x32_bf16;
//   fp32: eight v_mfma_f32_32x32x2_f32 / v_mfma_f32_16x16x4_f32, call e using
//         element e of every lane (so lane group G again supplies k = 8G+e).
// Both contract exactly the same (a, b) pairs, so one kernel template serves
// both storage types.
//
// Accumulator layouts (CDNA3/CDNA4 matrix cores):
//   32x32: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
//   16x16: lane l, register r holds row 4*(l/16) + r, column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace inkattn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct bf16 { uint16_t bits; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kHeadDim = 128;
constexpr int kPage = 128;          // KV-cache block (tokens per page)

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(uint32_t(x.bits) << 16);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return bf16{f32_to_bf16_bits(x)};
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer descriptor (gfx9 family): base address and byte count held in
// four scalar registers.  A load adds a 32-bit per-lane byte offset and a
// wave-uniform byte offset to the base, so wave-uniform address parts stay
// out of vector registers.  Word 3 selects untyped access with no swizzle.
// Reads past the byte count return zero rather than faulting.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
template <typename T> __device__ __forceinline__ T buf_load_elem(rsrc_t r, uint32_t voff);
template <> __device__ __forceinline__ bf16 buf_load_elem<bf16>(rsrc_t r, uint32_t voff) {
  return bf16{__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0))};
}
template <> __device__ __forceinline__ float buf_load_elem<float>(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// ---------------------------------------------------------------- frag8
template <typename T> struct Frag8;

template <> struct Frag8<bf16> {
  u32x4 v;                                   // 8 bf16, element e in bits 16*(e%2) of word e/2
  __device__ __forceinline__ static Frag8 load(const bf16* p) {
    Frag8 f; f.v = *reinterpret_cast<const u32x4*>(p); return f;
  }
  __device__ __forceinline__ static Frag8 load(rsrc_t r, uint32_t voff, uint32_t soff) {
    Frag8 f; f.v = buf_load16(r, voff, soff); return f;
  }
  __device__ __forceinline__ void store(bf16* p) const {
    *reinterpret_cast<u32x4*>(p) = v;
  }
  __device__ __forceinline__ static Frag8 zero() { Frag8 f; f.v = u32x4{0, 0, 0, 0}; return f; }
  __device__ __forceinline__ float get(int e) const {
    uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  // Pack 8 fp32 values (round to nearest even).
  __device__ __forceinline__ static Frag8 pack(const float* x) {
    Frag8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    return f;
  }
  // Keep elements e < n, zero the others (a per-lane select, no branch).
  __device__ __forceinline__ Frag8 keep_first(int n) const {
    Frag8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (2 * i < n) ? 0x0000ffffu : 0u;
      const uint32_t hi = (2 * i + 1 < n) ? 0xffff0000u : 0u;
      f.v[i] = v[i] & (lo | hi);
    }
    return f;
  }
  __device__ __forceinline__ bf16x8_t as_mfma() const {
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

template <> struct Frag8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ static Frag8 load(const float* p) {
    Frag8 f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
  }
  __device__ __forceinline__ static Frag8 load(rsrc_t r, uint32_t voff, uint32_t soff) {
    Frag8 f;
    f.lo = __builtin_bit_cast(f32x4, buf_load16(r, voff, soff));
    f.hi = __builtin_bit_cast(f32x4, buf_load16(r, voff + 16, soff));
    return f;
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<f32x4*>(p) = lo;
    *reinterpret_cast<f32x4*>(p + 4) = hi;
  }
  __device__ __forceinline__ static Frag8 zero() {
    Frag8 f; f.lo = f32x4{0, 0, 0, 0}; f.hi = f.lo; return f;
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
  __device__ __forceinline__ static Frag8 pack(const float* x) {
    Frag8 f;
    f.lo = f32x4{x[0], x[1], x[2], x[3]};
    f.hi = f32x4{x[4], x[5], x[6], x[7]};
    return f;
  }
  __device__ __forceinline__ Frag8 keep_first(int n) const {
    Frag8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.lo[e] = e < n ? lo[e] : 0.0f;
      f.hi[e] = e + 4 < n ? hi[e] : 0.0f;
    }
    return f;
  }
};

// Store 4 consecutive outputs (8 B for bf16, 16 B for fp32).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// ---------------------------------------------------------------- fp8 KV cache
// An FP8 cache element holds an OCP E4M3 code (1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits; largest finite value 448, no infinity) of the
// value divided by the cache's scale.  Every E4M3 value is exactly a bf16.
struct fp8e4 { uint8_t bits; };
constexpr float kFp8Max = 448.0f;

__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
// Four fp32 values -> four E4M3 codes in one word (byte e holds value e):
// clamped to +-448 first (saturation), then rounded to nearest even by
// v_cvt_pk_fp8_f32.
__device__ __forceinline__ uint32_t fp8x4_from_f32(float a, float b, float c, float d) {
  const auto sat = [](float x) { return fminf(fmaxf(x, -kFp8Max), kFp8Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}
// Eight E4M3 codes (byte e of word e/4 is element e) -> the bf16 fragment of
// their values, exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1).
__device__ __forceinline__ Frag8<bf16> fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  Frag8<bf16> f;
  f.v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  f.v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  f.v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  f.v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return f;
}

// 32x32 output, contracts 16 k-values (lane group lane/32 holds k = 8G..8G+7).
__device__ __forceinline__ f32x16 mfma32(const Frag8<bf16>& a, const Frag8<bf16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.as_mfma(), b.as_mfma(), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const Frag8<float>& a, const Frag8<float>& b, f32x16 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.get(e), b.get(e), c, 0, 0, 0);
  return c;
}
// 16x16 output, contracts 32 k-values (lane group lane/16 holds k = 8G..8G+7).
__device__ __forceinline__ f32x4 mfma16(const Frag8<bf16>& a, const Frag8<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.as_mfma(), b.as_mfma(), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const Frag8<float>& a, const Frag8<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.get(e), b.get(e), c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Reductions over the lane pair (l, l ^ 32) with v_permlane32_swap: after
// the swap one result register holds lane l's value and the other its
// partner's (which is which depends on the half), so max/sum of the two is
// the pair reduction in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace inkattn
