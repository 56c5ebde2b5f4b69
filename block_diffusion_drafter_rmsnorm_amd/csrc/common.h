// Device helpers shared by the gfx950 kernels: number formats, MFMA operand
// fragments and wave-level reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;

// bfloat16 held as raw bits; arithmetic always goes through fp32.
struct bf16_t {
  uint16_t bits;
};
struct fp8_t {
  uint8_t bits;
};

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bfloat16, round to nearest, ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP E4M3 ("fn"): bias 7, 3 mantissa bits, largest finite 448, no infinity,
// NaN = S.1111.111.  Encode rounds to nearest even and saturates to +-448.
__device__ __forceinline__ uint8_t f32_to_e4m3(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  if (!(a == a)) return (uint8_t)(sign | 0x7fu);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7eu);
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (exact scaling, then RNE)
    const float q = __builtin_rintf(a * 512.0f);
    return (uint8_t)(sign | (uint32_t)q);  // q == 8 is the smallest normal, code 0x08
  }
  const uint32_t ua = __float_as_uint(a);
  uint32_t e = (ua >> 23) - 127u + 7u;      // 1..15
  const uint32_t mant = ua & 0x7fffffu;
  const uint32_t r = mant + 0x7ffffu + ((mant >> 20) & 1u);  // RNE at bit 20
  uint32_t m3 = r >> 20;                    // 0..8
  if (m3 == 8u) {
    m3 = 0u;
    e += 1u;
  }
  uint32_t code = (e << 3) | m3;
  if (code > 0x7eu) code = 0x7eu;
  return (uint8_t)(sign | code);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  const uint32_t s = ((uint32_t)c & 0x80u) << 24;
  const uint32_t e = ((uint32_t)c >> 3) & 15u, m = (uint32_t)c & 7u;
  float v = (e == 0u) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return __uint_as_float(__float_as_uint(v) | s);
}

template <typename T> struct Num;
template <> struct Num<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
  // value as stored, re-read as fp32 (identity)
  static __device__ __forceinline__ float round(float x) { return x; }
};
template <> struct Num<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t x) { return bf16_to_f32(x.bits); }
  static __device__ __forceinline__ bf16_t from_f(float x) { return bf16_t{f32_to_bf16(x)}; }
  static __device__ __forceinline__ float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
};
template <> struct Num<fp8_t> {
  static __device__ __forceinline__ float to_f(fp8_t x) { return e4m3_to_f32(x.bits); }
  static __device__ __forceinline__ fp8_t from_f(float x) { return fp8_t{f32_to_e4m3(x)}; }
  static __device__ __forceinline__ float round(float x) { return e4m3_to_f32(f32_to_e4m3(x)); }
};

// ---------------------------------------------------------------- MFMA fragments
// A fragment is 8 consecutive K elements held by one lane.  For a 16x16 output
// tile, lane l supplies row (A) or column (B) l % 16 and the lanes with the same
// l % 16 (l / 16 = 0..3) supply disjoint K groups, so a 32-wide K step is one
// bf16 MFMA 16x16x32 or eight fp32 MFMA 16x16x4.  The accumulator holds
// rows 4 * (l / 16) + i, column l % 16 of the 16x16 tile.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  uint4 v;
};
template <> struct Frag<float> {
  float4 lo, hi;
};

__device__ __forceinline__ void load_frag(Frag<bf16_t>& f, const bf16_t* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const float4*>(p);
  f.hi = *reinterpret_cast<const float4*>(p + 4);
}
__device__ __forceinline__ void store_frag(bf16_t* p, const Frag<bf16_t>& f) {
  *reinterpret_cast<uint4*>(p) = f.v;
}
__device__ __forceinline__ void store_frag(float* p, const Frag<float>& f) {
  *reinterpret_cast<float4*>(p) = f.lo;
  *reinterpret_cast<float4*>(p + 4) = f.hi;
}
__device__ __forceinline__ void zero_frag(Frag<bf16_t>& f) { f.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
  f.lo = make_float4(0.f, 0.f, 0.f, 0.f);
  f.hi = f.lo;
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a.v),
                                                __builtin_bit_cast(bf16x8_v, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// Build a fragment from 8 fp32 values.
// Two fp32 -> two bf16 (round to nearest even) in one instruction on gfx950;
// equal to f32_to_bf16 on every non-NaN input.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_hw v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void frag_from_f32(Frag<bf16_t>& f, const float* x) {
  f.v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ void frag_from_f32(Frag<float>& f, const float* x) {
  f.lo = make_float4(x[0], x[1], x[2], x[3]);
  f.hi = make_float4(x[4], x[5], x[6], x[7]);
}

// Eight raw elements of one storage type held in registers (a load issued now,
// converted to fp32 later so the load overlaps other work).
template <typename KT> struct Raw8;
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void to_f(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct Raw8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_f(float* o) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
      o[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
};
template <> struct Raw8<fp8_t> {
  uint2 v;
  __device__ __forceinline__ void load(const fp8_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint2(0, 0); }
  __device__ __forceinline__ void to_f(float* o) const {
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = e4m3_to_f32((uint8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xffu));
  }
};

// Four raw elements of one storage type.
template <typename KT> struct Raw4;
template <> struct Raw4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void to_f(float* o) const {
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Raw4<bf16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void to_f(float* o) const {
    o[0] = bf16_to_f32((uint16_t)(v.x & 0xffffu));
    o[1] = bf16_to_f32((uint16_t)(v.x >> 16));
    o[2] = bf16_to_f32((uint16_t)(v.y & 0xffffu));
    o[3] = bf16_to_f32((uint16_t)(v.y >> 16));
  }
};
template <> struct Raw4<fp8_t> {
  uint32_t v;
  __device__ __forceinline__ void load(const fp8_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void to_f(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = e4m3_to_f32((uint8_t)((v >> (8 * i)) & 0xffu));
  }
};

// Raw storage -> MFMA operand fragment (bit copy when no conversion is needed).
template <typename CT, typename KT>
__device__ __forceinline__ void raw_to_frag(Frag<CT>& f, const Raw8<KT>& r) {
  float t[8];
  r.to_f(t);
  frag_from_f32(f, t);
}
template <>
__device__ __forceinline__ void raw_to_frag<bf16_t, bf16_t>(Frag<bf16_t>& f, const Raw8<bf16_t>& r) {
  f.v = r.v;
}
template <>
__device__ __forceinline__ void raw_to_frag<float, float>(Frag<float>& f, const Raw8<float>& r) {
  f.lo = r.a;
  f.hi = r.b;
}
// Two 4-element pieces -> fragment, element e zeroed unless bit e of keep is set.
template <typename CT, typename KT>
__device__ __forceinline__ void raw4x2_to_frag(Frag<CT>& f, const Raw4<KT>& a, const Raw4<KT>& b,
                                               unsigned keep) {
  float t[8];
  a.to_f(t);
  b.to_f(t + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (!((keep >> e) & 1u)) t[e] = 0.f;
  frag_from_f32(f, t);
}
template <>
__device__ __forceinline__ void raw4x2_to_frag<bf16_t, bf16_t>(Frag<bf16_t>& f,
                                                               const Raw4<bf16_t>& a,
                                                               const Raw4<bf16_t>& b,
                                                               unsigned keep) {
  const uint32_t w[4] = {a.v.x, a.v.y, b.v.x, b.v.y};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = (((keep >> (2 * i)) & 1u) ? 0x0000ffffu : 0u) |
                       (((keep >> (2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
    o[i] = w[i] & m;
  }
  f.v = make_uint4(o[0], o[1], o[2], o[3]);
}

// Four E4M3 bytes -> two words of two bf16 each, by the gfx950 conversion
// instruction (exact: every E4M3 value is a bf16 value; equal to
// f32_to_bf16(e4m3_to_f32(.)) on every code but the NaN payload).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ __forceinline__ void raw_to_frag<bf16_t, fp8_t>(Frag<bf16_t>& f, const Raw8<fp8_t>& r) {
  uint32_t w[4];
  e4m3x4_to_bf16x4(r.v.x, w[0], w[1]);
  e4m3x4_to_bf16x4(r.v.y, w[2], w[3]);
  f.v = make_uint4(w[0], w[1], w[2], w[3]);
}
// Two 4-element pieces -> fragment, without masking.
template <typename CT, typename KT>
__device__ __forceinline__ void raw4x2_to_frag_all(Frag<CT>& f, const Raw4<KT>& a,
                                                   const Raw4<KT>& b) {
  float t[8];
  a.to_f(t);
  b.to_f(t + 4);
  frag_from_f32(f, t);
}
template <>
__device__ __forceinline__ void raw4x2_to_frag_all<bf16_t, bf16_t>(Frag<bf16_t>& f,
                                                                   const Raw4<bf16_t>& a,
                                                                   const Raw4<bf16_t>& b) {
  f.v = make_uint4(a.v.x, a.v.y, b.v.x, b.v.y);
}
template <>
__device__ __forceinline__ void raw4x2_to_frag_all<bf16_t, fp8_t>(Frag<bf16_t>& f,
                                                                  const Raw4<fp8_t>& a,
                                                                  const Raw4<fp8_t>& b) {
  uint32_t w[4];
  e4m3x4_to_bf16x4(a.v, w[0], w[1]);
  e4m3x4_to_bf16x4(b.v, w[2], w[3]);
  f.v = make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ void raw4x2_to_frag_all<float, float>(Frag<float>& f,
                                                                 const Raw4<float>& a,
                                                                 const Raw4<float>& b) {
  f.lo = a.v;
  f.hi = b.v;
}
// Fragment from two 4-element halves (elements 0..3 at p0, 4..7 at p1).
__device__ __forceinline__ void load_frag_halves(Frag<bf16_t>& f, const bf16_t* p0, const bf16_t* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0), b = *reinterpret_cast<const uint2*>(p1);
  f.v = make_uint4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ void load_frag_halves(Frag<float>& f, const float* p0, const float* p1) {
  f.lo = *reinterpret_cast<const float4*>(p0);
  f.hi = *reinterpret_cast<const float4*>(p1);
}
// Element e of a fragment zeroed unless bit e of keep is set.
__device__ __forceinline__ void frag_keep(Frag<bf16_t>& f, unsigned keep) {
  uint32_t w[4] = {f.v.x, f.v.y, f.v.z, f.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] &= (((keep >> (2 * i)) & 1u) ? 0x0000ffffu : 0u) |
            (((keep >> (2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
  f.v = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void frag_keep(Frag<float>& f, unsigned keep) {
  float t[8] = {f.lo.x, f.lo.y, f.lo.z, f.lo.w, f.hi.x, f.hi.y, f.hi.z, f.hi.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (!((keep >> e) & 1u)) t[e] = 0.f;
  f.lo = make_float4(t[0], t[1], t[2], t[3]);
  f.hi = make_float4(t[4], t[5], t[6], t[7]);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Reduce over the 16 lanes that share l / 16 (one accumulator row group).
__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// ---------------------------------------------------------------- activations
// Offset of element (r, k) of an activation matrix.  blk == 0: row-major with
// row stride ld.  blk == 1 (the operands of calls of at most 64 rows, which
// the narrow GEMMs stream): 16 x 32 blocks, ld the row width K (a multiple of
// 32) -- block (r / 16, k / 32) at ((r / 16) (K / 32) + k / 32) 512, element
// (r mod 16) 32 + k mod 32 inside it -- so the 16 rows x 32 columns of an MFMA
// A fragment are one contiguous 1 KB (bf16) rather than 16 separate 64-byte
// pieces of 16 rows.  A blocked matrix takes its row count rounded up to 16.
__host__ __device__ __forceinline__ int64_t act_off(int r, int k, int64_t ld, int blk) {
  return blk ? ((int64_t)(r >> 4) * (ld >> 5) + (k >> 5)) * 512 + (r & 15) * 32 + (k & 31)
             : (int64_t)r * ld + k;
}

// RoPE (cos, sin) of pos * theta^(-2i/D), the angle formed and reduced in fp64.
__device__ __forceinline__ float2 rope_cs(int pos, int i, int D, double log_theta) {
  const double inv = exp(-(2.0 * (double)i / (double)D) * log_theta);
  double s, c;
  sincos((double)pos * inv, &s, &c);
  return make_float2((float)c, (float)s);
}
