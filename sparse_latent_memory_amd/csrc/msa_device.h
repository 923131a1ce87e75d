// Device-side helpers shared by the libmsa kernels (gfx950 only): vector
// types, bf16 conversion, 16-byte loads, RoPE phasors, score keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kEps = 1e-8f;          // cosine norm clamp
constexpr float kEps2 = 1e-16f;        // kEps squared (clamp on squared norms)
constexpr int kMaxTopK = 4096;

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Storage is raw uint16_t; bf16 is the top half of an fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32 (NaN stays
// NaN), two values per instruction in the packed form.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Element access templated on the storage type: float or uint16_t (bf16).
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void put(float *p, int64_t i, float x) { p[i] = x; }
  __device__ static __forceinline__ void unpack(const u32x4 &v, float *o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ u32x4 pack(const float *o) {
    u32x4 v; v.x = __float_as_uint(o[0]); v.y = __float_as_uint(o[1]);
    v.z = __float_as_uint(o[2]); v.w = __float_as_uint(o[3]);
    return v;
  }
};
template <> struct Elt<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float get(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void put(uint16_t *p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
  __device__ static __forceinline__ void unpack(const u32x4 &v, float *o) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ u32x4 pack(const float *o) {
    u32x4 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]);
    v.w = pack_bf16x2(o[6], o[7]);
    return v;
  }
};

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Accurate (cos, sin) of pos * omega for a large integer position: the angle
// is formed in fp64 in revolutions (omega / 2pi), its integer part dropped
// exactly, and the remaining half-revolution fraction evaluated with fp32
// sincospi, whose argument reduction is exact (no large-argument path).
__device__ __forceinline__ void rope_phasor_rev(double pos, double rev_per_pos, float *c, float *s) {
  double r = pos * rev_per_pos;
  r -= rint(r);                               // |r| <= 1/2 revolution
  sincospif((float)(2.0 * r), s, c);
}
__device__ __forceinline__ void rope_phasor(double pos, double omega, float *c, float *s) {
  rope_phasor_rev(pos, omega * 0.15915494309189533577, c, s);
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// x combined over the lanes l, l ^ 16, l ^ 32 and l ^ 48 - the four lanes
// that hold one column of a 16x16 matrix-core result - with gfx950's lane
// swaps (v_permlane32_swap exchanges the upper half of one operand with the
// lower half of the other, v_permlane16_swap odd 16-lane rows with even
// ones; given the same value twice, the two results hold x of lane l and of
// lane l ^ 32, resp. l ^ 16, in every lane): VALU only, no LDS round trip.
__device__ __forceinline__ float col_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace msa
