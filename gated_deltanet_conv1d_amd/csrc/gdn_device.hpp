// Device-side helpers shared by the GDN kernels (gfx950 / CDNA4 only).
//
// Wave64 everywhere.  Reductions over 16-lane DPP rows use quad_perm /
// row_half_mirror / row_mirror, so a "row" of 16 lanes can hold one vector
// of a head split 16 ways.  MFMA helpers cover the 16x16 fp32-accumulator
// shapes used by the chunked prefill: bf16 16x16x32 and fp32 16x16x4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

// 8 consecutive activations <-> 8 floats.  bf16: one 16-byte access; fp32: two.
__device__ __forceinline__ void load8(const bf16* p, float* v) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// 4 consecutive activations -> 4 floats (8 bytes bf16, 16 bytes fp32).
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}

// Nontemporal vector access, for streams a kernel touches once (the loaded or
// stored lines are not kept for reuse).
template <typename V>
__device__ __forceinline__ V nt_ld(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void nt_st(const V& v, V* p) { __builtin_nontemporal_store(v, p); }
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 8 consecutive activations, nontemporal (as load8 / store8)
__device__ __forceinline__ void load8_nt(const bf16* p, float* v) {
  const u32x4_t u = nt_ld(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_nt(const float* p, float* v) {
  const f32x4 a = nt_ld(reinterpret_cast<const f32x4*>(p)), b = nt_ld(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8_nt(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = from_f32<bf16>(v[i]);
  nt_st(o, reinterpret_cast<bf16x8*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float* v) {
  nt_st(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p));
  nt_st(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(p) + 1);
}

// Raw bits of 8 consecutive activations, so a load can be issued early and
// converted later: one 16-byte vector for bf16, two for fp32.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_nt(const bf16* p) {
    const u32x4_t v = nt_ld(reinterpret_cast<const u32x4_t*>(p));
    u = make_uint4(v[0], v[1], v[2], v[3]);
  }
  __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_f32(float* v) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  uint4 u[2];
  __device__ __forceinline__ void load(const float* p) {
    u[0] = reinterpret_cast<const uint4*>(p)[0];
    u[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    const u32x4_t a = nt_ld(reinterpret_cast<const u32x4_t*>(p)), b = nt_ld(reinterpret_cast<const u32x4_t*>(p) + 1);
    u[0] = make_uint4(a[0], a[1], a[2], a[3]);
    u[1] = make_uint4(b[0], b[1], b[2], b[3]);
  }
  __device__ __forceinline__ void zero() { u[0] = u[1] = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_f32(float* v) const {
    const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
};

// ------------------------------------------------------------------ math
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// Hardware reciprocal and reciprocal square root (about 1 ulp; no denormal
// fix-up branches): every use has a normal, positive or well-scaled argument.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }
// x * sigmoid(x); for x -> -inf the reciprocal of +inf is 0, so the result is -0.
__device__ __forceinline__ float fast_silu(float x) { return x * fast_rcp(1.0f + fast_exp(-x)); }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x / (1.0f + expf(-x)); }
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }

// ------------------------------------------------------------- lane moves
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp<0x140>(v); // row_mirror
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ------------------------------------------------------------------ MFMA
// 16x16 output tile, fp32 accumulator: lane l holds rows 4*(l/16)+i (i<4) of
// column l%16.  Operand fragments hold 4 values per lane for each 16-wide
// block of the contraction index: lane group g = l/16 holds contraction
// indices 4g..4g+3 of that block.  The MFMA only pairs A's and B's slots, so
// this assignment is consistent for every instruction used here.
__device__ __forceinline__ void mma_k32(f32x4& acc, const bf16x4& a0, const bf16x4& a1, const bf16x4& b0,
                                        const bf16x4& b1) {
  bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  bf16x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// A lone 16-wide block runs as 16x16x32 with a zero upper half, so every bf16
// MFMA in a dependent chain has the same shape.  For a 16x16x16 product that
// takes a 16x16x32 product's result as its accumulator (or the reverse), this
// toolchain emits the two back to back with no wait states on gfx950, and the
// second reads a stale accumulator: such mixed chains came out wrong and
// different from run to run, and exact once 16 wait states separated the two.
// One shape per chain needs no waits (the hardware forwards the accumulator).
__device__ __forceinline__ void mma_k16(f32x4& acc, const bf16x4& a, const bf16x4& b) {
  const bf16x4 zero = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
  mma_k32(acc, a, zero, b, zero);
}
__device__ __forceinline__ void mma_k16(f32x4& acc, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k32(f32x4& acc, const f32x4& a0, const f32x4& a1, const f32x4& b0,
                                        const f32x4& b1) {
  mma_k16(acc, a0, b0);
  mma_k16(acc, a1, b1);
}

// Operand precision policy: what the LDS tiles and MFMA fragments hold.
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x4 type; };
template <> struct Frag<float> { typedef f32x4 type; };

template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const T* p);  // 4 consecutive values
template <> __device__ __forceinline__ bf16x4 lds_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x4*>(p);
}
template <> __device__ __forceinline__ f32x4 lds_frag<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::type frag_from(const f32x4& v, float s = 1.0f) {
  typename Frag<T>::type r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = from_f32<T>(v[i] * s);
  return r;
}

__device__ __forceinline__ bool slot_ok(int32_t s, int32_t n_slots) { return s >= 0 && s < n_slots; }

}  // namespace gdn
