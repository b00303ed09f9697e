// MFMA fragments for v_mfma_f32_16x16x32_bf16 on gfx950 (wave64).
//
// Lane layout of the instruction (checked on the device):
//   A (16 x 32, M x K): lane l holds row l % 16, k = 8 (l / 16) + j, j = 0..7
//   B (32 x 16, K x N): lane l holds col l % 16, k = 8 (l / 16) + j
//   C (16 x 16):        lane l holds col l % 16, rows 4 (l / 16) + r, r = 0..3
// A and B fragments share one layout, so a C tile can feed the next product
// as either operand without moving data, once its rows are read as K: two
// vertically adjacent C tiles (rows 0..15 and 16..31) give, in lane group
// gq = l / 16, the K indices {4 gq + r} and {16 + 4 gq + r}.  Every operand
// loaded from memory uses that same K order ("perm32" below), so the sum over
// K is unchanged.
//
// Two precisions share the code:
//   FragB   one bf16 fragment per operand (bf16 inputs),
//   FragS   an fp32 value carried as hi + lo bf16 (fp32 inputs); a product
//           takes three MFMAs (lo*hi + hi*lo + hi*hi), which keeps about 16
//           significant bits per operand.
#pragma once
#include <type_traits>

#include "kda_common.hpp"

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct FragB {
  bf16x8_t v;
};
struct FragS {
  bf16x8_t hi, lo;
};

// Element k-index of fragment slot j inside a 32-wide K step, lane group gq.
__device__ __forceinline__ int perm32(int gq, int j) {
  return (j < 4) ? (4 * gq + j) : (16 + 4 * gq + (j - 4));
}

__device__ __forceinline__ bf16x8_t pack8(const float (&x)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
  return r;
}

template <bool SPLIT> struct FragOf;
template <> struct FragOf<false> {
  using T = FragB;
};
template <> struct FragOf<true> {
  using T = FragS;
};
template <bool SPLIT> using Frag = typename FragOf<SPLIT>::T;

template <bool SPLIT> __device__ __forceinline__ Frag<SPLIT> make_frag(const float (&x)[8]);
template <> __device__ __forceinline__ FragB make_frag<false>(const float (&x)[8]) {
  return FragB{pack8(x)};
}
template <> __device__ __forceinline__ FragS make_frag<true>(const float (&x)[8]) {
  FragS f;
  f.hi = pack8(x);
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = x[j] - (float)f.hi[j];
  f.lo = pack8(r);
  return f;
}

__device__ __forceinline__ void mma(f32x4_t& c, const FragB& a, const FragB& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t& c, const FragS& a, const FragS& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
}

// Fragment from two runs of 4 elements (K order perm32): p0 -> slots 0..3,
// p1 -> slots 4..7.  bf16 storage loads the bits as they are; fp32 storage is
// split into hi + lo.
__device__ __forceinline__ FragB frag_from(const bf16* p0, const bf16* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  return FragB{__builtin_bit_cast(bf16x8_t, u)};
}
__device__ __forceinline__ FragS frag_from(const float* p0, const float* p1) {
  const float4 a = *reinterpret_cast<const float4*>(p0);
  const float4 b = *reinterpret_cast<const float4*>(p1);
  float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return make_frag<true>(x);
}

// Four consecutive values of a C-tile row-run stored to memory.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  const bf16x4_t v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *reinterpret_cast<bf16x4_t*>(p) = v;
}
__device__ __forceinline__ void store4(_Float16* p, float a, float b, float c, float d) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  const f16x4_t v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
  *reinterpret_cast<f16x4_t*>(p) = v;
}

}  // namespace kda
