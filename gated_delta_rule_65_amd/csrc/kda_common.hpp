// Device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int D = 128;      // head size (K = V)
constexpr int C = 64;       // tokens per chunk
constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2_EPS = 1e-6f;

// Storage types of the inputs.
struct bf16 {
  uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) {
  return __uint_as_float(((uint32_t)v.x) << 16);
}
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) {
  return bf16{bf16_bits(f)};
}
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float f) {
  return (_Float16)f;
}

// 2^x on the hardware exp unit.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// 1/sqrt(x) on the hardware unit, for arguments kept normal by an epsilon.
__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp): the denominator is
// >= 1 or +inf, so there is no denormal or overflow case, and saturated inputs
// give exactly 1 and 0.
__device__ __forceinline__ float sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * LOG2E));
}

// Optional gate parameters (the raw gate g becomes the log-decay
// lower_bound * sigmoid(a (g + bias)), a = exp(A_log[h])).
struct GateArgs {
  const float* a_log;  // [Hv] or NULL
  const void* bias;    // [Hv, 128] fp32 or bf16
  int bias_bf16;
  float lower_bound;
};
// Elements between consecutive tokens of each input (heads stay 128 apart
// inside a token, 1 apart for beta).
struct InStrides {
  int64_t q, k, v, g, beta;
};

__device__ __forceinline__ float gate_bias(const GateArgs& ga, int h, int c) {
  const size_t i = (size_t)h * D + c;
  return ga.bias_bf16 ? to_f32(reinterpret_cast<const bf16*>(ga.bias)[i])
                      : reinterpret_cast<const float*>(ga.bias)[i];
}
// The 8 biases of channels c0 .. c0 + 7 (c0 a multiple of 8).
__device__ __forceinline__ void gate_bias8(const GateArgs& ga, int h, int c0, float (&b)[8]) {
  const size_t i = (size_t)h * D + c0;
  if (ga.bias_bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16*>(ga.bias) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      b[2 * d] = __uint_as_float(w[d] << 16);
      b[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
    }
  } else {
    const float4 x = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(ga.bias) + i)[0];
    const float4 y = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(ga.bias) + i)[1];
    b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
    b[4] = y.x; b[5] = y.y; b[6] = y.z; b[7] = y.w;
  }
}
// The same 8 biases fetched as raw bits with no branch (two 16-byte loads,
// both inside the bias array: a bf16 row reads its one piece twice), so that a
// caller can issue them among other prefetches and decode them later.
__device__ __forceinline__ void gate_bias8_bits(const GateArgs& ga, int h, int c0, uint4& b0,
                                                uint4& b1) {
  const size_t i = (size_t)h * D + c0;
  const char* p = reinterpret_cast<const char*>(ga.bias) + i * (ga.bias_bf16 ? 2 : 4);
  b0 = *reinterpret_cast<const uint4*>(p);
  b1 = *reinterpret_cast<const uint4*>(p + (ga.bias_bf16 ? 0 : 16));
}
__device__ __forceinline__ void gate_bias8_decode(const GateArgs& ga, const uint4& b0,
                                                  const uint4& b1, float (&b)[8]) {
  const uint32_t w[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  if (ga.bias_bf16) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      b[2 * d] = __uint_as_float(w[d] << 16);
      b[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 8; ++d) b[d] = __uint_as_float(w[d]);
  }
}
__device__ __forceinline__ float gate_apply(float graw, float a, float bias, float lb) {
  return lb * sigmoid(a * (graw + bias));
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a full
// release/acquire fence and so also waits for every global load still in
// flight; this one waits for LDS traffic alone, so prefetches issued before it
// keep streaming across it.  (LDS DMA writes are covered by an explicit vmcnt
// wait before the barrier.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane moves inside a 16-lane DPP row.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

}  // namespace kda
