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

__device__ __forceinline__ float sigmoid(float x) {
  return 1.0f / (1.0f + exp2_fast(-x * LOG2E));
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
