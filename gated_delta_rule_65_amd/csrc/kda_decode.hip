// One-token KDA decode over a paged, V-first fp32 state cache, in place.
//
// Per (request n, value head h) with slot = state_indices[n] (identity when
// no index array is given), every state row v (one value channel; the row
// holds S[:, v] over the 128 key channels) evolves on its own:
//   row   <- exp(g) * row                     (decay on the key channels)
//   u_v    = b * (v[v] - row . kn)            (delta residual)
//   row   <- row + u_v * kn                   (rank-one write)
//   o[v]   = scale * row . qn                 (read after the write)
// which is gated_delta_rule_decode's in-place V-first fp32 case (page
// "mate.kda") with the per-row solve of KdaTcVerify (page
// "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify") at window 1.  A
// negative slot produces a zero output row and no state traffic (the null
// slot of KdaTcVerify); a slot at or past the pool size is treated the same
// way so that a bad index can never address outside the cache.  With gate
// parameters, g is a raw gate: log-decay = lower_bound sigmoid(exp(A_log[h])
// (g + dt_bias[h][c])), KdaTcVerify's activation.
//
// Mapping (HBM-bound: 64 KiB read + 64 KiB written per unit): one 256-thread
// workgroup per unit; 16 lanes (one DPP row) own one state row, each lane
// holding 8 key channels {4j..4j+3} and {64+4j..64+4j+3} (j = lane % 16) so
// that each float4 access of a 16-lane group is 256 contiguous bytes.  The
// 8 row-steps of a thread are all loaded before any arithmetic, which keeps
// 16 KiB per wave in flight.  The two dot products per row are 16-lane DPP
// reductions; (row . qn) after the write is formed as
// (decayed row . qn) + u_v (kn . qn) so that one reduction pass suffices.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

// This lane's 8 values of a V-first state row (key channels 4j..4j+3 and
// 64+4j..64+4j+3): fp32, or bf16 widened on load and rounded (to nearest
// even) on store.
__device__ __forceinline__ void row_load(const float* row, int j, float4 (&h)[2]) {
  h[0] = reinterpret_cast<const float4*>(row)[j];
  h[1] = reinterpret_cast<const float4*>(row)[16 + j];
}
__device__ __forceinline__ float4 widen4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void row_load(const bf16* row, int j, float4 (&h)[2]) {
  h[0] = widen4(reinterpret_cast<const uint2*>(row)[j]);
  h[1] = widen4(reinterpret_cast<const uint2*>(row)[16 + j]);
}
// The state is written back with nontemporal stores: the rows are not read
// again soon, and decode steps run back to back stream the pool faster when
// the written lines do not linger in the caches (256 x 32 fp32 rows:
// 0.215 -> 0.169 ms per back-to-back step).
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void row_store(float* row, int j, const float4 (&h)[2]) {
  f32x4_nt* p = reinterpret_cast<f32x4_nt*>(row);
  __builtin_nontemporal_store(f32x4_nt{h[0].x, h[0].y, h[0].z, h[0].w}, p + j);
  __builtin_nontemporal_store(f32x4_nt{h[1].x, h[1].y, h[1].z, h[1].w}, p + 16 + j);
}
__device__ __forceinline__ uint2 narrow4(float4 x) {
  return make_uint2((uint32_t)bf16_bits(x.x) | ((uint32_t)bf16_bits(x.y) << 16),
                    (uint32_t)bf16_bits(x.z) | ((uint32_t)bf16_bits(x.w) << 16));
}
__device__ __forceinline__ void row_store(bf16* row, int j, const float4 (&h)[2]) {
  u32x2_nt* p = reinterpret_cast<u32x2_nt*>(row);
  const uint2 a = narrow4(h[0]), b = narrow4(h[1]);
  __builtin_nontemporal_store(u32x2_nt{a.x, a.y}, p + j);
  __builtin_nontemporal_store(u32x2_nt{b.x, b.y}, p + 16 + j);
}
// Four consecutive elements widened to fp32 (one 16-byte or 8-byte load).
__device__ __forceinline__ void load4(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4(const bf16* p, float* x) {
  const float4 a = widen4(*reinterpret_cast<const uint2*>(p));
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4(const _Float16* p, float* x) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x & 0xffffu));
  x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x >> 16));
  x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y & 0xffffu));
  x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y >> 16));
}
// This lane's 8 channels of a 128-vector: 4j..4j+3 and 64+4j..64+4j+3.
template <typename T>
__device__ __forceinline__ void lane8(const T* p, int j, float (&x)[8]) {
  load4(p + 4 * j, x);
  load4(p + 64 + 4 * j, x + 4);
}
// One token's q, k and per-channel decay factor exp(g) on this lane's 8
// channels.  All loads are issued before the gate arithmetic so that they
// stay vector loads in one block.
template <typename T>
__device__ __forceinline__ void token_qk_decay(const T* qp, const T* kp, const T* gp, int j,
                                               int h, const GateArgs& ga, float ga_a,
                                               float (&qv)[8], float (&kv)[8],
                                               float (&al)[8]) {
  float gl[8];
  lane8(qp, j, qv);
  lane8(kp, j, kv);
  lane8(gp, j, gl);
  if (ga.a_log) {
    float bias[8];
    if (ga.bias_bf16) {
      lane8(reinterpret_cast<const bf16*>(ga.bias) + (size_t)h * D, j, bias);
    } else {
      lane8(reinterpret_cast<const float*>(ga.bias) + (size_t)h * D, j, bias);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) gl[e] = gate_apply(gl[e], ga_a, bias[e], ga.lower_bound);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) al[e] = exp2_fast(gl[e] * LOG2E);
}

// The stored value of a state element (bf16 state: rounded and widened back).
__device__ __forceinline__ float4 as_stored(float4 x, float*) { return x; }
__device__ __forceinline__ float4 as_stored(float4 x, bf16*) { return widen4(narrow4(x)); }

template <typename T, typename S>
__global__ __launch_bounds__(256) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, S* __restrict__ cache,
    const int32_t* __restrict__ idx, T* __restrict__ out, int hqk, int hv, float scale,
    int use_l2, int num_slots, const GateArgs ga, const InStrides is, int64_t slot_stride) {
  const int unit = blockIdx.x;
  const int req = unit / hv, h = unit - req * hv;
  const int hq = h / (hv / hqk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, rsub = lane >> 4;
  T* o = out + ((size_t)req * hv + h) * D;
  const int slot = idx ? idx[req] : req;
  if (slot < 0 || slot >= num_slots) {
    if (tid < D) o[tid] = from_f32<T>(0.0f);
    return;
  }
  S* st = cache + (size_t)slot * slot_stride + (size_t)h * (D * D);

  // Issue the state loads first: rows r = 16 s + 4 wave + rsub, s = 0..7.
  float4 hs[8][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) row_load(st + (16 * s + 4 * wave + rsub) * D, j, hs[s]);

  const T* qp = q + (size_t)req * is.q + hq * D;
  const T* kp = k + (size_t)req * is.k + hq * D;
  const T* gp = g + (size_t)req * is.g + h * D;
  const T* vp = v + (size_t)req * is.v + h * D;
  float qv[8], kv[8], al[8];
  const float ga_a = ga.a_log ? exp2_fast(ga.a_log[h] * LOG2E) : 0.f;  // exp(A_log[h])
  token_qk_decay(qp, kp, gp, j, h, ga, ga_a, qv, kv, al);
  float vr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) vr[s] = to_f32(vp[16 * s + 4 * wave + rsub]);
  const float b = sigmoid(to_f32(beta[(size_t)req * is.beta + h]));

  if (use_l2) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sq += qv[e] * qv[e];
      sk += kv[e] * kv[e];
    }
    sq = row_sum16(sq);
    sk = row_sum16(sk);
    const float rq = rsq(sq + L2_EPS), rk = rsq(sk + L2_EPS);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] *= rq;
      kv[e] *= rk;
    }
  }
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) kq += kv[e] * qv[e];
  kq = row_sum16(kq);

#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float x[8] = {hs[s][0].x, hs[s][0].y, hs[s][0].z, hs[s][0].w,
                  hs[s][1].x, hs[s][1].y, hs[s][1].z, hs[s][1].w};
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= al[e];
      pk += x[e] * kv[e];
      pq += x[e] * qv[e];
    }
    pk = row_sum16(pk);
    pq = row_sum16(pq);
    const float u = b * (vr[s] - pk);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += u * kv[e];
    const int r = 16 * s + 4 * wave + rsub;
    const float4 nh[2] = {make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
    row_store(st + r * D, j, nh);
    if (j == 0) o[r] = from_f32<T>(scale * (pq + u * kq));
  }
}

// Multi-token (speculative) decode: the same row mapping, with the state kept
// in registers across the request's tokens.  Request req starts from row
// idx[req][acc[req] - 1] (idx[req][0] without counts); after token t the state
// is written to row idx[req][t] when that row is in the pool.  A start row
// outside the pool (or a count outside [1, cols]) zeroes the request's output
// rows and touches no state.  This is gated_delta_rule_decode's [B, T]
// state_indices with num_accepted_tokens (page "mate.kda").
template <typename T, typename S>
__global__ __launch_bounds__(256) void decode_multi_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ g, const T* __restrict__ beta, S* __restrict__ cache,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ acc, T* __restrict__ out,
    int ntok, int cols, int hqk, int hv, float scale, int use_l2, int num_slots,
    const GateArgs ga, const InStrides is, int64_t slot_stride) {
  const int unit = blockIdx.x;
  const int req = unit / hv, h = unit - req * hv;
  const int hq = h / (hv / hqk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, rsub = lane >> 4;
  const int32_t* ir = idx + (size_t)req * cols;
  int row0 = -1;
  if (acc) {
    const int a = acc[req];
    if (a >= 1 && a <= cols) row0 = ir[a - 1];
  } else {
    row0 = ir[0];
  }
  if (row0 < 0 || row0 >= num_slots) {
    if (tid < D)
      for (int t = 0; t < ntok; ++t)
        out[(((size_t)req * ntok + t) * hv + h) * D + tid] = from_f32<T>(0.0f);
    return;
  }
  const S* st0 = cache + (size_t)row0 * slot_stride + (size_t)h * (D * D);
  float4 hs[8][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) row_load(st0 + (16 * s + 4 * wave + rsub) * D, j, hs[s]);
  const float ga_a = ga.a_log ? exp2_fast(ga.a_log[h] * LOG2E) : 0.f;  // exp(A_log[h])
  for (int t = 0; t < ntok; ++t) {
    const size_t tok = (size_t)req * ntok + t;
    const T* qp = q + tok * is.q + hq * D;
    const T* kp = k + tok * is.k + hq * D;
    const T* gp = g + tok * is.g + h * D;
    const T* vp = v + tok * is.v + h * D;
    float qv[8], kv[8], al[8];
    token_qk_decay(qp, kp, gp, j, h, ga, ga_a, qv, kv, al);
    float vr[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) vr[s] = to_f32(vp[16 * s + 4 * wave + rsub]);
    const float b = sigmoid(to_f32(beta[tok * is.beta + h]));
    if (use_l2) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sq += qv[e] * qv[e];
        sk += kv[e] * kv[e];
      }
      sq = row_sum16(sq);
      sk = row_sum16(sk);
      const float rq = rsq(sq + L2_EPS), rk = rsq(sk + L2_EPS);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qv[e] *= rq;
        kv[e] *= rk;
      }
    }
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq += kv[e] * qv[e];
    kq = row_sum16(kq);
    const int rt = ir[t];
    S* dst = (rt >= 0 && rt < num_slots)
                 ? cache + (size_t)rt * slot_stride + (size_t)h * (D * D)
                 : nullptr;
    T* o = out + (tok * hv + h) * D;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float x[8] = {hs[s][0].x, hs[s][0].y, hs[s][0].z, hs[s][0].w,
                    hs[s][1].x, hs[s][1].y, hs[s][1].z, hs[s][1].w};
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] *= al[e];
        pk += x[e] * kv[e];
        pq += x[e] * qv[e];
      }
      pk = row_sum16(pk);
      pq = row_sum16(pq);
      const float u = b * (vr[s] - pk);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += u * kv[e];
      // the next token starts from the state as stored (rounded when bf16)
      hs[s][0] = as_stored(make_float4(x[0], x[1], x[2], x[3]), (S*)nullptr);
      hs[s][1] = as_stored(make_float4(x[4], x[5], x[6], x[7]), (S*)nullptr);
      const int r = 16 * s + 4 * wave + rsub;
      if (dst) row_store(dst + r * D, j, hs[s]);
      if (j == 0) o[r] = from_f32<T>(scale * (pq + u * kq));
    }
  }
}

template <typename T, typename S>
static hipError_t launch_decode_t(const DecodeLaunch& L) {
  const dim3 grid((unsigned)((size_t)L.n * L.hv)), block(256);
  if (L.tokens > 1 || L.cols > 0) {
    hipLaunchKernelGGL((decode_multi_kernel<T, S>), grid, block, 0, (hipStream_t)L.stream,
                       (const T*)L.q, (const T*)L.k, (const T*)L.v, (const T*)L.g,
                       (const T*)L.beta, (S*)L.cache, L.idx, L.accepted, (T*)L.out, L.tokens,
                       L.cols, L.hqk, L.hv, L.scale, L.use_l2, L.num_slots, L.gate, L.strides,
                       L.slot_stride);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<T, S>), grid, block, 0, (hipStream_t)L.stream,
                     (const T*)L.q, (const T*)L.k, (const T*)L.v, (const T*)L.g,
                     (const T*)L.beta, (S*)L.cache, L.idx, (T*)L.out, L.hqk, L.hv, L.scale,
                     L.use_l2, L.num_slots, L.gate, L.strides, L.slot_stride);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_s(const DecodeLaunch& L) {
  return L.state_bf16 ? launch_decode_t<T, bf16>(L) : launch_decode_t<T, float>(L);
}

hipError_t launch_decode(const DecodeLaunch& L) {
  switch (L.dtype) {
    case 0: return launch_decode_s<float>(L);
    case 1: return launch_decode_s<bf16>(L);
    default: return launch_decode_s<_Float16>(L);
  }
}

}  // namespace kda
