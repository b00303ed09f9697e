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
// holding 8 key channels (j = lane % 16): {4j..4j+3} and {64+4j..64+4j+3} for
// an fp32 state, so that each float4 access of a 16-lane group is 256
// contiguous bytes, and {8j..8j+7} for a bf16 state, so that a lane's share
// of a row is one 16-byte access.  q, k, g and the gate bias follow the same
// channel split.  The
// 8 row-steps of a thread are all loaded before any arithmetic, which keeps
// 16 KiB per wave in flight.  The two dot products per row are 16-lane DPP
// reductions; (row . qn) after the write is formed as
// (decayed row . qn) + u_v (kn . qn) so that one reduction pass suffices.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

// The two 4-channel pieces of lane j's 8 key channels for a state of type S.
template <typename S> __device__ __forceinline__ int piece0(int j) {
  return std::is_same<S, bf16>::value ? 8 * j : 4 * j;
}
template <typename S> __device__ __forceinline__ int piece1(int j) {
  return std::is_same<S, bf16>::value ? 8 * j + 4 : 64 + 4 * j;
}

// This lane's 8 values of a V-first state row (key channels piece0.., piece1..):
// fp32, or bf16 widened on load and rounded (to nearest even) on store.
__device__ __forceinline__ void row_load(const float* row, int j, float4 (&h)[2]) {
  h[0] = reinterpret_cast<const float4*>(row)[j];
  h[1] = reinterpret_cast<const float4*>(row)[16 + j];
}
__device__ __forceinline__ float4 widen4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void row_load(const bf16* row, int j, float4 (&h)[2]) {
  const uint4 u = reinterpret_cast<const uint4*>(row)[j];  // channels 8j .. 8j + 7
  h[0] = widen4(make_uint2(u.x, u.y));
  h[1] = widen4(make_uint2(u.z, u.w));
}
// The state is written back with nontemporal stores: the rows are not read
// again soon, and decode steps run back to back stream the pool faster when
// the written lines do not linger in the caches (256 x 32 fp32 rows:
// 0.215 -> 0.169 ms per back-to-back step).
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
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
  const uint2 a = narrow4(h[0]), b = narrow4(h[1]);
  __builtin_nontemporal_store(u32x4_nt{a.x, a.y, b.x, b.y},
                              reinterpret_cast<u32x4_nt*>(row) + j);
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
// This lane's 8 channels of a 128-vector, split as the state S's rows are.
template <typename S, typename T>
__device__ __forceinline__ void lane8(const T* p, int j, float (&x)[8]) {
  load4(p + piece0<S>(j), x);
  load4(p + piece1<S>(j), x + 4);
}
// One token's q, k and per-channel decay factor exp(g) on this lane's 8
// channels.  All loads are issued before the gate arithmetic so that they
// stay vector loads in one block.
template <typename S, typename T>
__device__ __forceinline__ void token_qk_decay(const T* qp, const T* kp, const T* gp, int j,
                                               int h, const GateArgs& ga, float ga_a,
                                               float (&qv)[8], float (&kv)[8],
                                               float (&al)[8]) {
  float gl[8];
  lane8<S>(qp, j, qv);
  lane8<S>(kp, j, kv);
  lane8<S>(gp, j, gl);
  if (ga.a_log) {
    float bias[8];
    if (ga.bias_bf16) {
      lane8<S>(reinterpret_cast<const bf16*>(ga.bias) + (size_t)h * D, j, bias);
    } else {
      lane8<S>(reinterpret_cast<const float*>(ga.bias) + (size_t)h * D, j, bias);
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
  token_qk_decay<S>(qp, kp, gp, j, h, ga, ga_a, qv, kv, al);
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
// The raw bits of one token's inputs on this lane (q, k, g: 8 channels each;
// the lane's 8 v rows; beta), so that the next token can be fetched before this
// token's state stores: the memory counter completes operations in issue
// order, and a fetch issued after the stores would wait for them.
template <typename T> struct Raw4 { using U = uint2; };
template <> struct Raw4<float> { using U = float4; };
template <typename T>
__device__ __forceinline__ typename Raw4<T>::U raw4(const T* p) {
  return *reinterpret_cast<const typename Raw4<T>::U*>(p);
}
__device__ __forceinline__ void unraw4(const float4& a, const float*, float* x) {
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void unraw4(const uint2& u, const bf16*, float* x) {
  const float4 a = widen4(u);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void unraw4(const uint2& u, const _Float16*, float* x) {
  x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x & 0xffffu));
  x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x >> 16));
  x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y & 0xffffu));
  x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y >> 16));
}
template <typename T> struct TokRaw {
  typename Raw4<T>::U q0, q1, k0, k1, g0, g1;
  T v[8];
  T b;
};

// The multi-token decode's per-request context.
template <typename T, typename S> struct MultiCtx {
  const T *q, *k, *v, *g, *beta;
  S* cache;
  const int32_t* ir;  // this request's row of state_indices
  T* out;
  int ntok, hv, hq, h, req, num_slots;
  float scale, ga_a;
  int use_l2;
  InStrides is;
  int64_t slot_stride;
  GateArgs ga;
};

template <typename T, typename S>
__device__ __forceinline__ void tok_fetch(const MultiCtx<T, S>& c, int t, int j, int wave,
                                          int rsub, TokRaw<T>& r) {
  const size_t tok = (size_t)c.req * c.ntok + t;
  const T* qp = c.q + tok * c.is.q + c.hq * D;
  const T* kp = c.k + tok * c.is.k + c.hq * D;
  const T* gp = c.g + tok * c.is.g + c.h * D;
  const T* vp = c.v + tok * c.is.v + c.h * D;
  r.q0 = raw4(qp + piece0<S>(j));
  r.q1 = raw4(qp + piece1<S>(j));
  r.k0 = raw4(kp + piece0<S>(j));
  r.k1 = raw4(kp + piece1<S>(j));
  r.g0 = raw4(gp + piece0<S>(j));
  r.g1 = raw4(gp + piece1<S>(j));
#pragma unroll
  for (int s = 0; s < 8; ++s) r.v[s] = vp[16 * s + 4 * wave + rsub];
  r.b = c.beta[tok * c.is.beta + c.h];
}

// Token t: decay, delta write and read-out on the state rows in hs; its
// inputs are in cur, and the next token's are fetched into nxt first (the
// last token fetches its own again: in bounds, unused).  ALL: every stored
// row is valid, so the stores need no branch.
template <typename T, typename S, bool GATE, bool ALL>
__device__ __forceinline__ void multi_token_step(const MultiCtx<T, S>& c, int t, int j, int wave,
                                                 int rsub, const float (&bias)[8],
                                                 float4 (&hs)[8][2], TokRaw<T>& nxt) {
  const TokRaw<T> cur = nxt;
  tok_fetch(c, min(t + 1, c.ntok - 1), j, wave, rsub, nxt);
  float qv[8], kv[8], gl[8], vr[8], al[8];
  unraw4(cur.q0, (const T*)nullptr, qv);
  unraw4(cur.q1, (const T*)nullptr, qv + 4);
  unraw4(cur.k0, (const T*)nullptr, kv);
  unraw4(cur.k1, (const T*)nullptr, kv + 4);
  unraw4(cur.g0, (const T*)nullptr, gl);
  unraw4(cur.g1, (const T*)nullptr, gl + 4);
#pragma unroll
  for (int s = 0; s < 8; ++s) vr[s] = to_f32(cur.v[s]);
  if constexpr (GATE) {
#pragma unroll
    for (int e = 0; e < 8; ++e) gl[e] = gate_apply(gl[e], c.ga_a, bias[e], c.ga.lower_bound);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) al[e] = exp2_fast(gl[e] * LOG2E);
  const float b = sigmoid(to_f32(cur.b));
  if (c.use_l2) {
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
  const int rt = c.ir[t];
  S* dst = (ALL || (rt >= 0 && rt < c.num_slots))
               ? c.cache + (size_t)rt * c.slot_stride + (size_t)c.h * (D * D)
               : nullptr;
  float ov[8];
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
    if (ALL)
      row_store(dst + r * D, j, hs[s]);
    else if (dst)
      row_store(dst + r * D, j, hs[s]);
    ov[s] = c.scale * (pq + u * kq);
  }
  // Outputs: every lane of a 16-lane row group holds the values of the group's
  // 8 rows; lanes j and j + 8 both write row s = j & 7 (the same value), so
  // the store needs no branch either.
  const int so = j & 7;
  float val = ov[0];
#pragma unroll
  for (int s = 1; s < 8; ++s) val = so == s ? ov[s] : val;
  T* o = c.out + (((size_t)c.req * c.ntok + t) * c.hv + c.h) * D;
  o[16 * so + 4 * wave + rsub] = from_f32<T>(val);
}

template <typename T, typename S, bool GATE, bool ALL>
__device__ __forceinline__ void multi_tokens(const MultiCtx<T, S>& c, int j, int wave, int rsub,
                                             const float (&bias)[8], float4 (&hs)[8][2],
                                             TokRaw<T>& nxt) {
  // token 0 peeled: inside the loop every iteration then starts with the same
  // operations in flight (the next token's fetch, then the previous token's
  // stores), and the compiler's wait for the fetch leaves the stores alone
  multi_token_step<T, S, GATE, ALL>(c, 0, j, wave, rsub, bias, hs, nxt);
  for (int t = 1; t < c.ntok; ++t) multi_token_step<T, S, GATE, ALL>(c, t, j, wave, rsub, bias, hs, nxt);
}

template <typename T, typename S, bool GATE>
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
  MultiCtx<T, S> c{q, k, v, g, beta, cache, ir, out, ntok, hv, hq, h, req, num_slots,
                   scale, 0.f, use_l2, is, slot_stride, ga};
  float bias[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (GATE) {
    c.ga_a = exp2_fast(ga.a_log[h] * LOG2E);  // exp(A_log[h])
    if (ga.bias_bf16)
      lane8<S>(reinterpret_cast<const bf16*>(ga.bias) + (size_t)h * D, j, bias);
    else
      lane8<S>(reinterpret_cast<const float*>(ga.bias) + (size_t)h * D, j, bias);
  }
  bool all = true;  // every state the request stores lands in the pool
  for (int t = 0; t < ntok; ++t) {
    const int rt = ir[t];
    all = all && rt >= 0 && rt < num_slots;
  }
  const S* st0 = cache + (size_t)row0 * slot_stride + (size_t)h * (D * D);
  float4 hs[8][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) row_load(st0 + (16 * s + 4 * wave + rsub) * D, j, hs[s]);
  TokRaw<T> nxt;
  tok_fetch(c, 0, j, wave, rsub, nxt);
  if (all)
    multi_tokens<T, S, GATE, true>(c, j, wave, rsub, bias, hs, nxt);
  else
    multi_tokens<T, S, GATE, false>(c, j, wave, rsub, bias, hs, nxt);
}

template <typename T, typename S>
static hipError_t launch_decode_t(const DecodeLaunch& L) {
  const dim3 grid((unsigned)((size_t)L.n * L.hv)), block(256);
  if (L.tokens > 1 || L.cols > 0) {
    auto mk = L.gate.a_log ? decode_multi_kernel<T, S, true> : decode_multi_kernel<T, S, false>;
    hipLaunchKernelGGL(mk, grid, block, 0, (hipStream_t)L.stream,
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
