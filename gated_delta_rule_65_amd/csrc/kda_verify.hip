// Record-based speculative verify, and the commit that rebuilds the accepted
// state from the records (KdaTcVerify, page
// "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify").
//
// verify_kernel, one 256-thread workgroup per (request, value head) with a
// window of n <= 8 tokens:
//   * the slot's state S0 is loaded once into registers (16 lanes per V-first
//     row, 8 key channels per lane: the decode kernel's split) and never
//     written back;
//   * token t's raw key and gate are copied to the kg record as they arrive;
//     its log-decay, normalised query and key go to LDS;
//   * the cumulative log-decay over the window gives the probes
//     p_t = e^cum kn, r_t = scale e^cum qn and the weights w_t = e^-cum kn
//     (|cum| <= 40 for step log-decays in [-5, 0], inside fp32);
//   * the couplings w_i . p_t, w_i . r_t (i <= t) are 128-dots reduced over a
//     16-lane row, and the projections S0^T p_t, S0^T r_t of every row are a
//     butterfly reduce-scatter over the row's 16 lanes (see project()): 8
//     probes for windows of up to 4 tokens, 16 for up to 8;
//   * thread r < 128 then runs the window's tiny triangular solve for value
//     row r and writes o_t[r] and the correction u_t[r].
// HBM per (request, head): the 64 KiB state read once, n tokens of input,
// out, and n x 1 KiB of records (fp32 corrections, raw key and gate) --
// against n further 64 KiB state writes when every token's state is stored.
//
// commit_kernel, one workgroup per (request, value head) with a = accepted
// count: S <- diag(e^g_t) S + kn_t u_t^T for t < a on the register-resident
// state rows, with kn_t and g_t recomputed from the kg record, then the rows
// are stored in place.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

constexpr int QMAX = 8;  // window tokens at most (the commit's record rows)

// This lane's two 4-channel pieces of a 128-vector, split as the state rows
// are: fp32 state {4j..4j+3} and {64+4j..}, so that a 16-lane row reads 256
// contiguous bytes per piece; bf16 state {8j..8j+7}, one 16-byte access.
template <typename S> __device__ __forceinline__ int chan0(int j) {
  return std::is_same<S, bf16>::value ? 8 * j : 4 * j;
}
template <typename S> __device__ __forceinline__ int chan1(int j) {
  return std::is_same<S, bf16>::value ? 8 * j + 4 : 64 + 4 * j;
}

// Four consecutive elements as stored (bits), and widened to fp32.
template <typename T> struct Bits4 { using U = uint2; };
template <> struct Bits4<float> { using U = float4; };
template <typename T>
__device__ __forceinline__ typename Bits4<T>::U ld4(const T* p) {
  return *reinterpret_cast<const typename Bits4<T>::U*>(p);
}
template <typename T>
__device__ __forceinline__ void st4(T* p, const typename Bits4<T>::U& x) {
  *reinterpret_cast<typename Bits4<T>::U*>(p) = x;
}
template <typename T>
__device__ __forceinline__ void widen4(const typename Bits4<T>::U& u, float* x) {
  if constexpr (std::is_same<T, float>::value) {
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  } else if constexpr (std::is_same<T, bf16>::value) {
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    x[0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x & 0xffffu));
    x[1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.x >> 16));
    x[2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y & 0xffffu));
    x[3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u.y >> 16));
  }
}

// This lane's 8 channels of a V-first state row, widened to fp32.
template <typename S>
__device__ __forceinline__ void state_load(const S* row, int j, float (&x)[8]) {
  if constexpr (std::is_same<S, float>::value) {
    const float4 a = reinterpret_cast<const float4*>(row)[j];
    const float4 b = reinterpret_cast<const float4*>(row)[16 + j];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 u = reinterpret_cast<const uint4*>(row)[j];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x[2 * d] = __uint_as_float(w[d] << 16);
      x[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
    }
  }
}
// ... and stored back (bf16: rounded to nearest even), nontemporal: the slot
// is not read again soon.
typedef float f32x4_v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
template <typename S>
__device__ __forceinline__ void state_store(S* row, int j, const float (&x)[8]) {
  if constexpr (std::is_same<S, float>::value) {
    f32x4_v* p = reinterpret_cast<f32x4_v*>(row);
    __builtin_nontemporal_store(f32x4_v{x[0], x[1], x[2], x[3]}, p + j);
    __builtin_nontemporal_store(f32x4_v{x[4], x[5], x[6], x[7]}, p + 16 + j);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
      w[d] = (uint32_t)bf16_bits(x[2 * d]) | ((uint32_t)bf16_bits(x[2 * d + 1]) << 16);
    __builtin_nontemporal_store(u32x4_v{w[0], w[1], w[2], w[3]},
                                reinterpret_cast<u32x4_v*>(row) + j);
  }
}

// 8 fp32 values of LDS row `v` at this lane's channels.
__device__ __forceinline__ void lds8(const float* v, int c0, int c1, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(v + c0);
  const float4 b = *reinterpret_cast<const float4*>(v + c1);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void lds8_put(float* v, int c0, int c1, const float (&x)[8]) {
  *reinterpret_cast<float4*>(v + c0) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(v + c1) = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ float dot8(const float (&a)[8], const float (&b)[8]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(a[e], b[e], s);
  return s;
}

// Gate biases of this lane's 8 channels.
__device__ __forceinline__ void bias8(const GateArgs& ga, int h, int c0, int c1, float (&b)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    b[e] = gate_bias(ga, h, c0 + e);
    b[4 + e] = gate_bias(ga, h, c1 + e);
  }
}

// LDS of one verify workgroup for windows of at most QH = NP / 2 tokens.
template <int NP> struct VerifyShared {
  static constexpr int QH = NP / 2;
  float lg[QH][D];              // step log-decay of token t
  float qn[QH][D];              // normalised query (0 past the window's tokens)
  float kn[QH][D];              // normalised key
  float probe[NP][D];           // p_t, then r_t
  float w[QH][D];               // w_t
  float cpl[2][QH][QH];         // [0][t][i] = w_i . p_t (i < t), [1][t][i] = w_i . r_t (i <= t)
  float proj[D][NP + 1];        // [value row][probe]: S0^T p_t, S0^T r_t
  float b[QH];                  // sigmoid(beta_t)
};

// Projections of this lane's 8 state rows on the NP probes, reduce-scattered
// over the row's 16 lanes (DPP), written to proj[row][probe].
//
// Step one pairs lane j with 15 - j (row_mirror, j ^ 15): the lane keeps the
// half of the probes with base (NP/2) bit3(j) and sends the other half; steps
// two and three pair j with j ^ 7 (row_half_mirror) and j ^ 3 (quad
// permutation), and for NP = 16 step four with j ^ 1 (for NP = 8 the two
// lanes j, j ^ 1 add their sums instead and both hold the total).  Slot m of a
// lane holds the probe of local index m ^ c(j), where c(j) is chosen so that at
// every step the lane's kept slots are the low half and the partner's matching
// sums arrive in the high half, in the same order: for NP = 16,
// c = 4 b2 + 2 (b1 ^ b2) + (b0 ^ b1); for NP = 8, c = 2 b2 + (b1 ^ b2) (b_k
// the bits of j).  So no step needs a per-lane selection, and the lane ends
// with probe (NP/2) b3 + c(j).  Each state element is multiplied once per
// probe and no sum is reduced twice.
template <int NP>
__device__ __forceinline__ void project(const float (&x)[8][8], const float (&pr)[NP][D], int j,
                                        int c0, int c1, int row0, float (&proj)[D][NP + 1]) {
  constexpr int H = NP / 2;
  const int b0 = j & 1, b1 = (j >> 1) & 1, b2 = (j >> 2) & 1, b3 = (j >> 3) & 1;
  const int c = NP == 16 ? 4 * b2 + 2 * (b1 ^ b2) + (b0 ^ b1) : 2 * b2 + (b1 ^ b2);
  const int keep0 = H * b3, send0 = H * (1 - b3), flip = H / 2;
  float a1[8][H];
#pragma unroll
  for (int m = 0; m < H; ++m) {
    float pk[8], ps[8];
    lds8(pr[keep0 + (m ^ c)], c0, c1, pk);
    lds8(pr[send0 + (m ^ c ^ flip)], c0, c1, ps);
#pragma unroll
    for (int s = 0; s < 8; ++s) a1[s][m] = dot8(x[s], pk) + dpp_mov<0x140>(dot8(x[s], ps));
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float v;
    if constexpr (NP == 16) {
      float a2[4], a3[2];
#pragma unroll
      for (int y = 0; y < 4; ++y) a2[y] = a1[s][y] + dpp_mov<0x141>(a1[s][4 + y]);
#pragma unroll
      for (int y = 0; y < 2; ++y) a3[y] = a2[y] + dpp_mov<0x1B>(a2[2 + y]);
      v = a3[0] + dpp_mov<0xB1>(a3[1]);
    } else {
      float a2[2];
#pragma unroll
      for (int y = 0; y < 2; ++y) a2[y] = a1[s][y] + dpp_mov<0x141>(a1[s][2 + y]);
      v = a2[0] + dpp_mov<0x1B>(a2[1]);
      v += dpp_mov<0xB1>(v);
    }
    if (NP == 16 || b0 == 0) proj[row0 + 16 * s][keep0 + c] = v;
  }
}

template <typename T, typename S, bool GATE, int NP>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyLaunch L) {
  constexpr int QH = NP / 2;
  constexpr int NPAIR = QH * (QH + 1) / 2;  // (t, i), i <= t
  __shared__ VerifyShared<NP> sh;
  const int unit = blockIdx.x;
  const int req = unit / L.hv, h = unit - req * L.hv;
  const int hq = h / (L.hv / L.hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, rsub = lane >> 4, grp = 4 * wave + rsub;
  const int bos = L.query_start[req];
  const int n = min(max(L.query_start[req + 1] - bos, 0), L.window);
  if (n == 0) return;
  T* out = reinterpret_cast<T*>(L.out);
  const int slot = L.idx[req];
  if (slot < 0 || slot >= L.num_slots) {
    if (tid < D)
      for (int t = 0; t < n; ++t) out[((size_t)(bos + t) * L.hv + h) * D + tid] = from_f32<T>(0.f);
    return;
  }
  const int c0 = chan0<S>(j), c1 = chan1<S>(j);
  const int row0 = 4 * wave + rsub;   // this lane's state rows: row0 + 16 s

  // Loads in the order they are consumed (a wait for an early load leaves the
  // later ones in flight): token t = grp's q, k, g and beta (waves 0 and 1),
  // the solver's v (thread r < 128 owns value row r), then the state.
  const int t = grp;
  const bool tok = t < QH && t < n;
  const size_t trow = (size_t)(bos + min(t, n - 1));
  const T* qp = reinterpret_cast<const T*>(L.q) + trow * L.strides.q + hq * D;
  const T* kp = reinterpret_cast<const T*>(L.k) + trow * L.strides.k + hq * D;
  const T* gp = reinterpret_cast<const T*>(L.g) + trow * L.strides.g + h * D;
  typename Bits4<T>::U q0{}, q1{}, k0{}, k1{}, g0{}, g1{};
  float bl = 0.f;
  if (tok) {
    q0 = ld4(qp + c0); q1 = ld4(qp + c1);
    k0 = ld4(kp + c0); k1 = ld4(kp + c1);
    g0 = ld4(gp + c0); g1 = ld4(gp + c1);
    bl = to_f32(reinterpret_cast<const T*>(L.beta)[trow * L.strides.beta + h]);
  }
  const T* vv = reinterpret_cast<const T*>(L.v);
  float vr[QH];
#pragma unroll
  for (int i = 0; i < QH; ++i)
    vr[i] = (tid < D && i < n) ? to_f32(vv[(size_t)(bos + i) * L.strides.v + h * D + tid]) : 0.f;
  const S* st = reinterpret_cast<const S*>(L.cache) + (size_t)slot * L.slot_stride +
                (size_t)h * (D * D);
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) state_load(st + (size_t)(row0 + 16 * s) * D, j, x[s]);

  // Token t: records, log-decay, normalised q and k.
  if (t < QH) {
    float qv[8] = {}, kv[8] = {}, gl[8] = {};
    if (tok) {
      T* rec = reinterpret_cast<T*>(L.kg) + (((size_t)req * L.hv + h) * L.window + t) * (2 * D);
      st4<T>(rec + c0, k0);
      st4<T>(rec + c1, k1);
      st4<T>(rec + D + c0, g0);
      st4<T>(rec + D + c1, g1);
      widen4<T>(q0, qv); widen4<T>(q1, qv + 4);
      widen4<T>(k0, kv); widen4<T>(k1, kv + 4);
      widen4<T>(g0, gl); widen4<T>(g1, gl + 4);
      if constexpr (GATE) {
        float bias[8];
        bias8(L.gate, h, c0, c1, bias);
        const float a = exp2_fast(L.gate.a_log[h] * LOG2E);
#pragma unroll
        for (int e = 0; e < 8; ++e) gl[e] = gate_apply(gl[e], a, bias[e], L.gate.lower_bound);
      }
      if (L.use_l2) {
        const float rq = rsq(row_sum16(dot8(qv, qv)) + L2_EPS);
        const float rk = rsq(row_sum16(dot8(kv, kv)) + L2_EPS);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qv[e] *= rq;
          kv[e] *= rk;
        }
      }
    }
    if (j == 0) sh.b[t] = tok ? sigmoid(bl) : 0.f;
    lds8_put(sh.lg[t], c0, c1, gl);
    lds8_put(sh.qn[t], c0, c1, qv);
    lds8_put(sh.kn[t], c0, c1, kv);
  }
  lds_barrier();

  // Probes and weights of token t.
  if (t < QH) {
    float cum[8] = {}, y[8];
    for (int i = 0; i <= t; ++i) {
      lds8(sh.lg[i], c0, c1, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) cum[e] += y[e];
    }
    float qv[8], kv[8], p[8], r[8], w[8];
    lds8(sh.qn[t], c0, c1, qv);
    lds8(sh.kn[t], c0, c1, kv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float up = exp2_fast(cum[e] * LOG2E), dn = exp2_fast(-cum[e] * LOG2E);
      p[e] = up * kv[e];
      r[e] = L.scale * up * qv[e];
      w[e] = dn * kv[e];
    }
    lds8_put(sh.probe[t], c0, c1, p);
    lds8_put(sh.probe[QH + t], c0, c1, r);
    lds8_put(sh.w[t], c0, c1, w);
  }
  lds_barrier();

  // Couplings: pair m = t (t + 1) / 2 + i over the 16 row groups; each
  // 16-lane row reduces its own pairs (rows with no pair idle).
  for (int m = grp; m < NPAIR; m += 16) {
    int tt = 0;
    while ((tt + 1) * (tt + 2) / 2 <= m) ++tt;
    const int i = m - tt * (tt + 1) / 2;
    float w[8], p[8], r[8];
    lds8(sh.w[i], c0, c1, w);
    lds8(sh.probe[tt], c0, c1, p);
    lds8(sh.probe[QH + tt], c0, c1, r);
    const float cp = row_sum16(dot8(w, p));
    const float cr = row_sum16(dot8(w, r));
    if (j == 0) {
      sh.cpl[0][tt][i] = i < tt ? cp : 0.f;
      sh.cpl[1][tt][i] = cr;
    }
  }
  project<NP>(x, sh.probe, j, c0, c1, row0, sh.proj);
  lds_barrier();

  // Thread r < 128 solves value row r over the window.
  if (tid < D) {
    const int r = tid;
    float u[QH];
    float* corr = L.corr + ((size_t)req * L.hv + h) * L.window * D;
#pragma unroll
    for (int tt = 0; tt < QH; ++tt) {
      if (tt < n) {
        float acc = vr[tt] - sh.proj[r][tt];
#pragma unroll
        for (int i = 0; i < tt; ++i) acc = fmaf(-sh.cpl[0][tt][i], u[i], acc);
        u[tt] = sh.b[tt] * acc;
        float o = sh.proj[r][QH + tt];
#pragma unroll
        for (int i = 0; i <= tt; ++i) o = fmaf(sh.cpl[1][tt][i], u[i], o);
        out[((size_t)(bos + tt) * L.hv + h) * D + r] = from_f32<T>(o);
        corr[(size_t)tt * D + r] = u[tt];
      }
    }
  }
}

template <typename T, typename S, bool GATE>
__global__ __launch_bounds__(256) void commit_kernel(const CommitLaunch L) {
  __shared__ float su[QMAX][D];
  const int unit = blockIdx.x;
  const int req = unit / L.hv, h = unit - req * L.hv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, rsub = lane >> 4;
  const int slot = L.idx[req], a = L.accepted[req];
  if (slot < 0 || slot >= L.num_slots || a < 1 || a > L.window) return;
  const int c0 = chan0<S>(j), c1 = chan1<S>(j);
  S* st = reinterpret_cast<S*>(L.cache) + (size_t)slot * L.slot_stride + (size_t)h * (D * D);
  float x[8][8];
#pragma unroll
  for (int s = 0; s < 8; ++s) state_load(st + (size_t)(16 * s + 4 * wave + rsub) * D, j, x[s]);

  const size_t rec = ((size_t)req * L.hv + h) * L.window;
  const float* cp = L.corr + rec * D;
  for (int e = tid; e < a * D; e += 256) su[e >> 7][e & (D - 1)] = cp[e];
  float bias[8] = {}, ga = 0.f;
  if constexpr (GATE) {
    bias8(L.gate, h, c0, c1, bias);
    ga = exp2_fast(L.gate.a_log[h] * LOG2E);
  }
  lds_barrier();

  const T* kg = reinterpret_cast<const T*>(L.kg) + rec * (2 * D);
  for (int t = 0; t < a; ++t) {
    const T* kp = kg + (size_t)t * (2 * D);
    float kv[8], gl[8], al[8];
    widen4<T>(ld4(kp + c0), kv);
    widen4<T>(ld4(kp + c1), kv + 4);
    widen4<T>(ld4(kp + D + c0), gl);
    widen4<T>(ld4(kp + D + c1), gl + 4);
    if constexpr (GATE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gl[e] = gate_apply(gl[e], ga, bias[e], L.gate.lower_bound);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) al[e] = exp2_fast(gl[e] * LOG2E);
    if (L.use_l2) {
      const float rk = rsq(row_sum16(dot8(kv, kv)) + L2_EPS);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] *= rk;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float us = su[t][16 * s + 4 * wave + rsub];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[s][e] = fmaf(al[e], x[s][e], kv[e] * us);
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) state_store(st + (size_t)(16 * s + 4 * wave + rsub) * D, j, x[s]);
}

template <typename T, typename S, int NP>
hipError_t verify_np(const VerifyLaunch& L) {
  auto k = L.gate.a_log ? verify_kernel<T, S, true, NP> : verify_kernel<T, S, false, NP>;
  hipLaunchKernelGGL(k, dim3((unsigned)((size_t)L.n * L.hv)), dim3(256), 0,
                     (hipStream_t)L.stream, L);
  return hipGetLastError();
}
template <typename T, typename S>
hipError_t commit_t(const CommitLaunch& L) {
  auto k = L.gate.a_log ? commit_kernel<T, S, true> : commit_kernel<T, S, false>;
  hipLaunchKernelGGL(k, dim3((unsigned)((size_t)L.n * L.hv)), dim3(256), 0,
                     (hipStream_t)L.stream, L);
  return hipGetLastError();
}
// Windows of at most 4 tokens need 8 probes, longer ones 16.
template <typename T, typename S>
hipError_t verify_t(const VerifyLaunch& L) {
  return L.window <= 4 ? verify_np<T, S, 8>(L) : verify_np<T, S, 16>(L);
}
template <typename T>
hipError_t verify_s(const VerifyLaunch& L) {
  return L.state_bf16 ? verify_t<T, bf16>(L) : verify_t<T, float>(L);
}
template <typename T>
hipError_t commit_s(const CommitLaunch& L) {
  return L.state_bf16 ? commit_t<T, bf16>(L) : commit_t<T, float>(L);
}

}  // namespace

hipError_t launch_verify(const VerifyLaunch& L) {
  switch (L.dtype) {
    case 0: return verify_s<float>(L);
    case 1: return verify_s<bf16>(L);
    default: return verify_s<_Float16>(L);
  }
}

hipError_t launch_commit(const CommitLaunch& L) {
  switch (L.dtype) {
    case 0: return commit_s<float>(L);
    case 1: return commit_s<bf16>(L);
    default: return commit_s<_Float16>(L);
  }
}

}  // namespace kda
