// The staged KDA chunked forward on gfx950: chunk table -> prep -> WY -> walk.
//
// Chunked form (64-token chunks that restart at every sequence start; the
// last chunk of a sequence may be short).  Inside a chunk, with G the
// inclusive cumulative log2-decay per key channel (G = log2(e) * cumsum(g)):
//   qg = qn 2^G,  kg = kn 2^(G_last - G),  d = 2^G_last
//   A_kk[t][i] = b_t sum_c kn_t kn_i 2^(G_t - G_i)     (i < t)
//   A_qk[t][i] =     sum_c qn_t kn_i 2^(G_t - G_i)     (i <= t)
//   T = (I + A_kk)^-1,  w = T (b kn 2^G),  u = T (b v)
// and, with S the K x V state entering the chunk,
//   U = u - w S,  O = scale (qg S + A_qk U),  S <- diag(d) S + kg^T U.
// The operand set and its layouts (qg, kg_t, decay, w, u, aqk) follow the
// fused_kda_prologue / fused_kda_chunk description on page
// "vllm.models.kimi_k3.amd.ops.kda_chunk"; the chunk boundaries follow its
// chunk offsets/indices built from cu_seqlens.  Working in base 2 is only a
// change of base of the natural-log decay.
//
// Exponent range.  Per-step g lies in [-5, 0], so G spans up to 460 (log2
// units) across a chunk and 2^(-G_i) alone would overflow fp32.  The WY
// kernel therefore evaluates 2^(G_t - G_i) through a reference token m_a in
// the middle of each 16-token block a of the row index t:
//   2^(G_t - G_i) = 2^(G_t - G_ma) * 2^(G_ma - G_i)
// For i in an earlier block both factors are <= 1; inside block a both
// exponents stay within 8 steps (<= 58 in log2 units), which fp32 and bf16
// hold.  Products for i > t may be large but finite and are masked away.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"
#include "kda_mfma.hpp"

namespace kda {

// ---------------------------------------------------------------- chunk table

struct SeqSpan {
  int bos, eos;
};

// Token range of sequence n; device-side values are clamped into [0, T] so a
// malformed cu_seqlens can never address outside the inputs.
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int n, int dense_len, int T) {
  if (!cu) return {n * dense_len, (n + 1) * dense_len};
  int b = cu[n], e = cu[n + 1];
  b = min(max(b, 0), T);
  e = min(max(e, b), T);
  return {b, e};
}

// offs[n] = first chunk of sequence n; offs[N] = number of chunks.
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* cu, int N,
                                                             int dense_len, int T,
                                                             int32_t* offs) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int s0 = min(N, tid * per), s1 = min(N, s0 + per);
  int sum = 0;
  for (int n = s0; n < s1; ++n) {
    const SeqSpan s = seq_span(cu, n, dense_len, T);
    sum += (s.eos - s.bos + C - 1) / C;
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int n = s0; n < s1; ++n) {
    offs[n] = run;
    const SeqSpan s = seq_span(cu, n, dense_len, T);
    run += (s.eos - s.bos + C - 1) / C;
  }
  if (tid == 1023) offs[N] = part[1023];
}

struct ChunkPos {
  int n, t0, L;
};

// Chunk c -> (sequence, first token, length) by binary search of offs.
__device__ __forceinline__ bool locate_chunk(int c, const int32_t* offs, int N,
                                             const int32_t* cu, int dense_len, int T,
                                             ChunkPos& p) {
  if (c >= offs[N]) return false;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  const SeqSpan s = seq_span(cu, lo, dense_len, T);
  p.n = lo;
  p.t0 = s.bos + C * (c - offs[lo]);
  p.L = min(C, s.eos - p.t0);
  return p.L > 0;
}

// ------------------------------------------------------------ small helpers

__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  uint4 u;
  u.x = (uint32_t)bf16_bits(x[0]) | ((uint32_t)bf16_bits(x[1]) << 16);
  u.y = (uint32_t)bf16_bits(x[2]) | ((uint32_t)bf16_bits(x[3]) << 16);
  u.z = (uint32_t)bf16_bits(x[4]) | ((uint32_t)bf16_bits(x[5]) << 16);
  u.w = (uint32_t)bf16_bits(x[6]) | ((uint32_t)bf16_bits(x[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// A 64 x 128 token tile of q and k (L2-normalised when asked) into fp32 LDS.
// Thread mapping: 16 lanes (one DPP row) per token row, 8 channels per lane;
// all four row loads are issued before the first reduction.
template <typename E>
__device__ __forceinline__ void load_rows4(const E* src, int stride_t, int L, float (&x)[4][8]) {
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = rg + 16 * it;
    if (t < L) {
      load8(src + (size_t)t * stride_t + 8 * j, x[it]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[it][e] = 0.f;
    }
  }
}

__device__ __forceinline__ void l2norm_rows4(float (&x)[4][8]) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[it][e] * x[it][e];
    s = row_sum16(s);
    const float r = rsqrtf(s + L2_EPS);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[it][e] *= r;
  }
}

template <int SK>
__device__ __forceinline__ void rows4_to_lds(const float (&x)[4][8], float (*dst)[SK]) {
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = rg + 16 * it;
    *reinterpret_cast<float4*>(&dst[t][8 * j]) =
        make_float4(x[it][0], x[it][1], x[it][2], x[it][3]);
    *reinterpret_cast<float4*>(&dst[t][8 * j + 4]) =
        make_float4(x[it][4], x[it][5], x[it][6], x[it][7]);
  }
}

// g rows (already in registers, x log2 e applied here) into LDS, then the
// inclusive cumulative sum over tokens per channel.  Rows past L hold g = 0,
// so G stays at G_{L-1} there.
template <int SK>
__device__ __forceinline__ void gate_cumsum(const float (&x)[4][8], float (*sG)[SK]) {
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = rg + 16 * it;
#pragma unroll
    for (int e = 0; e < 8; ++e) sG[t][8 * j + e] = x[it][e] * LOG2E;
  }
  __syncthreads();
  const int c = tid & 127, half = tid >> 7;  // 256 threads: two halves of 32 tokens
  float run = 0.f;
#pragma unroll 8
  for (int tt = 0; tt < 32; ++tt) {
    run += sG[32 * half + tt][c];
    sG[32 * half + tt][c] = run;
  }
  __syncthreads();
  if (half == 1) {
    const float base = sG[31][c];
#pragma unroll 8
    for (int tt = 0; tt < 32; ++tt) sG[32 + tt][c] += base;
  }
  __syncthreads();
}

// ----------------------------------------------------------------------- prep

// One workgroup per (chunk, query/key head); loops over the value heads of the
// GVA group.  Streaming: reads q, k, g once, writes qg, kg_t, decay.
template <typename E>
__global__ __launch_bounds__(256) void prep_kernel(const E* __restrict__ q,
                                                   const E* __restrict__ k,
                                                   const E* __restrict__ g,
                                                   const int32_t* __restrict__ cu,
                                                   int dense_len, int T,
                                                   const int32_t* __restrict__ offs, int N,
                                                   int hqk, int hv, int use_l2,
                                                   E* __restrict__ qg, E* __restrict__ kg_t,
                                                   float* __restrict__ decay) {
  constexpr int SK = D + 4;
  __shared__ float sK[C][SK];
  __shared__ float sG[C][SK];
  ChunkPos p;
  if (!locate_chunk(blockIdx.x, offs, N, cu, dense_len, T, p)) return;
  const int c = blockIdx.x, hq = blockIdx.y, grp = hv / hqk;
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
  const int L = p.L;

  // q rows stay in registers, k rows go to LDS (kg is written transposed);
  // the first head's g rows are fetched together with q and k.
  float qn[4][8], kx[4][8], gx[4][8];
  load_rows4(q + ((size_t)p.t0 * hqk + hq) * D, hqk * D, L, qn);
  load_rows4(k + ((size_t)p.t0 * hqk + hq) * D, hqk * D, L, kx);
  load_rows4(g + ((size_t)p.t0 * hv + hq * grp) * D, hv * D, L, gx);
  if (use_l2) {
    l2norm_rows4(qn);
    l2norm_rows4(kx);
  }
  rows4_to_lds<SK>(kx, sK);

  for (int gi = 0; gi < grp; ++gi) {
    const int h = hq * grp + gi;
    if (gi > 0) {
      __syncthreads();
      load_rows4(g + ((size_t)p.t0 * hv + h) * D, hv * D, L, gx);
    }
    gate_cumsum<SK>(gx, sG);
    // qg = qn 2^G, token-major
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = rg + 16 * it;
      if (t < L) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qn[it][e] * exp2_fast(sG[t][8 * j + e]);
        store8(qg + ((size_t)(p.t0 + t) * hv + h) * D + 8 * j, x);
      }
    }
    // kg_t[c][h][kk][t] = kn_t[kk] 2^(G_last - G_t), zero past L
    {
      const int kk = tid >> 1, th = (tid & 1) * 32;
      const float glast = sG[L - 1][kk];
      E* dst = kg_t + (((size_t)c * hv + h) * D + kk) * C + th;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = th + 8 * blk + e;
          x[e] = (t < L) ? sK[t][kk] * exp2_fast(glast - sG[t][kk]) : 0.f;
        }
        store8(dst + 8 * blk, x);
      }
    }
    if (tid < D) decay[((size_t)c * hv + h) * D + tid] = exp2_fast(sG[L - 1][tid]);
  }
}

// ------------------------------------------------------------------------- WY

// (row block a, column block b) pairs of the lower 64x64 couplings per wave,
// and the strictly upper blocks of A_qk each wave writes as zeros.
__constant__ int8_t kWyPairs[4][3][2] = {{{3, 3}, {3, 2}, {3, 1}},
                                         {{3, 0}, {2, 2}, {2, 1}},
                                         {{2, 0}, {1, 1}, {-1, -1}},
                                         {{1, 0}, {0, 0}, {-1, -1}}};
__constant__ int8_t kWyZero[4][3][2] = {{{-1, -1}, {-1, -1}, {-1, -1}},
                                        {{-1, -1}, {-1, -1}, {-1, -1}},
                                        {{0, 1}, {0, 2}, {0, 3}},
                                        {{1, 2}, {1, 3}, {2, 3}}};

// X = sum_{c in [b, a)} A_ac T_cb into scratch (one 16x16 block per wave).
template <int SA>
__device__ __forceinline__ void wy_offdiag_x(int a, int b, const float (*sA)[SA],
                                             const float (*sT)[SA], float (*sX)[17],
                                             int lane) {
  const int col = lane & 15, rq = lane >> 4;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * rq + rr;
    float acc = 0.f;
    for (int cb = b; cb < a; ++cb) {
#pragma unroll
      for (int m = 0; m < 16; ++m) acc += sA[16 * a + row][16 * cb + m] * sT[16 * cb + m][16 * b + col];
    }
    sX[row][col] = acc;
  }
}

// T_ab = -T_aa X.
template <int SA>
__device__ __forceinline__ void wy_offdiag_t(int a, int b, float (*sT)[SA],
                                             const float (*sX)[17], int lane) {
  const int col = lane & 15, rq = lane >> 4;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * rq + rr;
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) acc += sT[16 * a + row][16 * a + m] * sX[m][col];
    sT[16 * a + row][16 * b + col] = -acc;
  }
}

// One workgroup (4 waves) per (chunk, value head): couplings on MFMA, the
// unit-lower inverse by blocked forward substitution in LDS (fp32), then
// w = T (b kn 2^G) and u = T (b v) on MFMA.
template <typename E>
__global__ __launch_bounds__(256) void wy_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ g, const E* __restrict__ beta, const int32_t* __restrict__ cu,
    int dense_len, int T, const int32_t* __restrict__ offs, int N, int hqk, int hv,
    int use_l2, E* __restrict__ w_out, E* __restrict__ u_out, E* __restrict__ aqk) {
  constexpr bool SPLIT = std::is_same<E, float>::value;
  constexpr int SK = D + 4;
  constexpr int SA = C + 4;
  __shared__ float sQ[C][SK];  // q, later v
  __shared__ float sK[C][SK];
  __shared__ float sG[C][SK];
  __shared__ float sA[C][SA];
  __shared__ float sT[C][SA];
  __shared__ float sB[C];
  __shared__ float sX[4][16][17];

  ChunkPos p;
  if (!locate_chunk(blockIdx.x, offs, N, cu, dense_len, T, p)) return;
  const int h = blockIdx.y, hq = h / (hv / hqk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int L = p.L;

  {
    float qx[4][8], kx[4][8], gx[4][8];
    load_rows4(q + ((size_t)p.t0 * hqk + hq) * D, hqk * D, L, qx);
    load_rows4(k + ((size_t)p.t0 * hqk + hq) * D, hqk * D, L, kx);
    load_rows4(g + ((size_t)p.t0 * hv + h) * D, hv * D, L, gx);
    const float braw = (tid < L) ? to_f32(beta[(size_t)(p.t0 + tid) * hv + h]) : 0.f;
    if (use_l2) {
      l2norm_rows4(qx);
      l2norm_rows4(kx);
    }
    rows4_to_lds<SK>(qx, sQ);
    rows4_to_lds<SK>(kx, sK);
    if (tid < C) sB[tid] = (tid < L) ? sigmoid(braw) : 0.f;
    gate_cumsum<SK>(gx, sG);
  }

  // ---- couplings A_kk (to LDS) and A_qk (to memory), transposed tiles:
  //      rows i (A operand R), columns t (B operand L).
  {
    int cur_a = -1;
    Frag<SPLIT> Lk[4], Lq[4];
    for (int pi = 0; pi < 3; ++pi) {
      const int a = kWyPairs[wave][pi][0], b = kWyPairs[wave][pi][1];
      if (a < 0) break;
      const int ma = 16 * a + 7;
      if (a != cur_a) {
        cur_a = a;
        const int t = 16 * a + l16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float lk[8], lq[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int c = 32 * s + 8 * gq + jj;
            const float e = exp2_fast(sG[t][c] - sG[ma][c]);
            lk[jj] = sK[t][c] * e;
            lq[jj] = sQ[t][c] * e;
          }
          Lk[s] = make_frag<SPLIT>(lk);
          Lq[s] = make_frag<SPLIT>(lq);
        }
      }
      f32x4_t acck = {0.f, 0.f, 0.f, 0.f}, accq = {0.f, 0.f, 0.f, 0.f};
      const int i = 16 * b + l16;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float r[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 32 * s + 8 * gq + jj;
          r[jj] = sK[i][c] * exp2_fast(sG[ma][c] - sG[i][c]);
        }
        const Frag<SPLIT> R = make_frag<SPLIT>(r);
        mma(acck, R, Lk[s]);
        mma(accq, R, Lq[s]);
      }
      const int t = 16 * a + l16;
      const int i0 = 16 * b + 4 * gq;
      float ak[4], aq[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ak[r] = (i0 + r < t) ? acck[r] * sB[t] : 0.f;
        aq[r] = (i0 + r <= t) ? accq[r] : 0.f;
      }
      store4(&sA[t][i0], ak[0], ak[1], ak[2], ak[3]);
      if (t < L) store4(aqk + ((size_t)(p.t0 + t) * hv + h) * C + i0, aq[0], aq[1], aq[2], aq[3]);
    }
#pragma unroll
    for (int zi = 0; zi < 3; ++zi) {
      const int a = kWyZero[wave][zi][0], b = kWyZero[wave][zi][1];
      if (a < 0) break;
      const int t = 16 * a + l16;
      if (t < L) store4(aqk + ((size_t)(p.t0 + t) * hv + h) * C + 16 * b + 4 * gq, 0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();

  float vx[4][8];
  load_rows4(v + ((size_t)p.t0 * hv + h) * D, hv * D, L, vx);

  // ---- T = (I + A_kk)^-1: diagonal 16x16 blocks by substitution (one wave
  //      each, one lane per column), then the off-diagonal blocks by levels.
  if (lane < 16) {
    const int a = wave;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float val = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int ii = 0; ii < r; ++ii) val -= sA[16 * a + r][16 * a + ii] * x[ii];
      x[r] = val;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[16 * a + r][16 * a + lane] = x[r];
  }
  for (int idx = tid; idx < C * C; idx += 256) {
    const int t = idx >> 6, i = idx & 63;
    if ((i >> 4) > (t >> 4)) sT[t][i] = 0.f;
  }
  __syncthreads();
  if (wave < 3) wy_offdiag_x<SA>(wave + 1, wave, sA, sT, sX[wave], lane);
  __syncthreads();
  if (wave < 3) wy_offdiag_t<SA>(wave + 1, wave, sT, sX[wave], lane);
  __syncthreads();
  if (wave < 2) wy_offdiag_x<SA>(wave + 2, wave, sA, sT, sX[wave], lane);
  __syncthreads();
  if (wave < 2) wy_offdiag_t<SA>(wave + 2, wave, sT, sX[wave], lane);
  __syncthreads();
  if (wave == 0) wy_offdiag_x<SA>(3, 0, sA, sT, sX[0], lane);
  __syncthreads();
  if (wave == 0) wy_offdiag_t<SA>(3, 0, sT, sX[0], lane);

  // ---- v into the q slot (q is no longer needed; its loads were issued
  //      before the inversion)
  rows4_to_lds<SK>(vx, sQ);
  __syncthreads();

  // ---- w^T = (b kn 2^G)^T T^T and u^T = (b v)^T T^T: rows c (A operand),
  //      columns t (B operand = T^T), K = i; T is lower, so tiles of t < 32
  //      need only i < 32.
  {
    Frag<SPLIT> Tf[4][2];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && ta < 2) continue;
        const int t = 16 * ta + l16;
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = sT[t][32 * s + 8 * gq + jj];
        Tf[ta][s] = make_frag<SPLIT>(x);
      }
    }
#pragma unroll
    for (int cbi = 0; cbi < 2; ++cbi) {
      const int cb = 2 * wave + cbi;
      const int c = 16 * cb + l16;
      Frag<SPLIT> Yk[2], Yv[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float yk[8], yv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int i = 32 * s + 8 * gq + jj;
          const float bi = sB[i];
          yk[jj] = bi * sK[i][c] * exp2_fast(sG[i][c]);
          yv[jj] = bi * sQ[i][c];
        }
        Yk[s] = make_frag<SPLIT>(yk);
        Yv[s] = make_frag<SPLIT>(yv);
      }
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        f32x4_t aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
        mma(aw, Yk[0], Tf[ta][0]);
        mma(au, Yv[0], Tf[ta][0]);
        if (ta >= 2) {
          mma(aw, Yk[1], Tf[ta][1]);
          mma(au, Yv[1], Tf[ta][1]);
        }
        const int t = 16 * ta + l16;
        if (t < L) {
          const size_t o = ((size_t)(p.t0 + t) * hv + h) * D + 16 * cb + 4 * gq;
          store4(w_out + o, aw[0], aw[1], aw[2], aw[3]);
          store4(u_out + o, au[0], au[1], au[2], au[3]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------- walk

// Register stage of a ROWS x COLS tile: each thread holds PER 16-byte pieces.
// load() only issues global loads (rows >= valid read as zero); store()
// writes them to LDS rows of stride LS.
template <typename E, int ROWS, int COLS, int NT>
struct TileReg {
  static constexpr int EPP = 16 / (int)sizeof(E);
  static constexpr int PPR = COLS / EPP;
  static constexpr int PIECES = ROWS * PPR;
  static constexpr int PER = (PIECES + NT - 1) / NT;
  uint4 v[PER];
  __device__ __forceinline__ void load(const E* src, size_t gstride, int valid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pc = (int)threadIdx.x + i * NT;
      const int r = pc / PPR, cc = (pc - r * PPR) * EPP;
      v[i] = make_uint4(0, 0, 0, 0);
      if (pc < PIECES && r < valid)
        v[i] = *reinterpret_cast<const uint4*>(src + (size_t)r * gstride + cc);
    }
  }
  template <int LS>
  __device__ __forceinline__ void store(E* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int pc = (int)threadIdx.x + i * NT;
      if (pc < PIECES) {
        const int r = pc / PPR, cc = (pc - r * PPR) * EPP;
        E* dst = lds + r * LS + cc;
        if ((LS * sizeof(E)) % 16 == 0) {
          *reinterpret_cast<uint4*>(dst) = v[i];
        } else {  // rows only 8-byte aligned
          reinterpret_cast<uint2*>(dst)[0] = make_uint2(v[i].x, v[i].y);
          reinterpret_cast<uint2*>(dst)[1] = make_uint2(v[i].z, v[i].w);
        }
      }
    }
  }
};

// The inter-chunk walk fused with the output projection.  One workgroup of NW
// waves per (sequence, value head, block of 16 NW value channels); each wave
// owns 16 value channels and keeps its 128 x 16 slice of the state in MFMA
// accumulators (fp32) for the whole sequence.  Per chunk, all waves share the
// K-side operands (w, qg, kg_t, aqk, decay) staged once in LDS.
template <typename E, int NW>
__global__ __launch_bounds__(64 * NW) void walk_kernel(
    const E* __restrict__ qg, const E* __restrict__ kg_t, const float* __restrict__ decay,
    const E* __restrict__ w, const E* __restrict__ u, const E* __restrict__ aqk,
    const int32_t* __restrict__ cu, int dense_len, int T, const int32_t* __restrict__ offs,
    int N, int hv, float scale, const float* __restrict__ init, float* __restrict__ fin,
    float* __restrict__ cache, const int32_t* __restrict__ slots,
    const uint8_t* __restrict__ has_init, int num_slots, E* __restrict__ out, int nvb,
    int units, int max_chunks) {
  constexpr bool SPLIT = std::is_same<E, float>::value;
  constexpr int NT = 64 * NW;
  constexpr int BV = 16 * NW;
  // Row strides (elements) of the LDS tiles.  A fragment read has 16 lanes
  // take 8 (bf16) or 16 (fp32) bytes from 16 consecutive rows at one column;
  // a stride of 4 elements past a 128-byte multiple puts those rows on
  // disjoint banks.
  constexpr int PAD = 4;
  constexpr int S128 = D + PAD, S64 = C + PAD, SU = BV + PAD;
  __shared__ E sW[C * S128];
  __shared__ E sQg[C * S128];
  __shared__ E sKg[D * S64];
  __shared__ E sAq[C * S64];
  __shared__ E sU[C * SU];
  __shared__ float sD[D];

  // The nvb blocks of one (sequence, head) get ids with equal id % 8, so they
  // land on one XCD and share its L2 for the K-side tiles.
  const int id = blockIdx.x;
  const int blk = id / (8 * nvb), rem = id - blk * 8 * nvb;
  const int vb = rem >> 3, unit = blk * 8 + (rem & 7);
  if (unit >= units) return;
  const int n = unit / hv, h = unit - n * hv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int v0 = vb * BV;                  // first value channel of the block
  const int vcol = v0 + 16 * wave + l16;   // this lane's C-tile column
  const SeqSpan sp = seq_span(cu, n, dense_len, T);

  const float* src = nullptr;
  float* dst = nullptr;
  if (cache) {
    const int slot = slots[n];
    if (slot < 0 || slot >= num_slots) {
      // null slot: zero output rows, no state traffic
      for (int idx = tid; idx < (sp.eos - sp.bos) * BV; idx += NT) {
        const int t = idx / BV, vv = idx - t * BV;
        out[((size_t)(sp.bos + t) * hv + h) * D + v0 + vv] = from_f32<E>(0.f);
      }
      return;
    }
    float* row = cache + ((size_t)slot * hv + h) * (size_t)(D * D);
    dst = row;
    if (has_init[n]) src = row;
  } else {
    if (init) src = init + ((size_t)n * hv + h) * (size_t)(D * D);
    if (fin) dst = fin + ((size_t)n * hv + h) * (size_t)(D * D);
  }

  // state slice: S[kb][r] = S[k = 16 kb + 4 gq + r][v = vcol]  (V-first row vcol)
  f32x4_t S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    if (src) {
      const float4 x = *reinterpret_cast<const float4*>(src + (size_t)vcol * D + 16 * kb + 4 * gq);
      S[kb] = f32x4_t{x.x, x.y, x.z, x.w};
    } else {
      S[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int c_first = offs[n];
  // a malformed cu_seqlens could claim chunks past the bound; never read them
  const int nch = max(0, min(offs[n + 1], max_chunks) - c_first);

  // K-side tiles of a chunk travel through registers: with bf16 operands the
  // next chunk's loads are issued before this chunk's products, so their
  // latency hides behind the MFMA work.
  constexpr bool PREFETCH = !SPLIT;
  TileReg<E, C, D, NT> rW, rQ;
  TileReg<E, C, C, NT> rA;
  TileReg<E, C, BV, NT> rU;
  TileReg<E, D, C, NT> rK;
  float rd = 0.f;
  auto fetch = [&](int jc) {
    const int c = c_first + jc;
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    rW.load(w + ((size_t)t0 * hv + h) * D, (size_t)hv * D, L);
    rQ.load(qg + ((size_t)t0 * hv + h) * D, (size_t)hv * D, L);
    rA.load(aqk + ((size_t)t0 * hv + h) * C, (size_t)hv * C, L);
    rU.load(u + ((size_t)t0 * hv + h) * D + v0, (size_t)hv * D, L);
    rK.load(kg_t + ((size_t)c * hv + h) * D * C, C, D);
    if (tid < D) rd = decay[((size_t)c * hv + h) * D + tid];
  };
  if (PREFETCH && nch > 0) fetch(0);

  for (int jc = 0; jc < nch; ++jc) {
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    if (!PREFETCH) fetch(jc);
    __syncthreads();
    rW.template store<S128>(sW);
    rQ.template store<S128>(sQg);
    rA.template store<S64>(sAq);
    rU.template store<SU>(sU);
    rK.template store<S64>(sKg);
    if (tid < D) sD[tid] = rd;
    __syncthreads();
    if (PREFETCH && jc + 1 < nch) fetch(jc + 1);

    // the state as an MFMA operand (K = key channel, in perm32 order)
    Frag<SPLIT> Hf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                    S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
      Hf[s] = make_frag<SPLIT>(x);
    }
    // HW = w S (rows t, cols v) and O^T = (qg S)^T (rows v, cols t)
    f32x4_t HW[4], O[4];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      HW[ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      O[ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const E* wr = sW + (16 * ta + l16) * S128 + 32 * s + 4 * gq;
        mma(HW[ta], frag_from(wr, wr + 16), Hf[s]);
        const E* qr = sQg + (16 * ta + l16) * S128 + 32 * s + 4 * gq;
        mma(O[ta], Hf[s], frag_from(qr, qr + 16));
      }
    }
    // U = u - w S   (C layout: col v, rows t = 16 ta + 4 gq + r)
    Frag<SPLIT> Uf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float x[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ta = 2 * s2 + half;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * ta + 4 * gq + r;
          x[4 * half + r] = to_f32(sU[t * SU + 16 * wave + l16]) - HW[ta][r];
        }
      }
      Uf[s2] = make_frag<SPLIT>(x);
    }
    // O^T += U^T A_qk^T  (A_qk lower: t < 32 needs i < 32 only)
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (s2 == 1 && ta < 2) continue;
        const E* ar = sAq + (16 * ta + l16) * S64 + 32 * s2 + 4 * gq;
        mma(O[ta], Uf[s2], frag_from(ar, ar + 16));
      }
      const int t = 16 * ta + l16;
      if (t < L) {
        E* op = out + ((size_t)(t0 + t) * hv + h) * D + v0 + 16 * wave + 4 * gq;
        store4(op, scale * O[ta][0], scale * O[ta][1], scale * O[ta][2], scale * O[ta][3]);
      }
    }
    // S <- diag(d) S + kg^T U   (rows k, cols v, K = t)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kb][r] *= sD[16 * kb + 4 * gq + r];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const E* kr = sKg + (16 * kb + l16) * S64 + 32 * s2 + 4 * gq;
        mma(S[kb], frag_from(kr, kr + 16), Uf[s2]);
      }
    }
  }
  if (dst) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      *reinterpret_cast<float4*>(dst + (size_t)vcol * D + 16 * kb + 4 * gq) =
          make_float4(S[kb][0], S[kb][1], S[kb][2], S[kb][3]);
  }
}

// --------------------------------------------------------------------- launch

static void mark(const ChunkLaunch& L, int i) {
  if (i < L.num_events && L.events[i]) (void)hipEventRecord((hipEvent_t)L.events[i], (hipStream_t)L.stream);
}

template <typename E>
static hipError_t launch_staged_t(const ChunkLaunch& L) {
  hipStream_t st = (hipStream_t)L.stream;
  mark(L, 0);
  const int N = L.num_seqs;
  const int T = (int)L.total_tokens;
  const int dense_len = L.cu ? 0 : (N > 0 ? T / N : 0);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, L.cu, N, dense_len, T,
                     L.chunk_offsets);
  mark(L, 1);
  if (L.max_chunks > 0 && T > 0) {
    hipLaunchKernelGGL(prep_kernel<E>, dim3((unsigned)L.max_chunks, L.hqk), dim3(256), 0, st,
                       (const E*)L.q, (const E*)L.k, (const E*)L.g, L.cu, dense_len, T,
                       L.chunk_offsets, N, L.hqk, L.hv, L.use_l2, (E*)L.qg, (E*)L.kg_t,
                       L.decay);
    mark(L, 2);
    hipLaunchKernelGGL(wy_kernel<E>, dim3((unsigned)L.max_chunks, L.hv), dim3(256), 0, st,
                       (const E*)L.q, (const E*)L.k, (const E*)L.v, (const E*)L.g,
                       (const E*)L.beta, L.cu, dense_len, T, L.chunk_offsets, N, L.hqk, L.hv,
                       L.use_l2, (E*)L.w, (E*)L.u, (E*)L.aqk);
  } else {
    mark(L, 2);
  }
  mark(L, 3);
  constexpr int NW = 4;
  const int nvb = D / (16 * NW);
  const int units = N * L.hv;
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * nvb);
  hipLaunchKernelGGL((walk_kernel<E, NW>), dim3(grid), dim3(64 * NW), 0, st, (const E*)L.qg,
                     (const E*)L.kg_t, L.decay, (const E*)L.w, (const E*)L.u,
                     (const E*)L.aqk, L.cu, dense_len, T, L.chunk_offsets, N, L.hv, L.scale,
                     L.init, L.fin, L.cache, L.slots, L.has_init, L.num_slots, (E*)L.out, nvb,
                     units, (int)L.max_chunks);
  mark(L, 4);
  mark(L, 5);
  mark(L, 6);
  return hipGetLastError();
}

hipError_t launch_chunk_staged(const ChunkLaunch& L) {
  if (L.groups > 1) return hipErrorNotSupported;
  return L.dtype == 0 ? launch_staged_t<float>(L) : launch_staged_t<bf16>(L);
}

}  // namespace kda
