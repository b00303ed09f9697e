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
// kernel therefore evaluates 2^(G_t - G_i) through a reference token m_a =
// 16 a + 7 of each 16-token block a (t in block a, i in block b):
//   2^(G_t - G_i) = 2^(G_t - G_ma) * 2^(G_ma - G_mb) * 2^(G_mb - G_i)
// The outer factors span at most 8 steps each (within 2^(+-58), finite in
// fp32 and bf16); the middle one (b < a) is <= 1, at least 2^-115.4 for
// adjacent blocks with g >= -5, and rounds to zero only for blocks two or
// more apart whose true coupling is then below 2^-21.  Products for i > t may
// be large but finite and are masked away.
#include <algorithm>
#include <type_traits>

#include "kda_chunk_common.hpp"

namespace kda {

// ---------------------------------------------------------------- chunk table

// Chunk table: per-sequence chunk offsets (offs[n] = first chunk of sequence
// n, offs[N] = number of chunks) and one record (sequence, first token,
// length, 0) per chunk below max_chunks, length 0 past the last chunk, so a
// kernel finds its chunk with one 16-byte load.
// The chunk counts are scanned with wave shuffles and one LDS pass over the
// 16 wave totals; the records are then filled in parallel, each thread
// finding its chunk's sequence by binary search over the offsets (held in LDS
// up to OFFS_LDS sequences; beyond that each thread writes its own sequences'
// records in turn).
constexpr int OFFS_LDS = 8192;
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* cu, int N,
                                                             int dense_len, int T,
                                                             int32_t* offs, int4* table,
                                                             int max_chunks, uint4* zero) {
  __shared__ int32_t wsum[16], wmax[16], ccount[64];
  __shared__ int32_t soffs[OFFS_LDS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 65) zero[tid] = make_uint4(0, 0, 0, 0);  // the zero page the walk DMAs from,
                                                     // then the WY work counter
  const int per = (N + 1023) / 1024;
  const int s0 = min(N, tid * per), s1 = min(N, s0 + per);
  int sum = 0, longest = 0;
  for (int n = s0; n < s1; ++n) {
    const SeqSpan s = seq_span(cu, n, dense_len, T);
    const int nc = (s.eos - s.bos + C - 1) / C;
    sum += nc;
    longest = max(longest, nc);
  }
  // the longest sequence's chunk count (the group scan's group length comes
  // from it), capped at the chunk bound like every walk's own count
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) longest = max(longest, __shfl_xor(longest, off));
  if (lane == 0) wmax[wave] = longest;
  // inclusive scan inside the wave, then across the 16 wave totals
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (tid < 16) {
    int x = wsum[tid];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int v = __shfl_up(x, off, 16);
      if (tid >= off) x += v;
    }
    wsum[tid] = x;  // inclusive over waves
  }
  __syncthreads();
  if (tid == 0) {
    int m = 0;
    for (int w = 0; w < 16; ++w) m = max(m, wmax[w]);
    reinterpret_cast<int32_t*>(reinterpret_cast<char*>(zero) + KDA_NCH_MAX_OFFSET)[0] =
        min(m, max_chunks);
  }
  const int run0 = (wave > 0 ? wsum[wave - 1] : 0) + incl - sum;  // exclusive
  const int total = wsum[15];
  const bool in_lds = N <= OFFS_LDS;
  {
    int run = run0;
    for (int n = s0; n < s1; ++n) {
      offs[n] = run;
      if (in_lds) soffs[n] = run;
      const SeqSpan s = seq_span(cu, n, dense_len, T);
      const int nc = (s.eos - s.bos + C - 1) / C;
      if (!in_lds)
        for (int j = 0; j < nc; ++j)
          if (run + j < max_chunks)
            table[run + j] = make_int4(n, s.bos + C * j, min(C, s.eos - s.bos - C * j), 0);
      run += nc;
    }
  }
  if (tid == 1023) offs[N] = total;
  {
    // The sequences in decreasing chunk count, after offs[N]: a counting
    // sort over quarter-octave classes (ties in any order), so that the
    // walks, whose workgroups start in index order, begin with the longest
    // chains and the short ones fill in around them.
    auto cls = [](int nc) {
      if (nc <= 0) return 0;
      const int e = 31 - __clz(nc);
      const int f = e >= 2 ? (nc >> (e - 2)) & 3 : (nc << (2 - e)) & 3;
      return min(63, 4 * e + f + 1);
    };
    for (int i = tid; i < 64; i += 1024) ccount[i] = 0;
    __syncthreads();
    for (int n = s0; n < s1; ++n) {
      const SeqSpan s = seq_span(cu, n, dense_len, T);
      atomicAdd(&ccount[cls((s.eos - s.bos + C - 1) / C)], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int c = 63; c >= 0; --c) {
        const int k = ccount[c];
        ccount[c] = run;
        run += k;
      }
    }
    __syncthreads();
    int32_t* order = offs + N + 1;
    for (int n = s0; n < s1; ++n) {
      const SeqSpan s = seq_span(cu, n, dense_len, T);
      order[atomicAdd(&ccount[cls((s.eos - s.bos + C - 1) / C)], 1)] = n;
    }
  }
  if (in_lds) {
    if (tid == 0) soffs[N] = total;
    __syncthreads();
    for (int c = tid; c < min(total, max_chunks); c += 1024) {
      // the sequence n with soffs[n] <= c < soffs[n + 1] (empty sequences share
      // their offset with the next one; the search lands on the last of them,
      // which is the non-empty one)
      int lo = 0, hi = N - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (soffs[mid] <= c) lo = mid; else hi = mid - 1;
      }
      const SeqSpan s = seq_span(cu, lo, dense_len, T);
      const int t0 = s.bos + C * (c - soffs[lo]);
      table[c] = make_int4(lo, t0, min(C, s.eos - t0), 0);
    }
  }
  for (int c = total + tid; c < max_chunks; c += 1024) table[c] = make_int4(0, 0, 0, 0);
}

struct ChunkPos {
  int n, t0, L;
};

__device__ __forceinline__ bool locate_chunk(int c, const int4* table, ChunkPos& p) {
  const int4 e = table[c];
  p.n = e.x;
  p.t0 = e.y;
  p.L = e.z;
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
__device__ __forceinline__ void load8(const _Float16* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
    x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
// A 64 x 128 token tile of q and k (L2-normalised when asked) into fp32 LDS.
// Thread mapping: 16 lanes (one DPP row) per token row, 8 channels per lane;
// all four row loads are issued before the first reduction.
template <typename E>
__device__ __forceinline__ void load_rows4(const E* src, int stride_t, int L, float (&x)[4][8]) {
  // Rows past L re-read row L - 1 (always in bounds, L >= 1) and are zeroed
  // afterwards, so the four loads go out back to back with no branch.
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = min(rg + 16 * it, L - 1);
    load8(src + (size_t)t * stride_t + 8 * j, x[it]);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const bool live = rg + 16 * it < L;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[it][e] = live ? x[it][e] : 0.f;
  }
}

// The same tile with each thread holding four consecutive tokens: rows
// 4 rg + it, so wave w holds the 16-token block w.
template <typename E>
__device__ __forceinline__ void load_rows4c(const E* src, int stride_t, int L, float (&x)[4][8]) {
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = min(4 * rg + it, L - 1);
    load8(src + (size_t)t * stride_t + 8 * j, x[it]);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const bool live = 4 * rg + it < L;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[it][e] = live ? x[it][e] : 0.f;
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
  lds_barrier();
  const int c = tid & 127, half = tid >> 7;  // 256 threads: two halves of 32 tokens
  float run = 0.f;
#pragma unroll 8
  for (int tt = 0; tt < 32; ++tt) {
    run += sG[32 * half + tt][c];
    sG[32 * half + tt][c] = run;
  }
  lds_barrier();
  if (half == 1) {
    const float base = sG[31][c];
#pragma unroll 8
    for (int tt = 0; tt < 32; ++tt) sG[32 + tt][c] += base;
  }
  lds_barrier();
}

// ----------------------------------------------------------------------- prep

// LDS element type of the staged operand tiles: bf16 inputs keep bf16 tiles,
// fp32 inputs keep fp32 tiles (their MFMA operands are split hi + lo).
template <typename E> struct TileT;
template <> struct TileT<bf16> { using T = bf16; };
template <> struct TileT<float> { using T = float; };

__device__ __forceinline__ void st_elem(bf16* p, float x) { p->x = bf16_bits(x); }
__device__ __forceinline__ void st_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ float ld_elem(const bf16* p) { return to_f32(*p); }
__device__ __forceinline__ float ld_elem(const float* p) { return *p; }

// One workgroup per (chunk, query/key head); loops over the value heads of the
// GVA group.  Streaming: reads q, k, g once and writes qg (token-major, key
// channel packed), kg_t (chunk-major, token packed) and decay.  The LDS G tile
// doubles as the transpose buffer of kg.
template <typename E, typename I>
__global__ __launch_bounds__(256) void prep_kernel(const I* __restrict__ q,
                                                   const I* __restrict__ k,
                                                   const I* __restrict__ g,
                                                   const int4* __restrict__ table,
                                                   int hqk, int hv, int use_l2,
                                                   E* __restrict__ qg, E* __restrict__ kg_t,
                                                   float* __restrict__ decay,
                                                   const GateArgs ga, const InStrides is) {
  constexpr int SK = D + 4;
  __shared__ float sG[C][SK];
  E* sKg = reinterpret_cast<E*>(&sG[0][0]);   // kg tile [64][SKG] after G is consumed
  constexpr int SKG = sizeof(E) == 4 ? D + 4 : D + 8;  // must fit in the G tile
  ChunkPos p;
  if (!locate_chunk(blockIdx.x, table, p)) return;
  const int c = blockIdx.x, hq = blockIdx.y, grp = hv / hqk;
  const int tid = threadIdx.x, rg = tid >> 4, j = tid & 15;
  const int L = p.L;

  float qn[4][8], kn[4][8], gx[4][8];
  load_rows4(q + (size_t)p.t0 * is.q + hq * D, (int)is.q, L, qn);
  load_rows4(k + (size_t)p.t0 * is.k + hq * D, (int)is.k, L, kn);
  load_rows4(g + (size_t)p.t0 * is.g + hq * grp * D, (int)is.g, L, gx);
  if (use_l2) {
    l2norm_rows4(qn);
    l2norm_rows4(kn);
  }
  const int cb = 32 * (j >> 2), run0 = cb + pack32(8 * (j & 3)), run1 = cb + pack32(8 * (j & 3) + 4);

  for (int gi = 0; gi < grp; ++gi) {
    const int h = hq * grp + gi;
    if (gi > 0) {
      lds_barrier();
      load_rows4(g + (size_t)p.t0 * is.g + h * D, (int)is.g, L, gx);
    }
    if (ga.a_log) {
      // raw gate -> log-decay; rows past L stay 0
      const float a = exp2_fast(ga.a_log[h] * LOG2E);
      float bias[8];
      gate_bias8(ga, h, 8 * j, bias);
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          gx[it][e] = rg + 16 * it < L ? gate_apply(gx[it][e], a, bias[e], ga.lower_bound) : 0.f;
    }
    gate_cumsum<SK>(gx, sG);
    float G[4][8], Gl[8];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[it][e] = sG[rg + 16 * it][8 * j + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) Gl[e] = sG[L - 1][8 * j + e];
    lds_barrier();  // G consumed; the tile now holds kg
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = rg + 16 * it;
      float xq[8], xk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xq[e] = qn[it][e] * exp2_fast(G[it][e]);
        xk[e] = kn[it][e] * exp2_fast(Gl[e] - G[it][e]);
        st_elem(sKg + t * SKG + 8 * j + e, xk[e]);
      }
      if (t < L) {
        E* dst = qg + ((size_t)(p.t0 + t) * hv + h) * D;
        store4(dst + run0, xq[0], xq[1], xq[2], xq[3]);
        store4(dst + run1, xq[4], xq[5], xq[6], xq[7]);
      }
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        decay[((size_t)c * hv + h) * D + 8 * j + e] = exp2_fast(Gl[e]);
    }
    lds_barrier();
    // kg_t[c][h][kk][packed t]: thread -> key channel kk, one 32-token block
    {
      const int kk = tid >> 1, tb = 32 * (tid & 1);
      E* dst = kg_t + (((size_t)c * hv + h) * D + kk) * C + tb;
#pragma unroll
      for (int m4 = 0; m4 < 8; ++m4) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = ld_elem(sKg + (tb + unpack32(4 * m4 + r)) * SKG + kk);
        store4(dst + 4 * m4, x[0], x[1], x[2], x[3]);
      }
    }
  }
}

// ------------------------------------------------------------------------- WY

// One workgroup (4 waves) per (chunk, value head).
//   phase 0: q, k normalised; G = log2(e) cumsum(g) in registers (a wave
//            holds one 16-token block, four consecutive tokens and eight
//            consecutive channels per thread); block-referenced operand tiles
//            QL = qn 2^(G - G_m), KL = kn 2^(G - G_m), KR = kn 2^(G_m - G)
//            (m = token 16 a + 7 of the row's block a); the decay factors
//            between block references E_ab = 2^(G_ma - G_mb), b < a.
//   phase 1: A_kk (to LDS, fp32) and A_qk (to memory) on MFMA:
//            A[t][i] = L_a[t] . KR_b[i] E_ab for t in block a, i in b.
//            Then kn 2^G and v are laid down transposed (token-contiguous).
//   Channel order inside the kernel is natural; the fragment order of the
//   outputs (qg, w) is applied when they are stored.
//   phase 2: T = (I + A_kk)^-1 in fp32 by blocked forward substitution.
//   phase 3: with T' = T diag(b): w = T' (kn 2^G) and u = T' v on MFMA.
//
// With PREP the kernel also writes the prep outputs (qg, kg_t, decay), so the
// inputs are read from HBM once for the whole intra-chunk stage.
// One token's qg row from the 16 lanes of a row group (lane j: channels
// 8 j .. 8 j + 7), stored in fragment order.  A lane's channels fall on two
// runs of 4 packed positions; lanes j and j ^ 2 (one DPP quad) swap a run so
// that each lane holds 8 consecutive positions, and the row leaves as sixteen
// 16-byte pieces that fill whole 64-byte segments.
__device__ __forceinline__ void qg_row_store(bf16* row, const float (&x)[8], int j) {
  const uint4 u = __builtin_bit_cast(uint4, pack8(x));
  const bool up = (j & 2) != 0;  // lanes 2, 3 of the quad keep their second run
  const uint32_t s0 = up ? u.x : u.z, s1 = up ? u.y : u.w;
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x4E, 0xF, 0xF, true);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x4E, 0xF, 0xF, true);
  const uint4 o = up ? make_uint4(r0, r1, u.z, u.w) : make_uint4(u.x, u.y, r0, r1);
  *reinterpret_cast<uint4*>(row + 32 * (j >> 2) + 16 * (j & 1) + 8 * ((j >> 1) & 1)) = o;
}
__device__ __forceinline__ void qg_row_store(float* row, const float (&x)[8], int j) {
  float* dst = row + 32 * (j >> 2);
  store4(dst + pack32(8 * (j & 3)), x[0], x[1], x[2], x[3]);
  store4(dst + pack32(8 * (j & 3) + 4), x[4], x[5], x[6], x[7]);
}

template <typename E, bool PREP, bool GATE, typename I>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void wy_kernel(
    const I* __restrict__ q, const I* __restrict__ k, const I* __restrict__ v,
    const I* __restrict__ g, const I* __restrict__ beta, const int4* __restrict__ table,
    int hqk, int hv, int use_l2, E* __restrict__ w_out, E* __restrict__ u_t,
    E* __restrict__ aqk, E* __restrict__ qg, E* __restrict__ kg_t, float* __restrict__ decay,
    int items, int* __restrict__ counter, const GateArgs ga, const InStrides is) {
  constexpr bool SPLIT = std::is_same<E, float>::value;
  using TE = typename TileT<E>::T;
  constexpr int ST = D + (SPLIT ? 4 : 8);        // row stride of the [64 t][128] tiles
  constexpr int TILE = C * ST * (int)sizeof(TE);
  constexpr int TTILE = D * C * (int)sizeof(TE);  // transposed [128][64 t] tile
  constexpr int SA = C + 4;                       // A_kk / T row stride (fp32)
  constexpr int AB = C * SA * 4;
  // regions: R0 = QL | (kn 2^G)^T ; R1 = KL | v^T ; R2 = KR | T ; R3 = A
  constexpr int R0SZ = TILE > TTILE ? TILE : TTILE;
  constexpr int R2SZ = TILE > AB ? TILE : AB;
  constexpr int R0 = 0, R1 = R0 + R0SZ, R2 = R1 + R0SZ, R3 = R2 + R2SZ;
  constexpr int RE = R3 + AB;          // E_ab [6][128] fp32
  constexpr int RP = RE + 6 * D * 4;   // per-wave inclusive sums at token 16 w + 7
  constexpr int RWT = RP + 4 * D * 4;  // per-wave gate totals
  constexpr int RB = RWT + 4 * D * 4;  // b [64]
  constexpr int BYTES = RB + C * 4;
  __shared__ __attribute__((aligned(16))) char smem[BYTES];
  TE* QL = reinterpret_cast<TE*>(smem + R0);
  TE* KL = reinterpret_cast<TE*>(smem + R1);
  TE* KR = reinterpret_cast<TE*>(smem + R2);
  uint4* KGt = reinterpret_cast<uint4*>(smem + R0);
  uint4* Vt = reinterpret_cast<uint4*>(smem + R1);
  float* sTt = reinterpret_cast<float*>(smem + R2);
  float* sA = reinterpret_cast<float*>(smem + R3);
  float* sE = reinterpret_cast<float*>(smem + RE);
  float* sP = reinterpret_cast<float*>(smem + RP);
  float* sWt = reinterpret_cast<float*>(smem + RWT);
  float* sB = reinterpret_cast<float*>(smem + RB);

  const int grp = hv / hqk;

  // Persistent: work item = (chunk, value head), chunk-major.  A workgroup
  // starts with item blockIdx.x and claims each following item from a
  // counter (zeroed by the chunk-table kernel) while it works on the current
  // one, so fast workgroups take more items.  The raw q, k, g rows and beta
  // of the next item are fetched during this item's phases 1-3.  Items past
  // the last chunk end the loop (their records have length 0, and every
  // later claim is past it too).
  __shared__ int s_next;
  int item = blockIdx.x;
  ChunkPos p;
  bool ok = item < items && locate_chunk(item / hv, table, p);
  RawRows<I> rq, rk, rgt;
  I rb;
  float gA = 0.f;  // gate parameters of the item's head (GATE): A_log, dt_bias bits
  uint4 gB0 = make_uint4(0, 0, 0, 0), gB1 = gB0;
  auto prefetch = [&](int it_, const ChunkPos& pp, int tid) {
    const int h_ = it_ % hv, hq_ = h_ / grp;
    raw_load(q + (size_t)pp.t0 * is.q + hq_ * D, (int)is.q, pp.L, rq, tid);
    raw_load(k + (size_t)pp.t0 * is.k + hq_ * D, (int)is.k, pp.L, rk, tid);
    raw_load(g + (size_t)pp.t0 * is.g + h_ * D, (int)is.g, pp.L, rgt, tid);
    rb = beta[(size_t)(pp.t0 + min(tid, pp.L - 1)) * is.beta + h_];
    if constexpr (GATE) {
      gA = ga.a_log[h_];
      gate_bias8_bits(ga, h_, 8 * (tid & 15), gB0, gB1);
    }
  };
  if (ok) prefetch(item, p, (int)threadIdx.x);

  while (ok) {
  // Lane-derived indices are rebuilt from an opaque copy of the thread id in
  // every iteration: hoisted out of the loop, the many per-lane LDS addresses
  // derived from them would stay live across the whole loop.
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int l16 = lane & 15, gq = lane >> 4;
  const int rg = tid >> 4, j = tid & 15, r4 = lane >> 4;
  const int c = item / hv, h = item - c * hv;
  const int L = p.L;
  int claim = 0;
  // the next item; published below.  atomicInc (with no wrap below 2^32) is
  // an add of 1 that the compiler's atomic combining leaves as it is: the
  // combined form reads its result back at once, so every item would start by
  // waiting for the atomic and for all of the previous item's stores.
  if (tid == 0) claim = (int)atomicInc(reinterpret_cast<unsigned*>(counter), 0xffffffffu);

  // kn 2^G for phase 3, kept (per channel, 4 tokens) across phase 1
  typename Col4<E>::T kgp[8];

  // ---- phase 0
  {
    float qx[4][8], kx[4][8], G[4][8];
    raw_decode(rq, L, qx, tid);
    raw_decode(rk, L, kx, tid);
    raw_decode(rgt, L, G, tid);
    if constexpr (GATE) {
      // raw gate -> log-decay; rows past L stay 0
      float gB[8];
      gate_bias8_decode(ga, gB0, gB1, gB);
      const float a = exp2_fast(gA * LOG2E);
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          G[it][e] = 4 * rg + it < L ? gate_apply(G[it][e], a, gB[e], ga.lower_bound) : 0.f;
    }
    const float braw = to_f32(rb);
    if (use_l2) {
      l2norm_rows4(qx);
      l2norm_rows4(kx);
    }
    // G: inclusive cumsum over tokens (rows past L hold g = 0, so G stays at
    // G_{L-1} there).  In-thread over the 4 tokens, across the 4 row groups
    // of the wave by shuffles, across waves through LDS.
    float excl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float run = 0.f;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        run += G[it][e] * LOG2E;
        G[it][e] = run;
      }
      float x = run, y;
      y = __shfl_up(x, 16);
      x += r4 >= 1 ? y : 0.f;
      y = __shfl_up(x, 32);
      x += r4 >= 2 ? y : 0.f;
      excl[e] = x - run;
      if (r4 == 1) sP[wv * D + 8 * j + e] = x;   // through token 16 w + 7
      if (r4 == 3) sWt[wv * D + 8 * j + e] = x;  // the whole block
    }
    lds_barrier();
    float Gl[8], Gm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float before = 0.f, all = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float x = sWt[w2 * D + 8 * j + e];
        before += w2 < wv ? x : 0.f;
        all += x;
      }
      Gl[e] = all;  // G at the last token of the chunk
#pragma unroll
      for (int it = 0; it < 4; ++it) G[it][e] += excl[e] + before;
      // reference token 16 wv + 7 of this wave's block: row group 1, it = 3
      Gm[e] = __shfl(G[3][e], 16 + j);
    }
    // E_ab = 2^(G_ma - G_mb) for the 6 pairs b < a (pair index a (a - 1) / 2 + b)
#pragma unroll
    for (int m = 0; m < 3; ++m) {
      const int idx = tid + 256 * m, pi = idx >> 7, ch = idx & (D - 1);
      const int a = pi < 1 ? 1 : (pi < 3 ? 2 : 3), b = pi - a * (a - 1) / 2;
      float ga = sP[a * D + ch], gb = sP[b * D + ch];
#pragma unroll
      for (int w2 = 0; w2 < 3; ++w2) {
        ga += w2 < a ? sWt[w2 * D + ch] : 0.f;
        gb += w2 < b ? sWt[w2 * D + ch] : 0.f;
      }
      sE[idx] = exp2_fast(ga - gb);
    }
    if (tid < C) sB[tid] = (tid < L) ? sigmoid(braw) : 0.f;
    float pm[8], pl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pm[e] = exp2_fast(Gm[e]);          // 2^G = 2^(G - G_m) 2^G_m
      pl[e] = exp2_fast(Gl[e] - Gm[e]);  // 2^(G_last - G) = 2^(G_m - G) 2^(G_last - G_m)
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = 4 * rg + it;
      float xq[8], xl[8], xr[8], xg[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dg = G[it][e] - Gm[e];
        const float up = exp2_fast(dg);
        const float dn = exp2_fast(-dg);  // the negation is a source modifier
        xq[e] = qx[it][e] * up;
        xl[e] = kx[it][e] * up;
        xr[e] = kx[it][e] * dn;
        G[it][e] = xl[e] * pm[e];    // kn 2^G (G is dead from here)
        xg[e] = xq[e] * pm[e];       // qn 2^G
        kx[it][e] = xr[e] * pl[e];   // kn 2^(G_last - G)
      }
      store8(QL + t * ST + 8 * j, xq);
      store8(KL + t * ST + 8 * j, xl);
      store8(KR + t * ST + 8 * j, xr);
      // (the row group's 16 lanes share t, so a quad is uniformly in or out)
      if (PREP && t < L) qg_row_store(qg + ((size_t)(p.t0 + t) * hv + h) * D, xg, j);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) col4(kgp[e], G[0][e], G[1][e], G[2][e], G[3][e]);
    if (PREP) {
      // kg_t[c][h][key channel][packed t]: this thread's 4 consecutive tokens
      // are 4 consecutive packed positions (zero past L)
      if constexpr (!SPLIT) {
        // staged in R3 (A_kk's region, free until phase 1) as [128][64]
        // with 16-byte pieces XOR-swizzled by (row >> 3) & 7, and stored
        // from there in whole 16-byte pieces after the barrier
        const int pos = packed_index(4 * rg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * j + e;
          col4(*reinterpret_cast<bf16x4_t*>(smem + R3 + r * 128 +
                                            (((pos >> 3) ^ (r >> 3 & 7)) << 4) + 2 * (pos & 7)),
               kx[0][e], kx[1][e], kx[2][e], kx[3][e]);
        }
      } else {
        E* kdst = kg_t + ((size_t)c * hv + h) * D * C + packed_index(4 * rg);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          store4(kdst + (size_t)(8 * j + e) * C, kx[0][e], kx[1][e], kx[2][e], kx[3][e]);
      }
      if (tid < 16) {
        float dv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) dv[e] = exp2_fast(Gl[e]);
        store8(decay + ((size_t)c * hv + h) * D + 8 * j, dv);
      }
    }
  }
  // v rows, requested as soon as phase 0's registers are free; they land
  // during phase 1.  Rows past L are not zeroed: they meet b = 0 columns
  // of T'.
  RawRows<I> rv;
  raw_load(v + (size_t)p.t0 * is.v + h * D, (int)is.v, L, rv, tid);
  if (tid == 0) s_next = claim + (int)gridDim.x;
  lds_barrier();
  const int nitem = s_next;
  ChunkPos np;
  const bool nok = nitem < items && locate_chunk(nitem / hv, table, np);
  if constexpr (PREP && !SPLIT) {
    // the item's kg_t (16 KB, contiguous in memory) leaves the staging tile
    // in whole rows: piece tid + 256 m is row (tid + 256 m) / 8, piece tid % 8
    E* kdst = kg_t + ((size_t)c * hv + h) * D * C;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = (tid >> 3) + 32 * m, pc = tid & 7;
      *reinterpret_cast<uint4*>(kdst + (size_t)r * C + 8 * pc) =
          *reinterpret_cast<const uint4*>(smem + R3 + r * 128 + ((pc ^ (r >> 3 & 7)) << 4));
    }
    lds_barrier();  // R3 becomes A_kk
  }

  // ---- phase 1: couplings, transposed tiles (rows i from KR, columns t from L).
  //      Each wave takes a fixed set of units (row block a, column blocks
  //      2 m and 2 m + 1): a lane's A_qk values of the two blocks are 8
  //      consecutive packed positions, stored as one 16-byte piece; blocks
  //      above the diagonal are stored as zeros.
  {
    auto pair = [&](const int a, const int b, float (&aq)[4]) {
      const int t = 16 * a + l16;
      const int i = 16 * b + l16;
      const float* eab = sE + (a * (a - 1) / 2 + b) * D;
      f32x4_t acck = {0.f, 0.f, 0.f, 0.f}, accq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c0 = 32 * s + 8 * gq;
        const Frag<SPLIT> Lk = frag_row(KL + t * ST + c0);
        const Frag<SPLIT> Lq = frag_row(QL + t * ST + c0);
        Frag<SPLIT> R;
        if (a == b) {
          R = frag_row(KR + i * ST + c0);
        } else {
          float x[8], ef[8];
          row8(KR + i * ST + c0, x);
          row8(eab + c0, ef);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= ef[e];
          R = make_frag<SPLIT>(x);
        }
        mma(acck, R, Lk);
        mma(accq, R, Lq);
      }
      const int i0 = 16 * b + 4 * gq;
      float ak[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ak[r] = (i0 + r < t) ? acck[r] * sB[t] : 0.f;
        aq[r] = (i0 + r <= t) ? accq[r] : 0.f;
      }
      store4(sA + t * SA + i0, ak[0], ak[1], ak[2], ak[3]);
    };
    auto unit = [&](const int a, const int m) {
      float aq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float lo[4], hi[4];
      if (2 * m <= a) {
        pair(a, 2 * m, lo);
#pragma unroll
        for (int r = 0; r < 4; ++r) aq[r] = lo[r];
      }
      if (2 * m + 1 <= a) {
        pair(a, 2 * m + 1, hi);
#pragma unroll
        for (int r = 0; r < 4; ++r) aq[4 + r] = hi[r];
      }
      const int t = 16 * a + l16;
      if (t < L) store8(aqk + ((size_t)(p.t0 + t) * hv + h) * C + 32 * m + 8 * gq, aq);
    };
    // ten block products over the four waves (3 / 2 / 3 / 2)
    if (wv == 0) {
      unit(3, 1); unit(0, 0);
    } else if (wv == 1) {
      unit(3, 0); unit(1, 1);
    } else if (wv == 2) {
      unit(2, 0); unit(2, 1);
    } else {
      unit(1, 0); unit(0, 1);
    }
  }
  // the next item's raw rows load during phases 2 and 3.  Without a next
  // item the first row of the current chunk is fetched by every lane (in
  // bounds, unused, a few hundred bytes): a branch-free fetch keeps the wait
  // for this item's v rows below from also waiting for these loads.
  const ChunkPos pf = nok ? np : ChunkPos{p.n, p.t0, 1};
  prefetch(nok ? nitem : item, pf, tid);
  lds_barrier();
  // (kn 2^G)^T into R0 and v^T into R1 (rows: channels 8 j + e), each
  // thread's 4 consecutive tokens as one run
  {
    constexpr int EPP = 16 / (int)sizeof(TE);
    const int piece = (4 * rg) / EPP, sub = (4 * rg) % EPP;
    using C4 = typename Col4<E>::T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * j + e;
      *reinterpret_cast<C4*>(reinterpret_cast<TE*>(KGt + tslot<TE>(r, piece)) + sub) = kgp[e];
      *reinterpret_cast<C4*>(reinterpret_cast<TE*>(Vt + tslot<TE>(r, piece)) + sub) =
          raw_column(rv, e);
    }
  }

  // ---- phase 2: T = (I + A_kk)^-1 (KR is dead: T takes its place)
  if (lane < 16) {
    // lane = column of the diagonal block; row r + 1 of A is read while row r
    // is substituted (every lane reads the same row: LDS broadcast)
    const int a = wave;
    const float* arow = sA + 16 * a * SA + 16 * a;
    float x[16];
    float4 cur[4], nxt[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) cur[q4] = *reinterpret_cast<const float4*>(arow + 4 * q4);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < 15) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          nxt[q4] = *reinterpret_cast<const float4*>(arow + (r + 1) * SA + 4 * q4);
      }
      const float av[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y,
                            cur[1].z, cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                            cur[3].x, cur[3].y, cur[3].z, cur[3].w};
      float val = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int ii = 0; ii < r; ++ii) val -= av[ii] * x[ii];
      x[r] = val;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sTt[(16 * a + r) * SA + 16 * a + lane] = x[r];
  }
  lds_barrier();
  // Off-diagonal blocks by columns: T_ab needs only T_aa and the blocks T_cb
  // (b <= c < a) of its own column, so wave b walks column b downwards, reading
  // back what it wrote itself (a wave's LDS accesses complete in order), and
  // one barrier closes the phase.
  if (wv < 3)
    for (int a = wv + 1; a < 4; ++a) wy_offdiag<SA>(a, wv, sA, sTt, lane);
  lds_barrier();

  // ---- phase 3: T' = T diag(b); w^T = (kn 2^G)^T T'^T and u = T' v
  Frag<SPLIT> Tf[4][2];  // T' rows t = 16 ta + l16, K = i = 32 s + 8 gq + jj
#pragma unroll
  for (int ta = 0; ta < 4; ++ta)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s == 1 && ta < 2) continue;  // T' is lower triangular
      const int i0 = 32 * s + 8 * gq;
      // Upper blocks of T are never written; the two that these fragments
      // span, (0, 1) and (2, 3), are taken as zero here.
      const bool upper = ((ta == 0 && s == 0) || (ta == 2 && s == 1)) && gq >= 2;
      float x[8], bb[8];
      row8(sTt + (16 * ta + l16) * SA + i0, x);
      row8(sB + i0, bb);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = upper ? 0.f : x[jj] * bb[jj];
      Tf[ta][s] = make_frag<SPLIT>(x);
    }
  // Paired 16-byte stores: a lane's w values of column blocks 2 wv and
  // 2 wv + 1 (same token) are adjacent in the packed key order, and its u_t
  // values of token blocks 2 m and 2 m + 1 (same channel) in the packed
  // token order.
  float wk[4][4];  // w of column block 2 wv, kept for the paired store
#pragma unroll
  for (int cbi = 0; cbi < 2; ++cbi) {
    const int cb = 2 * wv + cbi;
    const int row = 16 * cb + l16;  // key channel (w) / value channel (u) of this lane
    Frag<SPLIT> Yk[2], Yv[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (SPLIT) {
        float xk[8], xv[8];
        unit_vals_t(KGt, row, 8 * s + 2 * gq, xk);
        unit_vals_t(Vt, row, 8 * s + 2 * gq, xv);
        Yk[s] = make_frag<true>(xk);
        Yv[s] = make_frag<true>(xv);
      } else {
        Yk[s] = FragB{__builtin_bit_cast(bf16x8_t, KGt[tslot<TE>(row, 4 * s + gq)])};
        Yv[s] = FragB{__builtin_bit_cast(bf16x8_t, Vt[tslot<TE>(row, 4 * s + gq)])};
      }
    }
    float uk[4];  // u of the even token block, kept for the paired store
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      f32x4_t aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
      mma(aw, Yk[0], Tf[ta][0]);   // w^T: rows key channel, cols t
      mma(au, Tf[ta][0], Yv[0]);   // u:   rows t, cols value channel
      if (ta >= 2) {
        mma(aw, Yk[1], Tf[ta][1]);
        mma(au, Tf[ta][1], Yv[1]);
      }
      const int t = 16 * ta + l16;
      if (cbi == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) wk[ta][r] = aw[r];
      } else if (t < L) {
        const float x[8] = {wk[ta][0], wk[ta][1], wk[ta][2], wk[ta][3],
                            aw[0], aw[1], aw[2], aw[3]};
        store8(w_out + ((size_t)(p.t0 + t) * hv + h) * D + packed_index(32 * wv + 4 * gq), x);
      }
      // u_t[c][h][v][packed t]: rows t = 16 ta + 4 gq + r of column `row` (zero past L)
      if (ta & 1) {
        const float x[8] = {uk[0], uk[1], uk[2], uk[3], au[0], au[1], au[2], au[3]};
        store8(u_t + (((size_t)c * hv + h) * D + row) * C + packed_index(16 * (ta - 1) + 4 * gq),
               x);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) uk[r] = au[r];
      }
    }
  }
  lds_barrier();  // the next item rewrites every region
  item = nitem;
  p = np;
  ok = nok;
  }
}

// ----------------------------------------------------------------------- walk

// The inter-chunk walk fused with the output projection.  One workgroup of NW
// waves per (sequence, value head [, chunk group], block of 16 NW columns);
// each wave owns 16 columns of the state and keeps its 128 x 16 slice in MFMA
// accumulators (fp32) through the chunks.  The K-side tiles of a chunk (w,
// qg, aqk, kg_t, the block's u_t rows, decay) arrive by LDS DMA into a
// two-stage ring (one stage for fp32 operands), so the next chunk's tiles
// stream in while this chunk's products run.
//
// MODE 0: the whole sequence, outputs and final state.
// MODE 1: group pass one.  Group g of the sequence's chunks is walked from
//         zero; the first nvb column blocks are the 128 value columns (with
//         u: the group's partial state B_g), the next nvb blocks are 128
//         transfer columns started at the identity with u = 0 (the group
//         transfer P_g = prod_c (diag(d_c) - kg_c^T w_c)).  No outputs.  The
//         last group is left out: no later group starts from its transfer.
// MODE 2: group pass two.  Group g is walked from its composed start state
//         H_in(g); outputs for its tokens, the final state from the group
//         that holds the sequence's last chunk.
//
// With LW > 0 the workgroup carries LW loader waves besides the NW compute
// waves (on SIMDs the compute waves leave idle).  The loaders issue every
// DMA of the ring, so the compute waves issue no loads at all, and they
// also warm the L2 with the K-side lines of the chunk after next: a chunk
// step is bound by how fast a CU can pull its ~60 KB of tiles, which is
// far faster from L2 than from HBM.  Both roles pass the same single
// barrier per chunk.
template <typename E, int NW, int MODE, int LW = 0>
__global__ __launch_bounds__(64 * (NW + LW)) void walk_kernel(const WalkArgs<E> a) {
  constexpr bool SPLIT = std::is_same<E, float>::value;
  constexpr int STAGES = SPLIT ? 1 : 2;
  constexpr bool OUT = MODE != 1;
  constexpr int NT = 64 * NW;
  constexpr int BV = 16 * NW;
  constexpr int EPP = 16 / (int)sizeof(E);  // elements per 16-byte piece
  constexpr int P128 = D / EPP, P64 = C / EPP;
  // (qg and aqk only feed the outputs: pass one's stages leave them out)
  constexpr int OFF_W = 0, OFF_Q = OFF_W + C * P128, OFF_A = OFF_Q + (OUT ? C * P128 : 0);
  constexpr int OFF_K = OFF_A + (OUT ? C * P64 : 0), OFF_U = OFF_K + D * P64;
  constexpr int OFF_D = OFF_U + BV * P64;
  constexpr int STAGE = OFF_D + 64;
  // two distinct arrays (not one indexed ring) so that the compiler can tell
  // the stage being filled from the stage being read
  __shared__ uint4 smemA[STAGE];
  __shared__ uint4 smemB[STAGES == 2 ? STAGE : 1];

  // The column blocks of one (sequence, head, group) get ids with equal
  // id % 8, so they land on one XCD and share its L2 for the K-side tiles.
  const int G = MODE == 0 ? 1 : a.groups;
  const int ncb = MODE == 1 ? 2 * a.nvb : a.nvb;
  const int id = blockIdx.x;
  const int blk = id / (8 * ncb), rem = id - blk * 8 * ncb;
  const int cb = rem >> 3, ug = blk * 8 + (rem & 7);
  // pass one leaves out the last group: compose never reads its transfer
  const int GW = MODE == 1 ? G - 1 : G;  // groups this launch walks
  if (ug >= a.units * GW) return;
  const int unit = ug / GW, g = ug - unit * GW;
  const int hv = a.hv;
  // (sequence, head) in longest-first order: unit / hv indexes the order
  const int n = a.order[unit / hv], h = unit - (unit / hv) * hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // transfer columns of pass one (fp32 operands: a workgroup of their own)
  const bool tcols = MODE == 1 && cb >= a.nvb;
  const int vb = tcols ? cb - a.nvb : cb;
  static_assert(LW == 0 || STAGES == 2, "loader waves serve the two-stage ring");
  const bool loader = LW > 0 && wave >= NW;  // wave-uniform role
  constexpr int DW = LW > 0 ? LW : NW;         // waves that issue the DMA
  const int dwave = LW > 0 ? wave - NW : wave;
  const int l16 = lane & 15, gq = lane >> 4;
  const int v0 = vb * BV;                  // first column of the block
  const int vl = 16 * wave + l16;  // this lane's column in the block
  const int vcol = v0 + vl;
  const SeqSpan sp = seq_span(a.cu, n, a.dense_len, a.T);

  // this workgroup's chunks: group g of the sequence's chunk chain
  const int c_first = a.offs[n];
  // a malformed cu_seqlens could claim chunks past the bound; never read them
  const int nch_all = max(0, min(a.offs[n + 1], a.max_chunks) - c_first);
  const int cpg = MODE == 0 ? max(1, nch_all) : group_chunks(a.nch_max, G);
  const int jc0 = min(nch_all, g * cpg), jc1 = min(nch_all, jc0 + cpg);
  // Groups past the one holding the sequence's last chunk are empty: pass
  // one writes nothing for them (compose stops at that group), pass two has
  // neither tokens nor the final state to write.  (Group 0 of an empty
  // sequence is that group: its pass two writes the final state.)
  const int g_last = nch_all > 0 ? (nch_all - 1) / cpg : 0;
  if (MODE == 1 && jc0 >= jc1) return;
  if (MODE == 2 && g > g_last) return;

  void* row = nullptr;  // paged pool plane of this (sequence, head)
  if (a.cache) {
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.num_slots) {
      // null slot: zero output rows, no state traffic
      if (OUT && !loader) {
        const int tb = sp.bos + C * jc0, te = min(sp.eos, sp.bos + C * jc1);
        for (int idx = tid; idx < (te - tb) * BV; idx += NT) {
          const int t = idx / BV, vv = idx - t * BV;
          const size_t o = ((size_t)(tb + t) * hv + h) * D + v0 + vv;
          if (a.out16)
            a.out16[o] = (_Float16)0.f;
          else
            a.out[o] = from_f32<E>(0.f);
        }
      }
      return;
    }
    row = pool_plane(a.cache, a.slot_stride, slot, h, a.state_bf16 != 0);
  }
  // state in (src) and out (dst): fp32, or bf16 (dense states or the pool)
  const bool state_bf = a.state_bf16 != 0;
  const void* src = nullptr;
  void* dst = nullptr;
  bool src_bf = false, dst_bf = false;
  const size_t unit_plane = (size_t)n * hv + h;
  if (MODE == 0) {
    src = a.cache ? (a.has_init[n] ? row : nullptr)
                  : (a.init ? dense_plane(a.init, unit_plane, state_bf) : nullptr);
    dst = a.cache ? row : (a.fin ? dense_plane(a.fin, unit_plane, state_bf) : nullptr);
    src_bf = dst_bf = state_bf;
  } else if (MODE == 1) {
    dst = scan_plane(a.scan, g, n, h, a.N, hv, tcols ? 0 : 1);
  } else {
    src = scan_plane(a.scan, g, n, h, a.N, hv, 2);
    // the group holding the sequence's last chunk writes the final state
    // (group 0 for an empty sequence: its start state is an exact copy), so
    // the final state is the walk's own, as is a checkpoint at the end
    if (g == g_last) {
      dst = a.cache ? row : (a.fin ? dense_plane(a.fin, unit_plane, state_bf) : nullptr);
      dst_bf = state_bf;
    }
  }

  if (loader) {  // loader waves hold no state columns
    src = nullptr;
    dst = nullptr;
  }

  // mid-prefill snapshot: the step after which it is taken (-1: none).  Pass
  // one of the group scan walks from zero, so only modes 0 and 2 take it.
  int ck_step = -1;
  float* ck_dst = nullptr;
  if (MODE != 1 && a.ckpt && !loader) {
    const int off = a.ckpt_off[n];
    const int row = a.ckpt_idx ? a.ckpt_idx[n] : n;
    if (off > 0 && off % C == 0 && off <= sp.eos - sp.bos && row >= 0 && row < a.ckpt_rows) {
      ck_step = off / C - 1;
      ck_dst = a.ckpt + ((size_t)row * hv + h) * PLANE;
    }
  }

  // state slice: S[kb][r] = S[k = 16 kb + 4 gq + r][column vcol]  (V-first row vcol)
  f32x4_t S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    if (tcols) {
      const int k0 = 16 * kb + 4 * gq;
      S[kb] = f32x4_t{k0 == vcol ? 1.f : 0.f, k0 + 1 == vcol ? 1.f : 0.f,
                      k0 + 2 == vcol ? 1.f : 0.f, k0 + 3 == vcol ? 1.f : 0.f};
    } else if (src) {
      S[kb] = plane_load4(src, (size_t)vcol * D + 16 * kb + 4 * gq, src_bf);
    } else {
      S[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  const uint4* zero = a.zero;
  // K-side tiles of chunk jc into a stage, in two parts: w (and qg), then
  // aqk, kg_t, the block's u_t rows and decay.
  auto issue_wq = [&](int jc, uint4* base) {
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    const size_t rowb = (size_t)hv * D * sizeof(E);
    dma_tile<C, P128, DW, true>(base + OFF_W, a.w + ((size_t)t0 * hv + h) * D, rowb, L, zero,
                                dwave, lane);
    if constexpr (OUT)
      dma_tile<C, P128, DW, true>(base + OFF_Q, a.qg + ((size_t)t0 * hv + h) * D, rowb, L, zero,
                                  dwave, lane);
  };
  auto issue_rest = [&](int jc, uint4* base) {
    const int c = c_first + jc;
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    if constexpr (OUT)
      dma_tile<C, P64, DW, true>(base + OFF_A, a.aqk + ((size_t)t0 * hv + h) * C,
                                 (size_t)hv * C * sizeof(E), L, zero, dwave, lane);
    dma_tile<D, P64, DW, false>(base + OFF_K, a.kg_t + ((size_t)c * hv + h) * D * C,
                                C * sizeof(E), D, zero, dwave, lane);
    if (!tcols)
      dma_tile<BV, P64, DW, false>(base + OFF_U, a.u_t + (((size_t)c * hv + h) * D + v0) * C,
                                   C * sizeof(E), BV, zero, dwave, lane);
    if (dwave == DW - 1) {
      // decay: 32 pieces, lanes 32..63 fill the pad from the zero page
      const char* gp = lane < 32 ? (const char*)(a.decay + ((size_t)c * hv + h) * D) + 16 * lane
                                 : (const char*)zero;
      __builtin_amdgcn_global_load_lds(gp, (lds_vptr)(base + OFF_D), 16, 0, 0);
    }
  };
  if constexpr (LW > 0) {
    if (loader) {
      const size_t rowb = (size_t)hv * D * sizeof(E), rowa = (size_t)hv * C * sizeof(E);
      // Register sets of the ring fetch: this wave's pieces of one chunk's tiles.
      constexpr int PW = C * P128 / 64 / LW, PA = C * P64 / 64 / LW;
      constexpr int PK = D * P64 / 64 / LW, PU = BV * P64 / 64 / LW;
      struct Regs {
        u32x4_t w[PW], q[PW], a[PA], k[PK], u[PU], d;
      };
      const uint32_t offW = tile_off0<P128, LW>(rowb, dwave, lane);
      const uint32_t offA = tile_off0<P64, LW>(rowa, dwave, lane);
      const uint32_t offK = tile_off0<P64, LW>(C * sizeof(E), dwave, lane);
      // Every load is issued on every path (u_t and decay by both waves,
      // rows of a short chunk from the zero page), so each wave's load count
      // per chunk is fixed and the compiler's waits stay exact.
      auto fetch = [&](int jc, Regs& R) __attribute__((always_inline)) {
        const int c = c_first + jc;
        const int t0 = sp.bos + C * jc;
        const int L = min(C, sp.eos - t0);
        const E* wsrc = a.w + ((size_t)t0 * hv + h) * D;
        const E* qsrc = a.qg + ((size_t)t0 * hv + h) * D;
        const E* asrc = a.aqk + ((size_t)t0 * hv + h) * C;
        // (qg and aqk only feed the outputs: pass one of the scan skips them)
        if (L == C) {
          tile_fetch_full<C, P128, LW>(R.w, wsrc, rowb, offW);
          if (OUT) {
            tile_fetch_full<C, P128, LW>(R.q, qsrc, rowb, offW);
            tile_fetch_full<C, P64, LW>(R.a, asrc, rowa, offA);
          }
        } else {  // the last chunk of a sequence: rows past L come from the zero page
          tile_fetch<C, P128, LW, true>(R.w, wsrc, rowb, L, zero, dwave, lane);
          if (OUT) {
            tile_fetch<C, P128, LW, true>(R.q, qsrc, rowb, L, zero, dwave, lane);
            tile_fetch<C, P64, LW, true>(R.a, asrc, rowa, L, zero, dwave, lane);
          }
        }
        tile_fetch_full<D, P64, LW>(R.k, a.kg_t + ((size_t)c * hv + h) * D * C, C * sizeof(E),
                                    offK);
        tile_fetch_full<BV, P64, LW>(R.u, a.u_t + (((size_t)c * hv + h) * D + v0) * C,
                                     C * sizeof(E), offK);
        // decay: 32 pieces, lanes 32..63 fill the pad from the zero page
        const char* gp = lane < 32
                             ? (const char*)(a.decay + ((size_t)c * hv + h) * D) + 16 * lane
                             : (const char*)zero;
        R.d = *reinterpret_cast<const u32x4_t*>(gp);
      };
      auto put = [&](uint4* base, const Regs& R) __attribute__((always_inline)) {
        tile_put<C, P128, LW>(base + OFF_W, R.w, dwave, lane);
        if (OUT) {
          tile_put<C, P128, LW>(base + OFF_Q, R.q, dwave, lane);
          tile_put<C, P64, LW>(base + OFF_A, R.a, dwave, lane);
        }
        tile_put<D, P64, LW>(base + OFF_K, R.k, dwave, lane);
        if (!tcols) tile_put<BV, P64, LW>(base + OFF_U, R.u, dwave, lane);
        if (dwave == LW - 1) *reinterpret_cast<u32x4_t*>(base + OFF_D + lane) = R.d;
      };
      // L2 warm-up.  The column-block workgroups of a (sequence, head) share
      // one XCD's L2 and read the same K-side tiles; each touches its share
      // of their 128-byte lines (and its own u_t lines) of the chunk after
      // next, so the next step's fetch finds them in L2.  One word per line.
      static_assert((NW == 2 || NW == 4) && LW == 2 && sizeof(E) == 2,
                    "warm-up line map: bf16, 32 or 64 columns");
      constexpr int LW_ = 128, LQ = 128, LA = 64, LK = 128, LD = 4;  // lines per tile
      constexpr int NSH = LW_ + LQ + LA + LK + LD;                    // shared lines
      constexpr int LU = BV * C * 2 / 128;                            // own u_t lines
      constexpr int NVB = 8 / NW;                                     // workgroups sharing
      constexpr int PER = (NSH + NVB - 1) / NVB;                      // shared lines each
      constexpr int KW = (PER + LU + 64 * LW - 1) / (64 * LW);        // loads per wave
      const int per = PER;
      auto warm = [&](int jw, uint32_t (&W)[KW]) __attribute__((always_inline)) {
        const int c = c_first + jw;
        const int t0 = sp.bos + C * jw;
        const int L = min(C, sp.eos - t0);
        const char* wb = (const char*)(a.w + ((size_t)t0 * hv + h) * D);
        const char* qb = (const char*)(a.qg + ((size_t)t0 * hv + h) * D);
        const char* ab = (const char*)(a.aqk + ((size_t)t0 * hv + h) * C);
        const char* kb = (const char*)(a.kg_t + ((size_t)c * hv + h) * D * C);
        const char* db = (const char*)(a.decay + ((size_t)c * hv + h) * D);
        const char* ub = (const char*)(a.u_t + (((size_t)c * hv + h) * D + v0) * C);
        // the lane's line indices from an opaque copy of the lane id: hoisted
        // out of the loop, the per-branch line addresses would stay live
        // across it (and spill)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < KW; ++k) {
          const int f = 64 * LW * k + 64 * dwave + ln;
          const char* p = nullptr;
          if (f < per) {
            const int i = vb * per + f;
            if (i < LW_) {
              if ((i >> 1) < L) p = wb + (size_t)(i >> 1) * rowb + 128 * (i & 1);
            } else if (i < LW_ + LQ) {
              const int j = i - LW_;
              if (OUT && (j >> 1) < L) p = qb + (size_t)(j >> 1) * rowb + 128 * (j & 1);
            } else if (i < LW_ + LQ + LA) {
              const int r = i - LW_ - LQ;
              if (OUT && r < L) p = ab + (size_t)r * rowa;
            } else if (i < LW_ + LQ + LA + LK) {
              p = kb + 128 * (i - LW_ - LQ - LA);
            } else if (i < NSH) {
              p = db + 128 * (i - LW_ - LQ - LA - LK);
            }
          } else if (f < per + LU) {
            p = ub + 128 * (f - per);
          }
          // idle lanes read the zero page: every lane loads, on every path
          W[k] = *reinterpret_cast<const uint32_t*>(p ? p : (const char*)zero);
        }
      };
      // The warm-up words are consumed (by an empty asm) a step later, after
      // that step's fetch is issued, so the wait for them leaves it in flight.
      auto sink = [&](const uint32_t (&W)[KW]) __attribute__((always_inline)) {
        uint32_t x = 0;
#pragma unroll
        for (int k = 0; k < KW; ++k) x += W[k];
        asm volatile("" ::"v"(x));
      };
      // The loader loop: one barrier per chunk, as in the compute loop.  After
      // the barrier of chunk jc the stage of chunk jc - 1 is free: the loaders
      // request chunk jc + 1 into registers, warm chunk jc + 2, and write the
      // registers into the free stage once they land (from L2, thanks to the
      // warm-up a step earlier).  The barrier follows the loaders' LDS writes
      // (lgkmcnt(0)); no release fence, which would also wait for the
      // warm-up loads, and asm clobbers keep the compiler from moving memory
      // accesses across it.
      if (jc0 >= jc1) return;
      auto cl = [&](int j) { return min(j, jc1 - 1); };
      Regs R;
      uint32_t W[KW];
      fetch(jc0, R);
      warm(cl(jc0 + 1), W);
      put(smemA, R);
      for (int jc = jc0; jc < jc1; ++jc) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's stage writes are done
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (jc + 1 < jc1) {
          fetch(jc + 1, R);
          sink(W);
          warm(cl(jc + 2), W);
          put(((jc + 1 - jc0) & 1) ? smemB : smemA, R);
        }
      }
      sink(W);
      __builtin_amdgcn_s_waitcnt(0);  // no DMA in flight when the wave ends
      return;
    }
  }
  if (LW == 0 && jc0 < jc1) {
    issue_wq(jc0, smemA);
    issue_rest(jc0, smemA);
  }

  auto body = [&](int jc, uint4* cur, uint4* nxt) {
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    if (LW == 0) __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA of chunk jc has landed
    lds_barrier();  // ... and every other wave's (loaders: their LDS writes)
    const bool more = LW == 0 && STAGES == 2 && jc + 1 < jc1;
    // Eight-wave walks (one workgroup per chain, HBM-bound): the whole next
    // chunk's DMA goes out at the top of the step, for the most lead time.
    constexpr bool EARLY = NW >= 8 && STAGES == 2 && LW == 0;
    if (EARLY && more) {
      issue_wq(jc + 1, nxt);
      issue_rest(jc + 1, nxt);
    }
    const uint4* tW = cur + OFF_W;
    const uint4* tQ = cur + OFF_Q;
    const uint4* tA = cur + OFF_A;
    const uint4* tK = cur + OFF_K;
    const uint4* tU = cur + OFF_U;
    const float* sD = reinterpret_cast<const float*>(cur + OFF_D);

    // the state as an MFMA operand (K = key channel, perm32 order)
    Frag<SPLIT> Hf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                    S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
      Hf[s] = make_frag<SPLIT>(x);
    }
    // u values of this lane's column (zero for transfer columns)
    float uv[2][8];
    if (!tcols) {
      unit_vals<P64>(tU, vl, gq, SPLIT, uv[0]);
      unit_vals<P64>(tU, vl, 4 + gq, SPLIT, uv[1]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) uv[0][e] = uv[1][e] = 0.f;
    }

    // HW = w S (rows t, cols v) and O^T = (qg S)^T (rows v, cols t)
    f32x4_t HW[4], O[4];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta) {
      HW[ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      O[ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (!SPLIT) {
      FragB fw[2][4], fq[2][4];
      auto load_k = [&](int s, int buf) {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          fw[buf][ta] = frag_bf16<P128>(tW, 16 * ta + l16, 4 * s + gq);
          if (OUT) fq[buf][ta] = frag_bf16<P128>(tQ, 16 * ta + l16, 4 * s + gq);
        }
      };
      // The next chunk's w / qg DMA is spread over the K steps, so the wave
      // keeps issuing products while the memory pipeline takes it.
      constexpr int WQ_PER = C * P128 / 64 / NW;
      constexpr int NDMA = OUT ? 2 * WQ_PER : WQ_PER;
      const int tn = sp.bos + C * (jc + 1);
      const int Ln = min(C, sp.eos - tn);
      const size_t rowb = (size_t)hv * D * sizeof(E);
      const E* wsrc = a.w + ((size_t)tn * hv + h) * D;
      const E* qsrc = a.qg + ((size_t)tn * hv + h) * D;
      load_k(0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) load_k(s + 1, (s + 1) & 1);
        if (more && !EARLY) {
#pragma unroll
          for (int m = 0; m < (NDMA + 3) / 4; ++m) {
            const int mm = ((NDMA + 3) / 4) * s + m;
            if (mm < WQ_PER)
              dma_one<C, P128, NW, true>(mm, nxt + OFF_W, wsrc, rowb, Ln, zero, wave, lane);
            else if (mm < NDMA)
              dma_one<C, P128, NW, true>(mm - WQ_PER, nxt + OFF_Q, qsrc, rowb, Ln, zero, wave,
                                         lane);
          }
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          mma(HW[ta], fw[s & 1][ta], Hf[s]);
          if (OUT) mma(O[ta], Hf[s], fq[s & 1][ta]);
        }
      }
      // Pin the schedule: the fragment reads of a K step go out while the
      // products of the previous step run.
      constexpr int NF = OUT ? 8 : 4;
      __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // DS read
#pragma unroll
      for (int i = 0; i < 3 * NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          mma(HW[ta], frag_f32<P128>(tW, 16 * ta + l16, 4 * s + gq), Hf[s]);
          if (OUT) mma(O[ta], Hf[s], frag_f32<P128>(tQ, 16 * ta + l16, 4 * s + gq));
        }
    }
    if (more && !EARLY) issue_rest(jc + 1, nxt);
    // U = u - w S  (C layout: col v, rows t = 16 ta + 4 gq + r)
    Frag<SPLIT> Uf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float x[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = uv[s2][r] - HW[2 * s2][r];
        x[4 + r] = uv[s2][4 + r] - HW[2 * s2 + 1][r];
      }
      Uf[s2] = make_frag<SPLIT>(x);
    }
    if constexpr (!SPLIT) {
      // Every A_qk and kg^T fragment and the decay of this lane's state rows
      // are read up front (A_qk is lower: t < 32 needs i < 32 only); the
      // schedule is pinned so the reads go out together and the products
      // follow as they land, instead of each product waiting on its own read.
      FragB fa[4][2], fk[8][2];
      float4 dk[8];
      if (OUT) {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            if (!(s2 == 1 && ta < 2)) fa[ta][s2] = frag_bf16<P64>(tA, 16 * ta + l16, 4 * s2 + gq);
      }
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) fk[kb][s2] = frag_bf16<P64>(tK, 16 * kb + l16, 4 * s2 + gq);
        dk[kb] = *reinterpret_cast<const float4*>(sD + 16 * kb + 4 * gq);
      }
      // O^T += U^T A_qk^T
      if (OUT) {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          mma(O[ta], Uf[0], fa[ta][0]);
          if (ta >= 2) mma(O[ta], Uf[1], fa[ta][1]);
        }
      }
      // S <- diag(d) S + kg^T U   (rows k, cols v, K = t)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        S[kb][0] *= dk[kb].x;
        S[kb][1] *= dk[kb].y;
        S[kb][2] *= dk[kb].z;
        S[kb][3] *= dk[kb].w;
        mma(S[kb], fk[kb][0], Uf[0]);
        mma(S[kb], fk[kb][1], Uf[1]);
      }
      constexpr int NFA = OUT ? 6 : 0;
      __builtin_amdgcn_sched_group_barrier(0x100, NFA + 24, 0);  // DS reads
      if (OUT) __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);  // A_qk U
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // decay
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // kg^T U
      }
    } else {
      if (OUT) {
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          mma(O[ta], Uf[0], frag_f32<P64>(tA, 16 * ta + l16, gq));
          if (ta >= 2) mma(O[ta], Uf[1], frag_f32<P64>(tA, 16 * ta + l16, 4 + gq));
        }
      }
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const float4 d4 = *reinterpret_cast<const float4*>(sD + 16 * kb + 4 * gq);
        S[kb][0] *= d4.x;
        S[kb][1] *= d4.y;
        S[kb][2] *= d4.z;
        S[kb][3] *= d4.w;
        mma(S[kb], frag_f32<P64>(tK, 16 * kb + l16, gq), Uf[0]);
        mma(S[kb], frag_f32<P64>(tK, 16 * kb + l16, 4 + gq), Uf[1]);
      }
    }
    if (OUT) {
      // rows t = 16 ta + l16 of this lane's 4 output columns
      const size_t ob = ((size_t)(t0 + l16) * hv + h) * D + v0 + 16 * wave + 4 * gq;
      const size_t tstep = (size_t)16 * hv * D;
      auto put = [&](auto* op) {
        if (L == C) {
#pragma unroll
          for (int ta = 0; ta < 4; ++ta)
            store4(op + ta * tstep, a.scale * O[ta][0], a.scale * O[ta][1], a.scale * O[ta][2],
                   a.scale * O[ta][3]);
        } else {
#pragma unroll
          for (int ta = 0; ta < 4; ++ta)
            if (16 * ta + l16 < L)
              store4(op + ta * tstep, a.scale * O[ta][0], a.scale * O[ta][1],
                     a.scale * O[ta][2], a.scale * O[ta][3]);
        }
      };
      if constexpr (std::is_same<E, float>::value) {
        if (a.out16)
          put(a.out16 + ob);
        else
          put(a.out + ob);
      } else {
        put(a.out + ob);
      }
    }
    if (jc == ck_step) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        *reinterpret_cast<float4*>(ck_dst + (size_t)vcol * D + 16 * kb + 4 * gq) =
            make_float4(S[kb][0], S[kb][1], S[kb][2], S[kb][3]);
    }
    if (STAGES == 1 && jc + 1 < jc1) {
      lds_barrier();  // everyone is done with the single stage
      issue_wq(jc + 1, cur);
      issue_rest(jc + 1, cur);
    }
  };
  for (int jc = jc0; jc < jc1; jc += 2) {
    body(jc, smemA, smemB);
    if (jc + 1 < jc1) body(jc + 1, STAGES == 2 ? smemB : smemA, smemA);
  }
  if (dst) {
    if (tcols) {
      // transfer P[k][j] row-major, j = this lane's column (scan plane, fp32)
      float* pd = reinterpret_cast<float*>(dst);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) pd[(size_t)(16 * kb + 4 * gq + r) * D + vcol] = S[kb][r];
    } else {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        plane_store4(dst, (size_t)vcol * D + 16 * kb + 4 * gq, dst_bf, S[kb]);
    }
  }
}

// Group pass one with bf16 operands: one workgroup of eight waves per
// (group, sequence, head) for every group but the last.  Waves 0-3 carry the
// 128 value columns (walked from zero with u: the group's partial state B_g),
// waves 4-7 the 128 transfer columns (from the identity with u = 0: the
// transfer P_g).  Each wave holds two 16-column blocks of the state, so every
// w and kg_t fragment it reads from LDS feeds two products: a chunk step
// reads the shared tiles 8 times from LDS where sixteen waves of one block
// each read them 16 times, and LDS bandwidth is what bounds this pure read
// stream.  The K-side tiles (w, kg_t, the 128 u_t rows, decay) arrive by LDS
// DMA into a two-stage ring; the next chunk's DMA goes out at the top of each
// step.
template <typename E>
__global__ __launch_bounds__(512) void pass_one_kernel(const WalkArgs<E> a) {
  static_assert(!std::is_same<E, float>::value, "bf16 operands");
  constexpr int NW = 8;
  constexpr int EPP = 16 / (int)sizeof(E);
  constexpr int P128 = D / EPP, P64 = C / EPP;
  constexpr int OFF_W = 0, OFF_K = OFF_W + C * P128, OFF_U = OFF_K + D * P64;
  constexpr int OFF_D = OFF_U + D * P64, STAGE = OFF_D + 64;
  __shared__ uint4 smemA[STAGE];
  __shared__ uint4 smemB[STAGE];

  const int G = a.groups, GW = G - 1;  // the last group is not walked
  const int ug = blockIdx.x;
  if (ug >= a.units * GW) return;
  const int unit = ug / GW, g = ug - unit * GW;
  const int hv = a.hv;
  // (sequence, head) in longest-first order: unit / hv indexes the order
  const int n = a.order[unit / hv], h = unit - (unit / hv) * hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool tcols = wave >= 4;
  const int l16 = lane & 15, gq = lane >> 4;
  const int col0 = 32 * (wave & 3) + l16;  // this lane's columns: col0 and col0 + 16
  const SeqSpan sp = seq_span(a.cu, n, a.dense_len, a.T);
  const int c_first = a.offs[n];
  const int nch_all = max(0, min(a.offs[n + 1], a.max_chunks) - c_first);
  const int cpg = group_chunks(a.nch_max, G);
  const int jc0 = min(nch_all, g * cpg), jc1 = min(nch_all, jc0 + cpg);
  if (jc0 >= jc1) return;  // an empty group: compose does not read its planes

  // state slices: S[b][kb][r] = S[k = 16 kb + 4 gq + r][column col0 + 16 b]
  f32x4_t S[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const int k0 = 16 * kb + 4 * gq, col = col0 + 16 * b;
      S[b][kb] = tcols ? f32x4_t{k0 == col ? 1.f : 0.f, k0 + 1 == col ? 1.f : 0.f,
                                 k0 + 2 == col ? 1.f : 0.f, k0 + 3 == col ? 1.f : 0.f}
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  const uint4* zero = a.zero;
  auto issue = [&](int jc, uint4* base) {
    const int c = c_first + jc;
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    dma_tile<C, P128, NW, true>(base + OFF_W, a.w + ((size_t)t0 * hv + h) * D,
                                (size_t)hv * D * sizeof(E), L, zero, wave, lane);
    dma_tile<D, P64, NW, false>(base + OFF_K, a.kg_t + ((size_t)c * hv + h) * D * C,
                                C * sizeof(E), D, zero, wave, lane);
    dma_tile<D, P64, NW, false>(base + OFF_U, a.u_t + ((size_t)c * hv + h) * D * C,
                                C * sizeof(E), D, zero, wave, lane);
    if (wave == NW - 1) {
      // decay: 32 pieces, lanes 32..63 fill the pad from the zero page
      const char* gp = lane < 32 ? (const char*)(a.decay + ((size_t)c * hv + h) * D) + 16 * lane
                                 : (const char*)zero;
      __builtin_amdgcn_global_load_lds(gp, (lds_vptr)(base + OFF_D), 16, 0, 0);
    }
  };
  if (jc0 < jc1) issue(jc0, smemA);

  auto body = [&](int jc, const uint4* cur, uint4* nxt) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA of chunk jc has landed
    lds_barrier();                  // ... and every other wave's
    if (jc + 1 < jc1) issue(jc + 1, nxt);
    const uint4* tW = cur + OFF_W;
    const uint4* tK = cur + OFF_K;
    const uint4* tU = cur + OFF_U;
    const float* sD = reinterpret_cast<const float*>(cur + OFF_D);

    // the state blocks as MFMA operands (K = key channel, perm32 order)
    FragB Hf[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float x[8] = {S[b][2 * s][0],     S[b][2 * s][1],     S[b][2 * s][2],
                            S[b][2 * s][3],     S[b][2 * s + 1][0], S[b][2 * s + 1][1],
                            S[b][2 * s + 1][2], S[b][2 * s + 1][3]};
        Hf[b][s] = make_frag<false>(x);
      }
    // HW_b = w S_b (rows t, cols v); each w fragment feeds both blocks
    f32x4_t HW[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) HW[b][ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    FragB fw[2][4];
    auto load_w = [&](int s, int buf) {
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) fw[buf][ta] = frag_bf16<P128>(tW, 16 * ta + l16, 4 * s + gq);
    };
    load_w(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) load_w(s + 1, (s + 1) & 1);
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        mma(HW[0][ta], fw[s & 1][ta], Hf[0][s]);
        mma(HW[1][ta], fw[s & 1][ta], Hf[1][s]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // U_b = u_b - HW_b (C layout: col v, rows t = 16 ta + 4 gq + r); u = 0
    // for the transfer columns
    FragB Uf[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float uv[2][8];
      if (!tcols) {
        unit_vals<P64>(tU, col0 + 16 * b, gq, false, uv[0]);
        unit_vals<P64>(tU, col0 + 16 * b, 4 + gq, false, uv[1]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) uv[0][e] = uv[1][e] = 0.f;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = uv[s2][r] - HW[b][2 * s2][r];
          x[4 + r] = uv[s2][4 + r] - HW[b][2 * s2 + 1][r];
        }
        Uf[b][s2] = make_frag<false>(x);
      }
    }
    // S_b <- diag(d) S_b + kg^T U_b (rows k, cols v, K = t); each kg^T
    // fragment feeds both blocks
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const FragB k0 = frag_bf16<P64>(tK, 16 * kb + l16, gq);
      const FragB k1 = frag_bf16<P64>(tK, 16 * kb + l16, 4 + gq);
      const float4 d4 = *reinterpret_cast<const float4*>(sD + 16 * kb + 4 * gq);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        S[b][kb][0] *= d4.x;
        S[b][kb][1] *= d4.y;
        S[b][kb][2] *= d4.z;
        S[b][kb][3] *= d4.w;
        mma(S[b][kb], k0, Uf[b][0]);
        mma(S[b][kb], k1, Uf[b][1]);
      }
    }
  };
  for (int jc = jc0; jc < jc1; jc += 2) {
    body(jc, smemA, smemB);
    if (jc + 1 < jc1) body(jc + 1, smemB, smemA);
  }
  // transfer: P[k][j] row-major (plane 0); partial state: V-first [v][k] (plane 1)
  float* dst = scan_plane(a.scan, g, n, h, a.N, hv, tcols ? 0 : 1);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int col = col0 + 16 * b;
    if (tcols) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)(16 * kb + 4 * gq + r) * D + col] = S[b][kb][r];
    } else {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        plane_store4(dst, (size_t)col * D + 16 * kb + 4 * gq, false, S[b][kb]);
    }
  }
}

static void mark(const ChunkLaunch& L, int i) {
  if (i < L.num_events && L.events[i]) (void)hipEventRecord((hipEvent_t)L.events[i], (hipStream_t)L.stream);
}

// Loader waves of the walk: the two-wave bf16 walk leaves two SIMDs of the
// CU idle, and two loader waves there take over its DMA.
template <typename E, int NW>
constexpr int walk_loaders() {
  // two- and four-wave bf16 walks; an eight-wave workgroup already fills the
  // SIMDs, and its waves' registers leave no room for two more
  return (!std::is_same<E, float>::value && (NW == 2 || NW == 4)) ? 2 : 0;
}

template <typename E, int NW>
static void launch_walk(const ChunkLaunch& L, const WalkArgs<E>& wa) {
  hipStream_t st = (hipStream_t)L.stream;
  const int nvb = wa.nvb, units = wa.units, G = wa.groups;
  constexpr int LW = walk_loaders<E, NW>();
  const dim3 block(64 * (NW + LW));
  if (G <= 1) {
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * nvb);
    hipLaunchKernelGGL((walk_kernel<E, NW, 0, LW>), dim3(grid), block, 0, st, wa);
    mark(L, 4);
    mark(L, 5);
    mark(L, 6);
    return;
  }
  const int ug = units * G, ug1 = units * (G - 1);  // pass one: all groups but the last
  if constexpr (!std::is_same<E, float>::value) {
    // one eight-wave workgroup per group: value and transfer columns together
    hipLaunchKernelGGL((pass_one_kernel<E>), dim3((unsigned)ug1), dim3(512), 0, st, wa);
  } else {
    hipLaunchKernelGGL((walk_kernel<E, NW, 1, LW>),
                       dim3((unsigned)(((ug1 + 7) / 8) * 8 * 2 * nvb)), block, 0, st, wa);
  }
  mark(L, 4);
  hipLaunchKernelGGL((compose_kernel<E>), dim3((unsigned)(((units + 7) / 8) * 64)), dim3(64), 0,
                     st, wa);
  mark(L, 5);
  hipLaunchKernelGGL((walk_kernel<E, NW, 2, LW>), dim3((unsigned)(((ug + 7) / 8) * 8 * nvb)),
                     block, 0, st, wa);
  mark(L, 6);
}

// The WY kernel; without PREP the prep outputs come from prep_kernel.
template <typename E, bool PREP, bool GATE, typename I>
static void launch_wy(const ChunkLaunch& L, dim3 grid, int items, int* counter) {
  hipLaunchKernelGGL((wy_kernel<E, PREP, GATE, I>), grid, dim3(256), 0, (hipStream_t)L.stream,
                     (const I*)L.q, (const I*)L.k, (const I*)L.v, (const I*)L.g,
                     (const I*)L.beta, (const int4*)L.table, L.hqk, L.hv, L.use_l2, (E*)L.w,
                     (E*)L.u, (E*)L.aqk, PREP ? (E*)L.qg : (E*)nullptr,
                     PREP ? (E*)L.kg_t : (E*)nullptr, PREP ? L.decay : (float*)nullptr, items,
                     counter, L.gate, L.strides);
}

// E: intermediate and MFMA operand type (fp32 operands run as split bf16
// pairs); I: input and output type (fp16 inputs take the fp32 kernels,
// widened exactly on load).
template <typename E, typename I>
static hipError_t launch_staged_t(const ChunkLaunch& L) {
  hipStream_t st = (hipStream_t)L.stream;
  mark(L, 0);
  const int N = L.num_seqs;
  const int T = (int)L.total_tokens;
  const int dense_len = L.cu ? 0 : (N > 0 ? T / N : 0);
  launch_chunk_table(L);
  mark(L, 1);
  if (L.max_chunks > 0 && T > 0) {
    if (!L.fuse_prep)
      hipLaunchKernelGGL((prep_kernel<E, I>), dim3((unsigned)L.max_chunks, L.hqk), dim3(256), 0,
                         st, (const I*)L.q, (const I*)L.k, (const I*)L.g, (const int4*)L.table,
                         L.hqk, L.hv, L.use_l2, (E*)L.qg, (E*)L.kg_t, L.decay, L.gate,
                         L.strides);
    mark(L, 2);
    // persistent WY grid: the resident workgroups (LDS allows two per CU for
    // bf16 tiles, one for fp32)
    const int items = (int)L.max_chunks * L.hv;
    const int resident = cu_count() * (std::is_same<E, float>::value ? 1 : 2);
    const dim3 grid((unsigned)std::max(1, std::min(items, resident)));
    int* wy_counter = reinterpret_cast<int*>((char*)L.zero + 1024);
    if (L.gate.a_log) {
      if (L.fuse_prep)
        launch_wy<E, true, true, I>(L, grid, items, wy_counter);
      else
        launch_wy<E, false, true, I>(L, grid, items, wy_counter);
    } else {
      if (L.fuse_prep)
        launch_wy<E, true, false, I>(L, grid, items, wy_counter);
      else
        launch_wy<E, false, false, I>(L, grid, items, wy_counter);
    }
  } else {
    mark(L, 2);
  }
  mark(L, 3);
  WalkArgs<E> wa;
  wa.qg = (const E*)L.qg; wa.kg_t = (const E*)L.kg_t; wa.w = (const E*)L.w;
  wa.u_t = (const E*)L.u; wa.aqk = (const E*)L.aqk; wa.decay = L.decay;
  wa.cu = L.cu; wa.dense_len = dense_len; wa.T = T; wa.offs = L.chunk_offsets;
  wa.N = N; wa.hv = L.hv; wa.scale = L.scale;
  wa.init = L.init; wa.fin = L.fin; wa.state_bf16 = L.state_bf16;
  wa.cache = L.cache; wa.slot_stride = L.slot_stride; wa.slots = L.slots;
  wa.has_init = L.has_init; wa.num_slots = L.num_slots;
  wa.out = std::is_same<I, _Float16>::value ? nullptr : (E*)L.out;
  wa.out16 = std::is_same<I, _Float16>::value ? (_Float16*)L.out : nullptr;
  wa.units = N * L.hv; wa.max_chunks = (int)L.max_chunks; wa.groups = L.groups;
  wa.scan = L.scan; wa.zero = (const uint4*)L.zero;
  wa.nch_max = reinterpret_cast<const int32_t*>((const char*)L.zero + KDA_NCH_MAX_OFFSET);
  wa.order = L.chunk_offsets + N + 1;
  wa.ckpt = L.ckpt; wa.ckpt_off = L.ckpt_off; wa.ckpt_idx = L.ckpt_idx;
  wa.ckpt_rows = L.ckpt_rows;
  wa.nvb = D / (16 * L.walk_waves);
  switch (L.walk_waves) {
    case 8: launch_walk<E, 8>(L, wa); break;
    case 4: launch_walk<E, 4>(L, wa); break;
    default: launch_walk<E, 2>(L, wa); break;
  }
  return hipGetLastError();
}

int cu_count_host() { return cu_count(); }

void launch_chunk_table(const ChunkLaunch& L) {
  const int N = L.num_seqs;
  const int T = (int)L.total_tokens;
  const int dense_len = L.cu ? 0 : (N > 0 ? T / N : 0);
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, (hipStream_t)L.stream, L.cu, N,
                     dense_len, T, L.chunk_offsets, (int4*)L.table, (int)L.max_chunks,
                     (uint4*)L.zero);
}

hipError_t launch_chunk_staged(const ChunkLaunch& L) {
  switch (L.dtype) {
    case 0: return launch_staged_t<float, float>(L);
    case 1: return launch_staged_t<bf16, bf16>(L);
    default: return launch_staged_t<float, _Float16>(L);
  }
}

}  // namespace kda
