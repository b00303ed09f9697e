// The on-chip KDA chunked forward on gfx950.
//
// One workgroup (4 waves) walks one chain: a (sequence, value head) pair, or
// one chunk group of it under the group scan.  For every 64-token chunk it
// first forms the chunk's intra-chunk operands in LDS from the raw inputs,
// then advances the state, so that nothing but the inputs, the outputs and
// the states crosses HBM.
//
// The chunk step.  With G the inclusive cumulative log2-decay per key channel
// inside the chunk, b = sigmoid(beta), S the K x V state entering the chunk,
//   K2 = kn 2^G,  qg = qn 2^G,  kg = kn 2^(G_last - G),  d = 2^G_last
//   A_kk[t][i] = b_t sum_c kn_t kn_i 2^(G_t - G_i)   (i < t)
//   A_qk[t][i] =     sum_c qn_t kn_i 2^(G_t - G_i)   (i <= t)
//   T' = (I + A_kk)^-1 diag(b)
//   U = T' (v - K2 S)          (the per-token u_t of the recurrence)
//   O = scale (qg S + A_qk U),  S <- diag(d) S + kg^T U.
// This is the chunked (WY) form whose operand set (qg, kg, decay, A_qk and
// the w / u pair, here folded as T' K2 and T' v) the page
// "vllm.models.kimi_k3.amd.ops.kda_chunk" describes for fused_kda_prologue /
// fused_kda_chunk; the chunk boundaries follow its chunk offsets built from
// cu_seqlens, and its group scan (pass one from zero and the identity,
// compose, pass two) is taken over as MODE 1 / compose / MODE 2.
//
// Exponent range: 2^(G_t - G_i) is formed through a reference token in the
// middle of each 16-token block (per-step g in [-5, 0]): inside a block both
// factors stay within 2^58, and across blocks a third factor
// E_ab = 2^(G_ma - G_mb) >= 2^-116 joins them.
//
// Phases of a chunk (five LDS barriers):
//   P0  decode the prefetched rows, L2 norms, cumsum of the gate (one
//       exchange of the 16-token block totals); operand tiles QL, KL, KR for
//       the couplings; K2, kg^T, decay and b for the walk
//   P1  A_kk (fp32, for the inverse) and A_qk (bf16 tile) on MFMA; then qg and
//       v^T are laid down over the dead QL / KL tiles and the next chunk's rows
//       are requested
//   P2  the diagonal 16 x 16 blocks of (I + A_kk)^-1 by substitution, then the
//       blocks below them by columns on fp32 MFMA
//   walk  X = K2 S, O^T = S^T qg^T, Y = v - X, U = T' Y, O^T += U^T A_qk^T,
//         S = diag(d) S + kg^T U; each wave owns 32 state columns (64 in pass
//         one: 32 value and 32 transfer columns) in MFMA accumulators.
#include <string.h>

#include "kda_chunk_common.hpp"

namespace kda {

struct OnchipArgs {
  const bf16 *q, *k, *v, *g, *beta;
  InStrides is;
  GateArgs ga;
  const int32_t* cu;
  int dense_len, T;
  const int32_t* offs;
  int N, hqk, hv, max_chunks, groups, units, use_l2;
  float scale;
  const void* init;  // dense initial / final states: fp32, or bf16 with state_bf16
  void* fin;
  int state_bf16;
  void* cache;  // paged pool: fp32, or bf16 with state_bf16
  int64_t slot_stride;
  const int32_t* slots;
  const uint8_t* has_init;
  int num_slots;
  bf16* out;
  float* scan;  // group planes (g, n, h): P [k][j], B [v][k], H_in [v][k]
  const int32_t* nch_max;  // chunks of the batch's longest sequence (device)
  float* ckpt;
  const int32_t *ckpt_off, *ckpt_idx;
  int ckpt_rows;
  int per_xcd;  // chains per XCD slice of the grid
};

namespace onchip {
// LDS regions (bytes); two workgroups fit a CU.  Lifetimes inside a chunk
// (b1..b5: the five barriers), chosen so that no region is rewritten while
// another wave may still read it:
//   R0  QL (P0 -> P1), then the qg tile (after b3 -> walk)
//   R1  KL, then the K2 tile
//   R2  KR, then the kg^T tile
//   R3  the gate block sums (P0 up to b2), then A_kk in fp32 (P1 -> P2);
//       A_qk in bf16 at RAQ (P1 -> walk); the lower 16 x 16 blocks only
//   R4  the E_ab table (P0 -> P1), then T in fp32 (P2 -> walk); lower blocks
//   RD  decay, RB b, RTT the diagonal blocks of T transposed
// Every write of a chunk's P0 comes after its b1, which every wave reaches
// only after the previous chunk's walk.
constexpr int R0 = 0;
constexpr int R1 = 16384;
constexpr int R2 = 32768;
constexpr int R3 = 49152;
constexpr int RAQ = R3 + 10240;
constexpr int R4 = 65536;
constexpr int RD = R4 + 10240;
constexpr int RB = RD + 512;
constexpr int RTT = RB + 256;  // the diagonal T blocks transposed (P2 -> P2)
constexpr int BYTES = RTT + 4 * 1024;
static_assert(RAQ + 10 * 512 <= R4, "A_qk blocks fit R3");
}  // namespace onchip

// Lower 16 x 16 block (a, b), b <= a, of a packed triangular 64 x 64 matrix.
__device__ __forceinline__ int lblk(int a, int b) { return a * (a + 1) / 2 + b; }

// Swizzled piece slot of the [64 t][16 pieces] coupling tiles (QL, KL, KR):
// the P0 writes (16 pieces of one row) and the P1 fragment reads (16 rows at
// one piece) both spread over the banks.
__device__ __forceinline__ int cslot(int t, int p) { return t * 16 + (p ^ (t & 15)); }

// 8-byte write of 4 bf16 values into half `half` of piece slot `slot`.
__device__ __forceinline__ void put_half(char* tile, int slot, int half, bf16x4_t v) {
  *reinterpret_cast<bf16x4_t*>(tile + 16 * slot + 8 * half) = v;
}
__device__ __forceinline__ bf16x4_t pk4(float a, float b, float c, float d) {
  return bf16x4_t{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
}

// Row t of a [t][128 packed] tile (16 pieces per row) from this thread's 8
// channels 8 j .. 8 j + 7 (two runs of 4 packed positions).
__device__ __forceinline__ void put_row8(char* tile, int t, int j, bf16x4_t lo, bf16x4_t hi) {
  const int base = 32 * (j >> 2);
  const int p0 = base + pack32(8 * (j & 3)), p1 = base + pack32(8 * (j & 3) + 4);
  put_half(tile, swz<16>(t, p0 >> 3), (p0 >> 2) & 1, lo);
  put_half(tile, swz<16>(t, p1 >> 3), (p1 >> 2) & 1, hi);
}

__device__ __forceinline__ void unpack8(const uint4 u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Operands of v_mfma_f32_16x16x16_bf16 (4 values a lane): A lane l holds
// [row l % 16][k = 4 (l / 16) + j], B lane l holds [k = 4 (l / 16) + j][col
// l % 16], C lane l holds [rows 4 (l / 16) + r][col l % 16]; so a C tile is a
// B operand as it stands.  fp32 values are carried as a hi + lo bf16 pair and
// a product takes three MFMAs (lo*hi + hi*lo + hi*hi), about 16 significant
// bits per operand.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
struct Op16 {
  s16x4_t hi, lo;
};
__device__ __forceinline__ Op16 split4(float a, float b, float c, float d) {
  const bf16x4_t h = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  const bf16x4_t l = {(__bf16)(a - (float)h[0]), (__bf16)(b - (float)h[1]),
                      (__bf16)(c - (float)h[2]), (__bf16)(d - (float)h[3])};
  return Op16{__builtin_bit_cast(s16x4_t, h), __builtin_bit_cast(s16x4_t, l)};
}
__device__ __forceinline__ Op16 split4(const float4 v) { return split4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ void mma16(f32x4_t& c, const Op16& a, const Op16& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, c, 0, 0, 0);
}

// Column b of the blocks of T = (I + A)^-1 below the diagonal, A and T held
// as packed lower 16 x 16 blocks (row-major, 16 floats a row), the diagonal
// blocks of T also transposed (tt):
//   T_ab = -T_aa sum_{c = b}^{a-1} A_ac T_cb,   a = b + 1 .. 3.
// The blocks of the column stay in registers as B operands for the next one.
__device__ __forceinline__ void offdiag_column(int b, const float* sA, float* sT, const float* tt,
                                               int lane) {
  const int l16 = lane & 15, gq = lane >> 4;
  Op16 tcol[4];
  tcol[b] = split4(*reinterpret_cast<const float4*>(tt + 256 * b + 16 * l16 + 4 * gq));
#pragma unroll
  for (int ba = 1; ba < 4; ++ba) {
    if (ba <= b) continue;
    f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      if (c < b || c >= ba) continue;
      const Op16 ac = split4(*reinterpret_cast<const float4*>(sA + 256 * lblk(ba, c) + 16 * l16 + 4 * gq));
      mma16(x, ac, tcol[c]);
    }
    const Op16 taa = split4(*reinterpret_cast<const float4*>(sT + 256 * lblk(ba, ba) + 16 * l16 + 4 * gq));
    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
    mma16(y, taa, split4(x[0], x[1], x[2], x[3]));
    float* out = sT + 256 * lblk(ba, b);
#pragma unroll
    for (int r = 0; r < 4; ++r) out[16 * (4 * gq + r) + l16] = -y[r];
    tcol[ba] = split4(-y[0], -y[1], -y[2], -y[3]);
  }
}

// Two workgroups share a CU (LDS and 256 registers per wave allow it), so
// that one's latency-bound phases overlap the other's; pass one carries twice
// the state columns and runs one workgroup per CU.
template <int MODE, bool GATE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == 1 ? 1 : 2))) void
onchip_kernel(
    const OnchipArgs a) {
  using namespace onchip;
  constexpr bool OUT = MODE != 1;
  constexpr int NCT = MODE == 1 ? 4 : 2;  // 16-column tiles per wave
  __shared__ __attribute__((aligned(16))) char smem[BYTES];
  char* tQL = smem + R0;  // QL, then qg
  char* tKL = smem + R1;  // KL, then K2
  char* tKR = smem + R2;  // KR, then kg^T
  float* sP = reinterpret_cast<float*>(smem + R3);  // gate prefix table [4 w][4 row groups][128]
  float* sA = reinterpret_cast<float*>(smem + R3);  // A_kk blocks
  char* tAQ = smem + RAQ;                           // A_qk blocks (bf16)
  float* sE = reinterpret_cast<float*>(smem + R4);  // E_ab table
  float* sT = reinterpret_cast<float*>(smem + R4);  // T blocks
  float* sD = reinterpret_cast<float*>(smem + RD);
  float* sB = reinterpret_cast<float*>(smem + RB);
  float* sTT = reinterpret_cast<float*>(smem + RTT);

  // Chains in XCD-major order: the chains with blockIdx % 8 == x are
  // [x * per_xcd, (x + 1) * per_xcd), so consecutive heads (the value heads of
  // one query/key head among them) share an XCD and its L2.
  const int G = MODE == 0 ? 1 : a.groups;
  const int chain = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
  // pass one leaves out the last group: compose never reads its transfer
  const int GW = MODE == 1 ? G - 1 : G;  // groups this launch walks
  if (chain >= a.units * GW) return;
  const int unit = chain / GW, g = chain - unit * GW;
  const int hv = a.hv;
  const int n = unit / hv, h = unit - n * hv;
  const int hq = h / (hv / a.hqk);
  // Lane-derived indices are rebuilt from an opaque copy of the thread id at
  // the top of every chunk: hoisted out of the loop, the many per-lane LDS
  // and global addresses derived from them would stay live across it.
  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l16 = lane & 15, gq = lane >> 4;
  int rg = tid >> 4, j = tid & 15, r4 = lane >> 4;
  auto refresh_ids = [&]() {
    int t_ = (int)threadIdx.x;
    asm volatile("" : "+v"(t_));
    tid = t_;
    lane = t_ & 63;
    l16 = lane & 15;
    gq = lane >> 4;
    rg = t_ >> 4;
    j = t_ & 15;
    r4 = lane >> 4;
  };
  const SeqSpan sp = seq_span(a.cu, n, a.dense_len, a.T);

  const int c_first = a.offs[n];
  const int nch_all = max(0, min(a.offs[n + 1], a.max_chunks) - c_first);
  const int cpg = MODE == 0 ? max(1, nch_all) : group_chunks(a.nch_max, G);
  const int jc0 = min(nch_all, g * cpg), jc1 = min(nch_all, jc0 + cpg);
  // groups past the one holding the last chunk are empty (see the staged walk)
  const int g_last = nch_all > 0 ? (nch_all - 1) / cpg : 0;
  if (MODE == 1 && jc0 >= jc1) return;
  if (MODE == 2 && g > g_last) return;

  void* row = nullptr;  // paged pool plane of this (sequence, head)
  if (a.cache) {
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.num_slots) {
      // null slot: zero output rows, no state traffic
      if (OUT) {
        const int tb = sp.bos + C * jc0, te = min(sp.eos, sp.bos + C * jc1);
        for (int idx = tid; idx < (te - tb) * D; idx += 256) {
          const int t = idx / D, vv = idx - t * D;
          a.out[((size_t)(tb + t) * hv + h) * D + vv] = from_f32<bf16>(0.f);
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
  } else if (MODE == 2) {
    src = scan_plane(a.scan, g, n, h, a.N, hv, 2);
    if (g == g_last) {
      dst = a.cache ? row : (a.fin ? dense_plane(a.fin, unit_plane, state_bf) : nullptr);
      dst_bf = state_bf;
    }
  }
  int ck_step = -1;
  float* ck_dst = nullptr;
  if (MODE != 1 && a.ckpt) {
    const int off = a.ckpt_off[n];
    const int crow = a.ckpt_idx ? a.ckpt_idx[n] : n;
    if (off > 0 && off % C == 0 && off <= sp.eos - sp.bos && crow >= 0 && crow < a.ckpt_rows) {
      ck_step = off / C - 1;
      ck_dst = a.ckpt + ((size_t)crow * hv + h) * PLANE;
    }
  }

  // State columns of this lane: tile ct holds column col(ct) of S (V-first row
  // col), S[ct][kb][r] = S[k = 16 kb + 4 gq + r][col].  Pass one: tiles 0, 1
  // are value columns (from zero), tiles 2, 3 transfer columns (from I).
  auto col = [&](int ct) { return 32 * wave + 16 * (ct & 1) + l16; };
  f32x4_t S[NCT][8];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const int c = col(ct);
      if (MODE == 1 && ct >= 2) {
        const int k0 = 16 * kb + 4 * gq;
        S[ct][kb] = f32x4_t{k0 == c ? 1.f : 0.f, k0 + 1 == c ? 1.f : 0.f,
                            k0 + 2 == c ? 1.f : 0.f, k0 + 3 == c ? 1.f : 0.f};
      } else if (src) {
        S[ct][kb] = plane_load4(src, (size_t)c * D + 16 * kb + 4 * gq, src_bf);
      } else {
        S[ct][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }

  // gate parameters of this head (constant along the chain)
  float gA = 0.f, gB[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (GATE) {
    gA = exp2_fast(a.ga.a_log[h] * LOG2E);
    gate_bias8(a.ga, h, 8 * j, gB);
  }

  // The next chunk's inputs, fetched during the walk: q, k, g rows (thread
  // (rg, j) takes tokens 4 rg .. 4 rg + 3, channels 8 j .. 8 j + 7), beta of
  // token tid, and v already in the walk's layout (tokens 16 ta + 4 gq + r
  // of this lane's two value columns, packed in pairs of tokens).
  RawRows<bf16> rq, rk, rgt;
  bf16 rb;
  uint32_t vw[4][2][2];
  auto fetch = [&](int jc) {
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    if (OUT) raw_load(a.q + (size_t)t0 * a.is.q + hq * D, (int)a.is.q, L, rq, tid);
    raw_load(a.k + (size_t)t0 * a.is.k + hq * D, (int)a.is.k, L, rk, tid);
    raw_load(a.g + (size_t)t0 * a.is.g + h * D, (int)a.is.g, L, rgt, tid);
    rb = a.beta[(size_t)(t0 + min(tid, L - 1)) * a.is.beta + h];
  };
  auto fetch_v = [&](int jc) {
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    const uint16_t* vb =
        reinterpret_cast<const uint16_t*>(a.v) + (size_t)t0 * a.is.v + h * D + 32 * wave + l16;
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int t = 16 * ta + 4 * gq + 2 * pr;
          const uint32_t lo = vb[(size_t)min(t, L - 1) * a.is.v + 16 * ct];
          const uint32_t hi = vb[(size_t)min(t + 1, L - 1) * a.is.v + 16 * ct];
          vw[ta][ct][pr] = lo | (hi << 16);
        }
  };
  if (jc0 < jc1) fetch(jc0);

  // T fragments (rows t, K = i in perm32 order), shared by every column tile;
  // the blocks above the diagonal are zero.  (b scales Y's rows instead.)
  auto tfrag = [&](int ta, int s2) {
    const int i0 = 4 * gq;
    const float4 t0 = *reinterpret_cast<const float4*>(sT + 256 * lblk(ta, 2 * s2) + 16 * l16 + i0);
    float4 t1 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (2 * s2 + 1 <= ta)
      t1 = *reinterpret_cast<const float4*>(sT + 256 * lblk(ta, 2 * s2 + 1) + 16 * l16 + i0);
    const float x[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    return make_frag<false>(x);
  };
  // A_qk as the B operand of U^T A_qk^T (column t, K = i in perm32 order)
  auto aqfrag = [&](int ta, int s2) {
    const uint2 u0 = *reinterpret_cast<const uint2*>(tAQ + 512 * lblk(ta, 2 * s2) +
                                                     2 * (16 * l16 + 4 * gq));
    uint2 u1 = make_uint2(0u, 0u);
    if (2 * s2 + 1 <= ta)
      u1 = *reinterpret_cast<const uint2*>(tAQ + 512 * lblk(ta, 2 * s2 + 1) +
                                           2 * (16 * l16 + 4 * gq));
    return FragB{__builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y))};
  };

  for (int jc = jc0; jc < jc1; ++jc) {
    refresh_ids();
    const int t0 = sp.bos + C * jc;
    const int L = min(C, sp.eos - t0);
    const int jn = jc + 1 < jc1 ? jc + 1 : jc;  // past the last chunk: this one, unused
    // -------------------------------------------------------------- P0
    bf16x4_t qg_lo[4], qg_hi[4], k2_lo[4], k2_hi[4], kgc[8];
    {
      // the gate: decode, optional activation, inclusive cumsum over tokens
      // (in-thread over 4 tokens, across the 4 row groups of the wave by
      // shuffles, across waves through LDS)
      float Gx[4][8];
      raw_decode(rgt, L, Gx, tid);
      const float braw = to_f32(rb);
      if constexpr (GATE) {
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            Gx[it][e] = 4 * rg + it < L ? gate_apply(Gx[it][e], gA, gB[e], a.ga.lower_bound) : 0.f;
      }
      float excl[8], incl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float run = 0.f;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          run += Gx[it][e] * LOG2E;
          Gx[it][e] = run;
        }
      }
      // across the 4 row groups of the wave: an inclusive scan in two shuffle
      // rounds, all channels in flight together
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = __shfl_up(Gx[3][e], 16);
        incl[e] = Gx[3][e] + (r4 >= 1 ? y : 0.f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = __shfl_up(incl[e], 32);
        incl[e] += r4 >= 2 ? y : 0.f;
      }
      // the prefix through this row group, one table row per (wave, row
      // group): row group 1 ends at token 16 w + 7, row group 3 ends the block
      {
        float* trow = sP + (4 * wave + r4) * D + 8 * j;
        *reinterpret_cast<float4*>(trow) = make_float4(incl[0], incl[1], incl[2], incl[3]);
        *reinterpret_cast<float4*>(trow + 4) = make_float4(incl[4], incl[5], incl[6], incl[7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) excl[e] = incl[e] - Gx[3][e];
      lds_barrier();  // b1: block sums (every wave is also past the last walk)
      float Gl[8], Gm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float before = 0.f, all = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float x = sP[(4 * w2 + 3) * D + 8 * j + e];
          before += w2 < wave ? x : 0.f;
          all += x;
        }
        Gl[e] = all;
#pragma unroll
        for (int it = 0; it < 4; ++it) Gx[it][e] += excl[e] + before;
        Gm[e] = __shfl(Gx[3][e], 16 + j);  // token 16 w + 7
      }
      // E_ab = 2^(G_ma - G_mb) for the 6 pairs b < a (index a (a - 1) / 2 + b)
      float ev[3];
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const int idx = tid + 256 * m, pi = idx >> 7, ch = idx & (D - 1);
        const int aa = pi < 1 ? 1 : (pi < 3 ? 2 : 3), bb = pi - aa * (aa - 1) / 2;
        float ga = sP[(4 * aa + 1) * D + ch], gb = sP[(4 * bb + 1) * D + ch];
#pragma unroll
        for (int w2 = 0; w2 < 3; ++w2) {
          ga += w2 < aa ? sP[(4 * w2 + 3) * D + ch] : 0.f;
          gb += w2 < bb ? sP[(4 * w2 + 3) * D + ch] : 0.f;
        }
        ev[m] = exp2_fast(ga - gb);
      }
      float pm[8], pl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pm[e] = exp2_fast(Gm[e]);          // 2^G = 2^(G - G_m) 2^G_m
        pl[e] = exp2_fast(Gl[e] - Gm[e]);  // 2^(G_last - G) = 2^(G_m - G) 2^(G_last - G_m)
      }
      // q and k one token row at a time: decode, L2 norm, the block-referenced
      // coupling tiles, and the walk's operands (held until the couplings are
      // done with the tiles they replace)
      float kg[4][8];
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int t = 4 * rg + it;
        const bool live = t < L;
        float qr[8], kr[8];
        raw_vals(rk, it, kr);
        if (OUT) {
          raw_vals(rq, it, qr);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qr[e] = 0.f;
        }
        if (L < C) {  // a ragged chunk (uniform): rows past L are zero
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kr[e] = live ? kr[e] : 0.f;
            qr[e] = live ? qr[e] : 0.f;
          }
        }
        if (a.use_l2) {
          float sk = 0.f, sq = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sk += kr[e] * kr[e];
            sq += qr[e] * qr[e];
          }
          const float rk_ = rsq(row_sum16(sk) + L2_EPS);
          const float rq_ = OUT ? rsq(row_sum16(sq) + L2_EPS) : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kr[e] *= rk_;
            qr[e] *= rq_;
          }
        }
        float xq[8], xl[8], xr[8], x2[8], xg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dg = Gx[it][e] - Gm[e];
          const float up = exp2_fast(dg);
          const float dn = exp2_fast(-dg);
          xq[e] = qr[e] * up;
          xl[e] = kr[e] * up;
          xr[e] = kr[e] * dn;
          xg[e] = xq[e] * pm[e];      // qg
          x2[e] = xl[e] * pm[e];      // K2 = kn 2^G
          kg[it][e] = xr[e] * pl[e];  // kn 2^(G_last - G)
        }
        if (OUT) {
          qg_lo[it] = pk4(xg[0], xg[1], xg[2], xg[3]);
          qg_hi[it] = pk4(xg[4], xg[5], xg[6], xg[7]);
          *reinterpret_cast<bf16x8_t*>(tQL + 16 * cslot(t, j)) = pack8(xq);
        }
        k2_lo[it] = pk4(x2[0], x2[1], x2[2], x2[3]);
        k2_hi[it] = pk4(x2[4], x2[5], x2[6], x2[7]);
        *reinterpret_cast<bf16x8_t*>(tKL + 16 * cslot(t, j)) = pack8(xl);
        *reinterpret_cast<bf16x8_t*>(tKR + 16 * cslot(t, j)) = pack8(xr);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) kgc[e] = pk4(kg[0][e], kg[1][e], kg[2][e], kg[3][e]);
      // the block sums are read; E, b and decay go to their own regions
#pragma unroll
      for (int m = 0; m < 3; ++m) sE[tid + 256 * m] = ev[m];
      if (tid < C) sB[tid] = tid < L ? sigmoid(braw) : 0.f;
      if (tid < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sD[8 * j + e] = exp2_fast(Gl[e]);
      }
    }
    lds_barrier();  // b2: coupling tiles, E, b, decay

    // -------------------------------------------------------------- P1
    // Each wave takes a fixed set of (row block, column block) pairs.
    {
      auto pair = [&](const int pa, const int pb) {
        const int t = 16 * pa + l16;
        const int i = 16 * pb + l16;
        const float* eab = sE + (pa * (pa - 1) / 2 + pb) * D;
        f32x4_t acck = {0.f, 0.f, 0.f, 0.f}, accq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int p = 4 * s + gq;
          const uint4 kr = *reinterpret_cast<const uint4*>(tKR + 16 * cslot(i, p));
          FragB R;
          if (pa == pb) {
            R = FragB{__builtin_bit_cast(bf16x8_t, kr)};
          } else {
            float x[8], ef[8];
            unpack8(kr, x);
            const float4 e0 = *reinterpret_cast<const float4*>(eab + 8 * p);
            const float4 e1 = *reinterpret_cast<const float4*>(eab + 8 * p + 4);
            ef[0] = e0.x; ef[1] = e0.y; ef[2] = e0.z; ef[3] = e0.w;
            ef[4] = e1.x; ef[5] = e1.y; ef[6] = e1.z; ef[7] = e1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= ef[e];
            R = make_frag<false>(x);
          }
          const FragB Lk{__builtin_bit_cast(bf16x8_t,
                                            *reinterpret_cast<const uint4*>(tKL + 16 * cslot(t, p)))};
          mma(acck, R, Lk);
          if (OUT) {
            const FragB Lq{__builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4*>(tQL + 16 * cslot(t, p)))};
            mma(accq, R, Lq);
          }
        }
        const int i0 = 4 * gq;  // column inside block pb
        float ak[4], aq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ak[r] = (16 * pb + i0 + r < t) ? acck[r] * sB[t] : 0.f;
          aq[r] = (16 * pb + i0 + r <= t) ? accq[r] : 0.f;
        }
        *reinterpret_cast<float4*>(sA + 256 * lblk(pa, pb) + 16 * l16 + i0) =
            make_float4(ak[0], ak[1], ak[2], ak[3]);
        if (OUT)
          *reinterpret_cast<bf16x4_t*>(tAQ + 512 * lblk(pa, pb) + 2 * (16 * l16 + i0)) =
              pk4(aq[0], aq[1], aq[2], aq[3]);
      };
      if (wave == 0) {
        pair(3, 3); pair(3, 2); pair(3, 1);
      } else if (wave == 1) {
        pair(3, 0); pair(2, 2); pair(2, 1);
      } else if (wave == 2) {
        pair(2, 0); pair(1, 1);
      } else {
        pair(1, 0); pair(0, 0);
      }
    }
    lds_barrier();  // b3: A_kk and A_qk complete; QL, KL, KR and E dead

    // the walk's operand tiles over the dead coupling tiles
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (OUT) put_row8(tQL, 4 * rg + it, j, qg_lo[it], qg_hi[it]);
      put_row8(tKL, 4 * rg + it, j, k2_lo[it], k2_hi[it]);
    }
    {
      const int pp = packed_index(4 * rg);
#pragma unroll
      for (int e = 0; e < 8; ++e) put_half(tKR, tslot<bf16>(8 * j + e, pp >> 3), (pp >> 2) & 1, kgc[e]);
    }

    fetch_v(jc);  // this chunk's v, in the walk's layout

    // -------------------------------------------------------------- P2
    // T = (I + A_kk)^-1; diagonal blocks by substitution (lane = column of
    // the block; row r + 1 of A is read while row r is substituted, and each
    // row's sum runs as four partial sums so that only its last term waits
    // for the row before)
    if (lane < 16) {
      const int ba = wave;
      const float* arow = sA + 256 * lblk(ba, ba);
      float x[16];
      float4 cur[4], nxt[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) cur[q4] = *reinterpret_cast<const float4*>(arow + 4 * q4);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r < 15) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            nxt[q4] = *reinterpret_cast<const float4*>(arow + 16 * (r + 1) + 4 * q4);
        }
        const float av[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y,
                              cur[1].z, cur[1].w, cur[2].x, cur[2].y, cur[2].z, cur[2].w,
                              cur[3].x, cur[3].y, cur[3].z, cur[3].w};
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ii = 0; ii < r; ++ii) ps[ii & 3] += av[ii] * x[ii];
        x[r] = ((r == lane) ? 1.f : 0.f) - ((ps[0] + ps[1]) + (ps[2] + ps[3]));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
      }
      float* trow = sT + 256 * lblk(ba, ba);
#pragma unroll
      for (int r = 0; r < 16; ++r) trow[16 * r + lane] = x[r];
      float* tcol = sTT + 256 * ba + 16 * lane;  // column `lane` as a row
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(tcol + 4 * q4) =
            make_float4(x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    }
    lds_barrier();  // b4: diagonal blocks; the walk's tiles
    // blocks below the diagonal by columns: wave b walks column b downwards
    if (wave == 0) {
      offdiag_column(0, sA, sT, sTT, lane);
    } else if (wave == 1) {
      offdiag_column(1, sA, sT, sTT, lane);
    } else if (wave == 2) {
      offdiag_column(2, sA, sT, sTT, lane);
    }
    lds_barrier();  // b5: T complete

    // ------------------------------------------------------------ walk
    const uint4* uK2 = reinterpret_cast<const uint4*>(tKL);
    const uint4* uQ = reinterpret_cast<const uint4*>(tQL);
    const uint4* uKG = reinterpret_cast<const uint4*>(tKR);
    FragB Tf[4][2];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        if (!(s2 == 1 && ta < 2)) Tf[ta][s2] = tfrag(ta, s2);
    // column tiles in pairs (one pair; two in pass one)
#pragma unroll
    for (int cp = 0; cp < NCT / 2; ++cp) {
      const bool vcols = cp == 0;  // pass one: the second pair is the transfer columns
      FragB Hf[2][4];  // the state as an MFMA operand (K = key channel, perm32)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f32x4_t& lo = S[2 * cp + c2][2 * s];
          const f32x4_t& hi = S[2 * cp + c2][2 * s + 1];
          const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          Hf[c2][s] = make_frag<false>(x);
        }
      // X = K2 S (rows t, cols v)
      f32x4_t X[4][2];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) X[ta][0] = X[ta][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        FragB fk[4];
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) fk[ta] = frag_bf16<16>(uK2, 16 * ta + l16, 4 * s + gq);
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          mma(X[ta][0], fk[ta], Hf[0][s]);
          mma(X[ta][1], fk[ta], Hf[1][s]);
        }
      }
      // U = T diag(b) (v - X) (rows t, cols v), as the operand Uf (K = token,
      // perm32)
      FragB Uf[2][2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        FragB Yf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float x[8];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int ta = 2 * s2 + half;
            const float4 bt = *reinterpret_cast<const float4*>(sB + 16 * ta + 4 * gq);
            const float bb[4] = {bt.x, bt.y, bt.z, bt.w};
            float vv[4] = {0.f, 0.f, 0.f, 0.f};
            if (vcols) {
              const uint32_t p0 = vw[ta][c2][0], p1 = vw[ta][c2][1];
              vv[0] = __uint_as_float(p0 << 16);
              vv[1] = __uint_as_float(p0 & 0xffff0000u);
              vv[2] = __uint_as_float(p1 << 16);
              vv[3] = __uint_as_float(p1 & 0xffff0000u);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * half + r] = bb[r] * (vv[r] - X[ta][c2][r]);
          }
          Yf[s2] = make_frag<false>(x);
        }
        f32x4_t U[4];
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          U[ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          mma(U[ta], Tf[ta][0], Yf[0]);
          if (ta >= 2) mma(U[ta], Tf[ta][1], Yf[1]);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const float x[8] = {U[2 * s2][0], U[2 * s2][1], U[2 * s2][2], U[2 * s2][3],
                              U[2 * s2 + 1][0], U[2 * s2 + 1][1], U[2 * s2 + 1][2],
                              U[2 * s2 + 1][3]};
          Uf[c2][s2] = make_frag<false>(x);
        }
      }
      if (OUT) {
        // O^T = S^T qg^T + U^T A_qk^T (rows v, cols t)
        f32x4_t O[2][4];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int ta = 0; ta < 4; ++ta) O[c2][ta] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          FragB fq[4];
#pragma unroll
          for (int ta = 0; ta < 4; ++ta) fq[ta] = frag_bf16<16>(uQ, 16 * ta + l16, 4 * s + gq);
#pragma unroll
          for (int ta = 0; ta < 4; ++ta) {
            mma(O[0][ta], Hf[0][s], fq[ta]);
            mma(O[1][ta], Hf[1][s], fq[ta]);
          }
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 == 1 && ta < 2) continue;
            const FragB fa = aqfrag(ta, s2);
            mma(O[0][ta], Uf[0][s2], fa);
            mma(O[1][ta], Uf[1][s2], fa);
          }
        // rows t = 16 ta + l16 of this lane's 4 output columns per tile
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          bf16* op = a.out + ((size_t)(t0 + l16) * hv + h) * D + 32 * wave + 16 * c2 + 4 * gq;
          const size_t tstep = (size_t)16 * hv * D;
          if (L == C) {
#pragma unroll
            for (int ta = 0; ta < 4; ++ta)
              store4(op + ta * tstep, a.scale * O[c2][ta][0], a.scale * O[c2][ta][1],
                     a.scale * O[c2][ta][2], a.scale * O[c2][ta][3]);
          } else {
#pragma unroll
            for (int ta = 0; ta < 4; ++ta)
              if (16 * ta + l16 < L)
                store4(op + ta * tstep, a.scale * O[c2][ta][0], a.scale * O[c2][ta][1],
                       a.scale * O[c2][ta][2], a.scale * O[c2][ta][3]);
          }
        }
      }
      // S <- diag(d) S + kg^T U   (rows k, cols v, K = t)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const float4 dk = *reinterpret_cast<const float4*>(sD + 16 * kb + 4 * gq);
        const int r_ = 16 * kb + l16;
        const FragB f0 = FragB{__builtin_bit_cast(bf16x8_t, uKG[tslot<bf16>(r_, gq)])};
        const FragB f1 = FragB{__builtin_bit_cast(bf16x8_t, uKG[tslot<bf16>(r_, 4 + gq)])};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x4_t& st = S[2 * cp + c2][kb];
          st[0] *= dk.x;
          st[1] *= dk.y;
          st[2] *= dk.z;
          st[3] *= dk.w;
          mma(st, f0, Uf[c2][0]);
          mma(st, f1, Uf[c2][1]);
        }
      }
    }
    fetch(jn);  // the next chunk's q, k, g and beta
    if (jc == ck_step) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
          *reinterpret_cast<float4*>(ck_dst + (size_t)col(ct) * D + 16 * kb + 4 * gq) =
              make_float4(S[ct][kb][0], S[ct][kb][1], S[ct][kb][2], S[ct][kb][3]);
    }
  }

  refresh_ids();
  if (MODE == 1) {
    float* pd = scan_plane(a.scan, g, n, h, a.N, hv, 0);  // transfer P [k][j]
    float* bd = scan_plane(a.scan, g, n, h, a.N, hv, 1);  // partial state B [v][k]
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        if (ct >= 2) {
#pragma unroll
          for (int r = 0; r < 4; ++r) pd[(size_t)(16 * kb + 4 * gq + r) * D + col(ct)] = S[ct][kb][r];
        } else {
          plane_store4(bd, (size_t)col(ct) * D + 16 * kb + 4 * gq, false, S[ct][kb]);
        }
      }
  } else if (dst) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        plane_store4(dst, (size_t)col(ct) * D + 16 * kb + 4 * gq, dst_bf, S[ct][kb]);
  }
}

// ------------------------------------------------------------------ launch

static void mark_ev(const ChunkLaunch& L, int i) {
  if (i < L.num_events && L.events[i])
    (void)hipEventRecord((hipEvent_t)L.events[i], (hipStream_t)L.stream);
}

template <bool GATE>
static void launch_onchip_t(const ChunkLaunch& L, const OnchipArgs& oa) {
  hipStream_t st = (hipStream_t)L.stream;
  const int G = oa.groups;
  const int chains = oa.units * (G > 1 ? G : 1);
  OnchipArgs a = oa;
  a.per_xcd = (chains + 7) / 8;
  const dim3 grid((unsigned)(8 * a.per_xcd)), block(256);
  if (G <= 1) {
    hipLaunchKernelGGL((onchip_kernel<0, GATE>), grid, block, 0, st, a);
    mark_ev(L, 4);
    mark_ev(L, 5);
    mark_ev(L, 6);
    return;
  }
  OnchipArgs a1 = a;  // pass one: all groups but the last
  a1.per_xcd = (oa.units * (G - 1) + 7) / 8;
  hipLaunchKernelGGL((onchip_kernel<1, GATE>), dim3((unsigned)(8 * a1.per_xcd)), block, 0, st,
                     a1);
  mark_ev(L, 4);
  WalkArgs<bf16> wa;
  memset(&wa, 0, sizeof(wa));
  wa.cu = L.cu; wa.dense_len = a.dense_len; wa.T = a.T; wa.offs = L.chunk_offsets;
  wa.N = a.N; wa.hv = a.hv; wa.init = L.init; wa.state_bf16 = L.state_bf16;
  wa.cache = L.cache; wa.slot_stride = L.slot_stride; wa.slots = L.slots;
  wa.has_init = L.has_init; wa.num_slots = L.num_slots; wa.units = a.units;
  wa.max_chunks = a.max_chunks; wa.groups = G; wa.scan = L.scan; wa.nch_max = a.nch_max;
  hipLaunchKernelGGL((compose_kernel<bf16>), dim3((unsigned)(((a.units + 7) / 8) * 64)), dim3(64),
                     0, st, wa);
  mark_ev(L, 5);
  hipLaunchKernelGGL((onchip_kernel<2, GATE>), grid, block, 0, st, a);
  mark_ev(L, 6);
}

hipError_t launch_chunk_onchip(const ChunkLaunch& L) {
  mark_ev(L, 0);
  const int N = L.num_seqs;
  const int T = (int)L.total_tokens;
  const int dense_len = L.cu ? 0 : (N > 0 ? T / N : 0);
  launch_chunk_table(L);
  mark_ev(L, 1);
  mark_ev(L, 2);
  mark_ev(L, 3);
  OnchipArgs a;
  memset(&a, 0, sizeof(a));
  a.q = (const bf16*)L.q; a.k = (const bf16*)L.k; a.v = (const bf16*)L.v;
  a.g = (const bf16*)L.g; a.beta = (const bf16*)L.beta;
  a.is = L.strides; a.ga = L.gate;
  a.cu = L.cu; a.dense_len = dense_len; a.T = T; a.offs = L.chunk_offsets;
  a.N = N; a.hqk = L.hqk; a.hv = L.hv; a.max_chunks = (int)L.max_chunks;
  a.groups = L.groups; a.units = N * L.hv; a.use_l2 = L.use_l2; a.scale = L.scale;
  a.init = L.init; a.fin = L.fin; a.state_bf16 = L.state_bf16;
  a.cache = L.cache; a.slot_stride = L.slot_stride; a.slots = L.slots;
  a.has_init = L.has_init; a.num_slots = L.num_slots; a.out = (bf16*)L.out;
  a.scan = L.scan; a.ckpt = L.ckpt; a.ckpt_off = L.ckpt_off; a.ckpt_idx = L.ckpt_idx;
  a.nch_max = reinterpret_cast<const int32_t*>((const char*)L.zero + KDA_NCH_MAX_OFFSET);
  a.ckpt_rows = L.ckpt_rows;
  if (L.gate.a_log)
    launch_onchip_t<true>(L, a);
  else
    launch_onchip_t<false>(L, a);
  return hipGetLastError();
}

}  // namespace kda
