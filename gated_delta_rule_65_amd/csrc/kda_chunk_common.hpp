// Device helpers shared by the chunked-forward kernels (gfx950): sequence
// spans, raw row tiles, fragments, the diagonal-block inverse pieces, state
// planes, the walk arguments and the group-compose kernel.
#pragma once
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"
#include "kda_mfma.hpp"
#include "kda_tiles.hpp"

namespace kda {

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


__device__ __forceinline__ void l2norm_rows4(float (&x)[4][8]) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[it][e] * x[it][e];
    s = row_sum16(s);
    const float r = rsq(s + L2_EPS);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[it][e] *= r;
  }
}


// One off-diagonal block of T = (I + A)^-1 (A strictly lower, 16 x 16 blocks,
// fp32 row-major with row stride SA), on fp32 MFMA (16x16x4, exact products):
//   X = sum_{c = b}^{a-1} A_ac T_cb,   T_ab = -T_aa X.
// Operand layouts of v_mfma_f32_16x16x4_f32: A lane l holds [row l % 16][k =
// l / 16], B lane l holds [k = l / 16][col l % 16], C lane l holds [rows
// 4 (l / 16) + r][col l % 16].  X stays in registers: at step s of the second
// product lane group g takes k = 4 g + s, which is exactly C element r = s.
template <int SA>
__device__ __forceinline__ void wy_offdiag(int a, int b, const float* sA, float* sT, int lane) {
  const int l16 = lane & 15, gq = lane >> 4;
  f32x4_t x = {0.f, 0.f, 0.f, 0.f};
  for (int cb = b; cb < a; ++cb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kk = 16 * cb + 4 * s + gq;
      x = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * a + l16) * SA + kk],
                                               sT[kk * SA + 16 * b + l16], x, 0, 0, 0);
    }
  }
  f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * a + l16) * SA + 16 * a + 4 * gq + s], x[s],
                                             y, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) sT[(16 * a + 4 * gq + r) * SA + 16 * b + l16] = -y[r];
}

// 8 consecutive elements of an LDS tile row as floats.
__device__ __forceinline__ void row8(const bf16* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(wv[i] << 16);
    x[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void row8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Fragment straight from 8 consecutive elements of a bf16 / fp32 LDS row.
__device__ __forceinline__ FragB frag_row(const bf16* p) {
  return FragB{__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p))};
}
__device__ __forceinline__ FragS frag_row(const float* p) {
  float x[8];
  row8(p, x);
  return make_frag<true>(x);
}

// A q / k / v / g row tile: thread (rg, j) takes rows t = 4 rg + it (so
// wave w holds the 16-token block w) and channels 8 j .. 8 j + 7, kept
// undecoded (their bits) so that a tile can be fetched one work item ahead
// and decoded when its turn comes.
template <typename E> struct RawRows;
template <> struct RawRows<bf16> { uint4 r[4]; };
template <> struct RawRows<float> { float4 r[4][2]; };
template <> struct RawRows<_Float16> { uint4 r[4]; };
__device__ __forceinline__ void raw_row(const bf16* p, RawRows<bf16>& x, int it) {
  x.r[it] = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void raw_row(const _Float16* p, RawRows<_Float16>& x, int it) {
  x.r[it] = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void raw_row(const float* p, RawRows<float>& x, int it) {
  x.r[it][0] = reinterpret_cast<const float4*>(p)[0];
  x.r[it][1] = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void raw_vals(const RawRows<bf16>& x, int it, float* o) {
  const uint32_t w[4] = {x.r[it].x, x.r[it].y, x.r[it].z, x.r[it].w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    o[2 * d] = __uint_as_float(w[d] << 16);
    o[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_vals(const RawRows<_Float16>& x, int it, float* o) {
  const uint32_t w[4] = {x.r[it].x, x.r[it].y, x.r[it].z, x.r[it].w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    o[2 * d] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[d] & 0xffffu));
    o[2 * d + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[d] >> 16));
  }
}
__device__ __forceinline__ void raw_vals(const RawRows<float>& x, int it, float* o) {
  const float4 a = x.r[it][0], b = x.r[it][1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <typename E>
__device__ __forceinline__ void raw_load(const E* src, int stride_t, int L, RawRows<E>& x,
                                         int tid) {
  const int rg = tid >> 4, j = tid & 15;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = min(4 * rg + it, L - 1);  // rows past L re-read row L - 1 ...
    raw_row(src + (size_t)t * stride_t + 8 * j, x, it);
  }
}
template <typename E>
__device__ __forceinline__ void raw_decode(const RawRows<E>& x, int L, float (&out)[4][8],
                                           int tid) {
  const int rg = tid >> 4;
#pragma unroll
  for (int it = 0; it < 4; ++it) raw_vals(x, it, out[it]);
  if (L < C) {  // a ragged chunk (uniform in the workgroup): rows past L are zeroed here
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const bool live = 4 * rg + it < L;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[it][e] = live ? out[it][e] : 0.f;
    }
  }
}
// Channel e (0..7) of the 4 rows of a raw tile as 4 consecutive values.
__device__ __forceinline__ bf16x4_t raw_column(const RawRows<bf16>& x, int e) {
  uint32_t b[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint32_t w[4] = {x.r[it].x, x.r[it].y, x.r[it].z, x.r[it].w};
    b[it] = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu);
  }
  return __builtin_bit_cast(bf16x4_t, make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16)));
}
// fp16 inputs feed fp32 tiles: the column is widened (exactly).
__device__ __forceinline__ float4 raw_column(const RawRows<_Float16>& x, int e) {
  float c[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float o[8];
    raw_vals(x, it, o);
    c[it] = o[e];
  }
  return make_float4(c[0], c[1], c[2], c[3]);
}
__device__ __forceinline__ float4 raw_column(const RawRows<float>& x, int e) {
  float c[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float o[8];
    raw_vals(x, it, o);
    c[it] = o[e];
  }
  return make_float4(c[0], c[1], c[2], c[3]);
}
// Four values of one channel (4 consecutive tokens) in the tile element type.
template <typename E> struct Col4;
template <> struct Col4<bf16> { using T = bf16x4_t; };
template <> struct Col4<float> { using T = float4; };
__device__ __forceinline__ void col4(bf16x4_t& d, float a, float b, float c, float e) {
  d = bf16x4_t{(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)e};
}
__device__ __forceinline__ void col4(float4& d, float a, float b, float c, float e) {
  d = make_float4(a, b, c, e);
}

// 16-byte store of 8 values (bf16: one piece; fp32: two).
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  *reinterpret_cast<bf16x8_t*>(p) = pack8(x);
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// Transposed operand tile [128 rows][64 tokens] (rows: key positions or value
// channels), 16-byte pieces XOR-swizzled with (r ^ (r >> 3)) & 7 so that the
// 8-token-per-row writes of the phase-0 layout (rows 8 j + e) and the
// fragment reads (rows 16 cb + l16) both spread over the banks.
template <typename TE>
__device__ __forceinline__ int tslot(int r, int piece) {
  constexpr int PT = C * (int)sizeof(TE) / 16;  // pieces per row
  return r * PT + (piece ^ ((r ^ (r >> 3)) & 7));
}

// 8 consecutive tokens (two 16-byte pieces from `piece`) of row r of an fp32
// transposed tile.
__device__ __forceinline__ void unit_vals_t(const uint4* tile, int r, int piece, float (&x)[8]) {
  const float4 a = __builtin_bit_cast(float4, tile[tslot<float>(r, piece)]);
  const float4 b = __builtin_bit_cast(float4, tile[tslot<float>(r, piece + 1)]);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}


// Arguments of the walk kernels (one struct so the three modes share them).
template <typename E>
struct WalkArgs {
  const E *qg, *kg_t, *w, *u_t, *aqk;
  const float* decay;
  const int32_t* cu;
  int dense_len, T;
  const int32_t* offs;
  int N, hv;
  float scale;
  const void* init;  // dense initial / final states: fp32, or bf16 with state_bf16
  void* fin;
  int state_bf16;
  void* cache;          // paged pool: fp32, or bf16 with state_bf16
  int64_t slot_stride;  // elements between paged state slots
  const int32_t* slots;
  const uint8_t* has_init;
  int num_slots;
  E* out;
  _Float16* out16;  // fp16 output instead of `out` (fp16 inputs on the fp32 path), or NULL
  int nvb, units, max_chunks, groups;
  float* scan;  // group planes (g, n, h): P [k][j], B [v][k], H_in [v][k]
  const int32_t* nch_max;  // chunks of the batch's longest sequence (device)
  const int32_t* order;    // [N] sequences in decreasing chunk count (device)
  const uint4* zero;
  float* ckpt;  // mid-prefill snapshots [rows, hv, 128, 128] or NULL
  const int32_t *ckpt_off, *ckpt_idx;
  int ckpt_rows;
};

constexpr size_t PLANE = (size_t)D * D;

// Workspace bytes after the zero page (1 KiB of zeros, then the WY work
// counter) where the chunk-table kernel leaves the longest sequence's chunk
// count.
constexpr int KDA_NCH_MAX_OFFSET = 1040;

// Chunks per group of the group scan.  One length for the whole batch, from
// its longest sequence (the chunk-table kernel leaves that count beside the
// zero page): the longest sequences split into G groups, shorter ones into
// fewer (one when they fit a group), so the scan adds pass-one work only
// where it shortens the longest chains.
__device__ __forceinline__ int group_chunks(const int32_t* nch_max, int G) {
  return max(1, (*nch_max + G - 1) / G);
}

// Four values (elements off .. off + 3) of an fp32 or bf16 state plane; bf16
// is widened exactly on load and rounded to nearest even on store.
__device__ __forceinline__ f32x4_t plane_load4(const void* p, size_t off, bool bf) {
  if (bf) {
    const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16*>(p) + off);
    return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  }
  const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + off);
  return f32x4_t{x.x, x.y, x.z, x.w};
}
__device__ __forceinline__ void plane_store4(void* p, size_t off, bool bf, const f32x4_t& v) {
  if (bf) {
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16*>(p) + off) =
        make_uint2((uint32_t)bf16_bits(v[0]) | ((uint32_t)bf16_bits(v[1]) << 16),
                   (uint32_t)bf16_bits(v[2]) | ((uint32_t)bf16_bits(v[3]) << 16));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + off) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
}
// Plane (n, h) of a dense [N, hv, 128, 128] state array of either storage.
// The plane of value head h in slot `slot` of a paged pool (fp32 or bf16).
__device__ __forceinline__ void* pool_plane(void* cache, int64_t slot_stride, int slot, int h,
                                            bool bf) {
  const size_t off = (size_t)slot * slot_stride + (size_t)h * PLANE;
  return bf ? (void*)(reinterpret_cast<bf16*>(cache) + off)
            : (void*)(reinterpret_cast<float*>(cache) + off);
}
__device__ __forceinline__ const void* dense_plane(const void* base, size_t plane, bool bf) {
  return bf ? (const void*)(reinterpret_cast<const bf16*>(base) + plane * PLANE)
            : (const void*)(reinterpret_cast<const float*>(base) + plane * PLANE);
}
__device__ __forceinline__ void* dense_plane(void* base, size_t plane, bool bf) {
  return bf ? (void*)(reinterpret_cast<bf16*>(base) + plane * PLANE)
            : (void*)(reinterpret_cast<float*>(base) + plane * PLANE);
}
__device__ __forceinline__ float* scan_plane(float* scan, int g, int n, int h, int N, int hv,
                                             int which) {
  return scan + ((((size_t)g * N + n) * hv + h) * 3 + which) * PLANE;
}


// ------------------------------------------------------------ group compose

// H_in(0) = S0 and H_in(g+1) = H_in(g) P_g + B_g (V-first: row v of H is
// column v of S, so S_in(g+1) = P_g S_in(g) + B_g).  The rows of H are
// independent, so each one-wave workgroup carries 16 rows (v) through all
// groups of one (sequence, head).  P_g S is formed on MFMA with fp32
// operands split into hi + lo bf16 pairs (three products), keeping the
// composition close to fp32 however many groups there are.
template <typename E>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void compose_kernel(
    const WalkArgs<E> a) {
  // The 8 column-block workgroups of a (sequence, head) get ids with equal
  // id % 8, so they run on one XCD and read each group's transfer through its
  // L2 (blocks of 64 ids hold 8 units).
  const int id = blockIdx.x;
  const int unit = (id >> 6) * 8 + (id & 7), rb = (id >> 3) & 7;
  if (unit >= a.units) return;
  const int hv = a.hv;
  const int n = unit / hv, h = unit - n * hv;
  const int lane = threadIdx.x, l16 = lane & 15, gq = lane >> 4;
  const int vcol = 16 * rb + l16;
  const int G = a.groups;
  // the walk's split of the sequence's chunks into groups; the groups after
  // the one holding its last chunk are empty and walk nothing
  const int nch_all = max(0, min(a.offs[n + 1], a.max_chunks) - a.offs[n]);
  const int cpg = group_chunks(a.nch_max, G);
  const int g_last = nch_all > 0 ? (nch_all - 1) / cpg : 0;
  const void* src = nullptr;
  bool src_bf = false;
  if (a.cache) {
    const int slot = a.slots[n];
    if (slot < 0 || slot >= a.num_slots) return;
    src_bf = a.state_bf16 != 0;
    if (a.has_init[n]) src = pool_plane(a.cache, a.slot_stride, slot, h, src_bf);
  } else if (a.init) {
    src_bf = a.state_bf16 != 0;
    src = dense_plane(a.init, (size_t)n * hv + h, src_bf);
  }
  f32x4_t S[8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    if (src) {
      S[kb] = plane_load4(src, (size_t)vcol * D + 16 * kb + 4 * gq, src_bf);
    } else {
      S[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int g = 0; g <= g_last; ++g) {
    float* hin = scan_plane(a.scan, g, n, h, a.N, hv, 2);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
      *reinterpret_cast<float4*>(hin + (size_t)vcol * D + 16 * kb + 4 * gq) =
          make_float4(S[kb][0], S[kb][1], S[kb][2], S[kb][3]);
    if (g == g_last) break;
    // an empty group's transfer is exactly the identity and its B zero: the
    // state passes on bit for bit (a zero-length sequence keeps its state)
    if (min(nch_all, g * cpg) >= min(nch_all, g * cpg + cpg)) continue;
    const float* P = scan_plane(a.scan, g, n, h, a.N, hv, 0);
    const float* Bp = scan_plane(a.scan, g, n, h, a.N, hv, 1);
    // every load of the step first (one memory round trip per group, not one
    // per row block; the wave has the registers), then the products
    float4 pr[8][4][2], b4[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const float* prow = P + (size_t)(16 * kb + l16) * D;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pr[kb][s][0] = *reinterpret_cast<const float4*>(prow + 32 * s + 4 * gq);
        pr[kb][s][1] = *reinterpret_cast<const float4*>(prow + 32 * s + 16 + 4 * gq);
      }
      b4[kb] = *reinterpret_cast<const float4*>(Bp + (size_t)vcol * D + 16 * kb + 4 * gq);
    }
    FragS Hf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8] = {S[2 * s][0], S[2 * s][1], S[2 * s][2], S[2 * s][3],
                    S[2 * s + 1][0], S[2 * s + 1][1], S[2 * s + 1][2], S[2 * s + 1][3]};
      Hf[s] = make_frag<true>(x);
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      f32x4_t acc = {b4[kb].x, b4[kb].y, b4[kb].z, b4[kb].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float x[8] = {pr[kb][s][0].x, pr[kb][s][0].y, pr[kb][s][0].z, pr[kb][s][0].w,
                            pr[kb][s][1].x, pr[kb][s][1].y, pr[kb][s][1].z, pr[kb][s][1].w};
        mma(acc, make_frag<true>(x), Hf[s]);
      }
      S[kb] = acc;
    }
  }
}

// --------------------------------------------------------------------- launch

// Compute units of the current device, cached per device (relaxed atomics:
// host threads may launch concurrently, and they all store the same value).
inline int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}


}  // namespace kda
