// Tile layouts shared by the chunk kernels (gfx950).
//
// Packed contraction order.  Every intermediate that feeds an MFMA along a
// contraction axis (the key channel of qg and w, the token of kg_t and u_t,
// the column token of aqk) is stored with each 32-element block permuted so
// that position 8 g + j holds element perm32(g, j) of the block.  A lane of
// lane group g then finds its whole fragment in one 16-byte piece, in the K
// order that the register-resident operands (the state and U, which live in
// MFMA C layout) use.
//
// Swizzled LDS tiles.  A tile is R rows of P 16-byte pieces; piece p of row r
// sits in slot r * P + (p ^ (r & 7)).  A fragment read has 8 lanes per LDS
// cycle take one piece each from 8 consecutive rows at one logical column,
// which the XOR spreads over all 32 banks.  The tiles are filled with
// global_load_lds_dwordx4: one wave instruction writes 64 consecutive slots,
// lane l writing slot base + l, so each lane simply loads the global piece
// that belongs in its slot.
#pragma once
#include "kda_mfma.hpp"

namespace kda {

typedef __attribute__((address_space(3))) void* lds_vptr;

// element index inside a 32-block -> packed position
__device__ __forceinline__ int pack32(int x) {
  return 8 * ((x >> 2) & 3) + 4 * (x >> 4) + (x & 3);
}
// packed position -> element index inside a 32-block
__device__ __forceinline__ int unpack32(int m) { return perm32(m >> 3, m & 7); }
__device__ __forceinline__ int packed_index(int x) { return (x & ~31) | pack32(x & 31); }

template <int P>
__device__ __forceinline__ int swz(int r, int p) {
  return r * P + (p ^ (r & 7));
}

// Issue the DMA of an R x P-piece tile (row stride `stride` bytes in global
// memory) into LDS slots starting at `tile`.  With CHECK, rows >= valid come
// from `zero` (1 KiB of zeros); without it every row is read.  The NW waves of
// the workgroup share the wave instructions evenly; `wave` must be
// wave-uniform (readfirstlane) so the LDS base stays scalar.  Nothing waits
// here: the caller waits on vmcnt and then syncs the workgroup.
template <int R, int P, int NW, bool CHECK>
__device__ __forceinline__ void dma_tile(uint4* tile, const void* src, size_t stride, int valid,
                                         const void* zero, int wave, int lane) {
  static_assert((R * P) % (64 * NW) == 0, "tile must split evenly over the waves");
  constexpr int PER = R * P / 64 / NW;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int q = wave + NW * m;
    const int l = 64 * q + lane;
    const int r = l / P, ps = l - r * P;
    const int p = ps ^ (r & 7);
    const char* gp = (const char*)src + (size_t)r * stride + 16 * p;
    if (CHECK) gp = (r < valid) ? gp : (const char*)zero;
    __builtin_amdgcn_global_load_lds(gp, (lds_vptr)(tile + 64 * q), 16, 0, 0);
  }
}

// Only wave instruction m (of R * P / 64 / NW per wave) of dma_tile, so that a
// caller can spread a tile's DMA across other work.
template <int R, int P, int NW, bool CHECK>
__device__ __forceinline__ void dma_one(int m, uint4* tile, const void* src, size_t stride,
                                        int valid, const void* zero, int wave, int lane) {
  const int q = wave + NW * m;
  const int l = 64 * q + lane;
  const int r = l / P, ps = l - r * P;
  const int p = ps ^ (r & 7);
  const char* gp = (const char*)src + (size_t)r * stride + 16 * p;
  if (CHECK) gp = (r < valid) ? gp : (const char*)zero;
  __builtin_amdgcn_global_load_lds(gp, (lds_vptr)(tile + 64 * q), 16, 0, 0);
}

// The pieces of dma_tile through registers: tile_fetch loads this wave's
// pieces (no wait), tile_put writes them to their LDS slots.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int R, int P, int NW, bool CHECK>
__device__ __forceinline__ void tile_fetch(u32x4_t* regs, const void* src, size_t stride,
                                           int valid, const void* zero, int wave, int lane) {
  static_assert((R * P) % (64 * NW) == 0, "tile must split evenly over the waves");
  constexpr int PER = R * P / 64 / NW;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int q = wave + NW * m;
    const int l = 64 * q + lane;
    const int r = l / P, ps = l - r * P;
    const int p = ps ^ (r & 7);
    const char* gp = (const char*)src + (size_t)r * stride + 16 * p;
    if (CHECK) gp = (r < valid) ? gp : (const char*)zero;
    regs[m] = *reinterpret_cast<const u32x4_t*>(gp);
  }
}
// Full tiles without row checks: when 64 / P rows per wave instruction times
// NW is a multiple of 8, a lane's swizzle is the same for every instruction,
// so one per-lane byte offset (tile_off0) and a uniform per-instruction base
// address the whole tile.
template <int P, int NW>
__device__ __forceinline__ uint32_t tile_off0(size_t stride, int wave, int lane) {
  const int l = 64 * wave + lane;
  const int r = l / P, ps = l - r * P;
  return (uint32_t)((size_t)r * stride + 16 * (ps ^ (r & 7)));
}
template <int R, int P, int NW>
__device__ __forceinline__ void tile_fetch_full(u32x4_t* regs, const void* src, size_t stride,
                                                uint32_t off0) {
  constexpr int PER = R * P / 64 / NW, RQ = 64 / P;
  static_assert((RQ * NW) % 8 == 0, "the swizzle must not change between instructions");
#pragma unroll
  for (int m = 0; m < PER; ++m)
    regs[m] = *reinterpret_cast<const u32x4_t*>(
        (const char*)src + (size_t)(RQ * NW * m) * stride + off0);
}
template <int R, int P, int NW>
__device__ __forceinline__ void tile_put(uint4* tile, const u32x4_t* regs, int wave, int lane) {
  constexpr int PER = R * P / 64 / NW;
#pragma unroll
  for (int m = 0; m < PER; ++m)
    *reinterpret_cast<u32x4_t*>(tile + 64 * (wave + NW * m) + lane) = regs[m];
}

// Fragment of a swizzled bf16 tile: logical piece `unit` of row r.
template <int P>
__device__ __forceinline__ FragB frag_bf16(const uint4* tile, int r, int unit) {
  return FragB{__builtin_bit_cast(bf16x8_t, tile[swz<P>(r, unit)])};
}
// Fragment of a swizzled fp32 tile: logical pieces 2 unit and 2 unit + 1.
template <int P>
__device__ __forceinline__ FragS frag_f32(const uint4* tile, int r, int unit) {
  const float4 a = __builtin_bit_cast(float4, tile[swz<P>(r, 2 * unit)]);
  const float4 b = __builtin_bit_cast(float4, tile[swz<P>(r, 2 * unit + 1)]);
  float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  return make_frag<true>(x);
}

// The 8 values of one fragment unit of a tile as floats.
template <int P>
__device__ __forceinline__ void unit_vals(const uint4* tile, int r, int unit, bool f32,
                                          float (&x)[8]) {
  if (!f32) {
    const uint4 u = tile[swz<P>(r, unit)];
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(wv[i] << 16);
      x[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
    }
  } else {
    const float4 a = __builtin_bit_cast(float4, tile[swz<P>(r, 2 * unit)]);
    const float4 b = __builtin_bit_cast(float4, tile[swz<P>(r, 2 * unit + 1)]);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

}  // namespace kda
