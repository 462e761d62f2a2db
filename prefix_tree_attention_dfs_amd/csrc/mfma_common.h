// Shared pieces of the bf16 MFMA attention kernels (gfx950, head dim 128).
//
// v_mfma_f32_32x32x16_bf16 operand layout (lane l, r = l % 32, h = l / 32):
//   A (32 x 16):  lane holds A[r][8h .. 8h+7]
//   B (16 x 32):  lane holds B[8h .. 8h+7][r]
//   C (32 x 32):  lane holds C[8*(i/4) + 4h + i%4][r], i = 0..15
// so the columns of a C tile are lanes and its rows are registers.  A C tile
// S^T[key][query] therefore feeds the B operand of the next product with its
// rows as the reduction index: register block 8c..8c+7 of lane-half h holds
// rows 16c + 8*(s/4) + 4h + s%4 (s = 0..7).  The A operand that pairs with it
// is read from a row-major LDS tile with ds_read_tr16_b64, which within each
// group of 16 lanes returns out[i][e] = (lane 4e + i/4's 8 bytes)[i % 4]: when
// lane r' of a group points at row key0 + r'/4, column col0 + 4*(r'%4), lane i
// receives column col0 + i of rows key0 .. key0+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int D = 128;     // head dim
constexpr int BQ = 64;     // query rows per plan block
constexpr int BK = 64;     // key rows per plan block
constexpr int KSTR = 136;  // LDS row stride (bf16) of tiles read with ds_read_b128
constexpr int32_t kFull = 0x40000000;
constexpr int32_t kKbMask = 0x3FFFFFFF;

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int s = 0; s < 8; ++s) z[s] = __bf16(0.f);
  return z;
}

// 16 copies of x, each made by its own move where the call stands: a splat of
// a loop-invariant value written this way is not hoisted out of the loop (a
// hoisted splat would keep 16 more registers live through the loop).
__device__ __forceinline__ f32x16 splat16_here(float x) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(x));
    r[i] = t;
  }
  return r;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 16 bytes from global memory (row guard done by the caller)
__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Raw buffer loads: the hardware compares (voffset + soffset) with the
// buffer's byte size and returns zeros past the end, so tile rows beyond a
// tensor need no clamp and no select.  Offsets are bytes; tensors used this
// way are below 2 GiB (checked on the host).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ bf16x8 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ int32_t bloadi(rsrc_t r, uint32_t voff, uint32_t soff) {
  return int32_t(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Byte size for the descriptor of a tile that starts `elems_left` bf16
// elements before the end of its tensor: reads past the tensor return zeros,
// and a tensor of 4 GiB or more is clamped to what a 32-bit offset reaches
// (a tile never spans more than a few MB).
__device__ __forceinline__ uint32_t tile_rec_bytes(int64_t elems_left) {
  const int64_t b = elems_left > 0 ? elems_left * 2 : 0;
  return b > int64_t(0xFFFFFFF0) ? 0xFFFFFFF0u : uint32_t(b);
}

// Query heads per workgroup of the forward and dQ kernels for a GQA group of
// G heads: 4, 2 or 1, the largest that divides G (a larger group runs as
// G / that many workgroups per block).
__host__ __device__ inline int group_split(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

// One int32 of the plan (read-only for the kernel's whole life) at a
// workgroup-uniform index, loaded through the scalar unit: the value lands in
// an SGPR, so the loop head needs no vector-memory wait, and buffer loads
// whose soffset derives from it need no per-lane loop.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int i) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  return ((const_i32*)p)[i];
}

// LDS byte address of a __shared__ object (the low 32 bits of its generic
// address are its offset in the LDS aperture).
__device__ __forceinline__ uint32_t lds_u32(const void* p) { return uint32_t(reinterpret_cast<uintptr_t>(p)); }

// 16 bytes per lane from a buffer straight into LDS: lane l's chunk lands at
// LDS address lds_base + 16 l (lds_base wave-uniform, via M0); lanes past the
// buffer's size write zeros.  Issued from assembly, so the compiler inserts
// no wait for it: the caller waits with wait_vmem() before the barrier that
// publishes the data.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(r),
                  "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}

// Wait until every vector-memory load issued so far has returned
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their maxima).  Placed
// after a kernel's prologue, it tells the compiler's wait insertion that the
// registers loaded there are ready, so the main loop's first use of them does
// not wait for the tile prefetch issued just before it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8 lds_read16(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Transposed 8-byte LDS read (see header comment).
__device__ __forceinline__ bf16x4 lds_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// A operand (rows = 32 "m" columns of a row-major LDS tile, reduction over 16
// tile rows) for the pairing described above: lane (r, h) gets tile column
// col0 + r of tile rows row0 + 16c + {4h..4h+3, 8+4h..8+4h+3}.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int stride, int row0, int col0, int lane) {
  const int g = lane >> 4, rr = lane & 15;
  const int h = g >> 1, half = g & 1;
  const uint16_t* p = tile + (row0 + 4 * h + (rr >> 2)) * stride + col0 + 16 * half + 4 * (rr & 3);
  const bf16x4 lo = lds_tr4(p);
  const bf16x4 hi = lds_tr4(p + 8 * stride);
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = lo[e];
    a[4 + e] = hi[e];
  }
  return a;
}

// LDS on gfx950: 64 banks of 4 bytes.  A 16-byte read is served 16 lanes per
// cycle and an 8-byte read (plain or transposed) 32 lanes per cycle, so a read
// is free of bank conflicts when each such group of lanes covers distinct banks.
//
// Padded tiles: a row stride of 272 bytes (KSTR) puts 16 consecutive rows of a
// 16-byte column read on distinct banks.
//
// Swizzled 128-column tiles (256-byte rows, no padding): 16-byte chunk c of
// row k lives at chunk c ^ swz(k), swz(k) = the two low 2-bit fields of k
// swapped.  Every row spans all 64 banks once, so a chunk's banks are set by
// its position alone, and
//   * a 16-byte row read by 16 consecutive (16-aligned) rows hits 16 distinct
//     positions, swz being a bijection on them, and
//   * a transposed read, 4 consecutive (4-aligned) rows x 4 adjacent chunks
//     per 32 lanes, hits 16 distinct positions: bits 2-3 of the position
//     follow k % 4 and bits 0-1 the chunk,
// i.e. both access patterns of the backward kernels are free of conflicts.
__device__ __forceinline__ int swz(int k) { return ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int soff(int row, int col) {
  return row * D + ((((col >> 3) ^ swz(row))) << 3) + (col & 7);
}

// tr_frag on a swizzled tile
__device__ __forceinline__ bf16x8 tr_frag_swz(const uint16_t* tile, int row0, int col0, int lane) {
  const int g = lane >> 4, rr = lane & 15;
  const int h = g >> 1, half = g & 1;
  const int row = row0 + 4 * h + (rr >> 2);
  const int col = col0 + 16 * half + 4 * (rr & 3);
  const bf16x4 lo = lds_tr4(tile + soff(row, col));
  const bf16x4 hi = lds_tr4(tile + soff(row + 8, col));
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = lo[e];
    a[4 + e] = hi[e];
  }
  return a;
}

// Register block c (regs 8c..8c+7) of a C tile as a bf16 B operand.
__device__ __forceinline__ bf16x8 c_to_b(const f32x16& x, int c) {
  bf16x8 b;
#pragma unroll
  for (int s = 0; s < 8; ++s) b[s] = __bf16(x[8 * c + s]);
  return b;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ttm
