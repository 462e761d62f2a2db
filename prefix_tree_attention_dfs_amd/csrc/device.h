// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "tt.h"

namespace ttd {

constexpr int kWave = 64;

// bf16 <-> f32 (bit-exact widening; RNE narrowing, finite values)
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// One RoPE pair (x1, x2) = (x[c], x[c + d/2]) rotated by (c, s) in fp32, each
// result rounded once to bf16: (x1 c - x2 s, x2 c + x1 s).  The products and
// their fusing are written out, so every kernel that rotates through this
// helper produces the same bits for the same inputs.
__device__ __forceinline__ void rot_pair_bf16(float x1, float x2, float c, float s, uint16_t& y1, uint16_t& y2) {
  y1 = f2bf(__builtin_fmaf(x1, c, -(x2 * s)));
  y2 = f2bf(__builtin_fmaf(x2, c, x1 * s));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace ttd

// Pointers into the uploaded plan (device addresses), resolved on the host.
struct PlanPtrs {
  const int32_t* depth;
  const int32_t* end;
  const int32_t* qb_ptr;
  const int32_t* qb_tiles;
  const int32_t* qb_order;
  const int32_t* kb_qlo;
  const int32_t* kb_qhi;
  const int32_t* kb_minend;
  const int32_t* kb_order;
  const int32_t* hdr;  // image header
  int32_t N, bq, bk, nqb, nkb;
  int32_t id;  // the tree's image identity (header word H_ID of its host copy)
};

// True when the device image at P.hdr is the one built for the tree these
// pointers were resolved from: magic word, row count and identity as the host
// recorded them.  Kernels that index plan arrays return at once otherwise, so
// a plan uploaded for another tree cannot make them read past its arrays.
// P is a kernel argument, so the loads are uniform (scalar unit).
__device__ __forceinline__ bool plan_matches(const PlanPtrs& P) {
  typedef __attribute__((address_space(4))) const int32_t cword;
  const cword* h = (const cword*)P.hdr;
  return h[ttp::H_MAGIC] == ttp::kMagic && h[ttp::H_N] == P.N && h[ttp::H_ID] == P.id;
}

// Geometry of one attention call after validation.
struct AttnGeom {
  int32_t q_off, n_q, n_k, h_q, h_kv, d;
  float scale, rope_base;
};
