// Data movement of the path walk (bf16 stack), one launch per segment, round
// or chunk instead of one per tensor and segment (AReaL-DTA, arXiv
// 2602.00482, summary page, Methodology in Plain English: entering a node
// pushes its rows onto the stack of the current path, leaving it pops them;
// Key Contributions 2: the backward runs over right-to-left chunks).
//
// srow[p] is the tree row held at stack position p.  A push writes it for the
// segment's positions; positions above stay untouched until the segment is
// popped, so the round's chunks and outputs look their rows up there.
#include <algorithm>

#include "device.h"
#include "kernels.h"

using namespace ttd;

namespace {

inline unsigned blocks_for(int64_t n, int per) { return unsigned((n + per - 1) / per); }

// One thread per (row, unit).  Units of a row: Q pair-octets (head h, pairs
// 8o..8o+7 with their partners at + d/2), then K pair-octets, then V copies
// of the same two 16-byte chunks.  Q is rotated at its position with the
// (cos, sin) table (null: no rotation) and multiplied by qmul, K rotated,
// both through rot_pair_bf16 (the arithmetic of the tree-mode RoPE kernel).
__global__ __launch_bounds__(256) void path_push_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, uint16_t* __restrict__ Qp,
                                                        uint16_t* __restrict__ Kp, uint16_t* __restrict__ Vp,
                                                        int32_t* __restrict__ srow, const float2* __restrict__ tab,
                                                        int32_t row0, int32_t pos0, int32_t n_rows, int32_t hq,
                                                        int32_t hk, int32_t d, float qmul) {
  const int oct = d >> 4, half = d >> 1;
  const int uq = hq * oct, uk = hk * oct, per_row = uq + 2 * uk;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n_rows) * per_row) return;
  const int r = int(idx / per_row), u = int(idx - int64_t(r) * per_row);
  const int pos = pos0 + r;
  if (u == 0) srow[pos] = row0 + r;
  const int t = u < uq ? 0 : u < uq + uk ? 1 : 2;  // Q, K, V
  const int w = u - (t == 0 ? 0 : t == 1 ? uq : uq + uk);
  const int h = w / oct, k0 = (w - h * oct) * 8;
  const int heads = t == 0 ? hq : hk;
  const uint16_t* src = t == 0 ? q : t == 1 ? k : v;
  uint16_t* dst = t == 0 ? Qp : t == 1 ? Kp : Vp;
  const int64_t sb = (int64_t(row0 + r) * heads + h) * d + k0, db = (int64_t(pos) * heads + h) * d + k0;
  const uint4 a1 = *reinterpret_cast<const uint4*>(src + sb);
  const uint4 a2 = *reinterpret_cast<const uint4*>(src + sb + half);
  if (t == 2) {
    *reinterpret_cast<uint4*>(dst + db) = a1;
    *reinterpret_cast<uint4*>(dst + db + half) = a2;
    return;
  }
  const float mf = t == 0 ? qmul : 1.f;
  const float2* tr = tab ? tab + int64_t(pos) * half + k0 : nullptr;
  const uint32_t w1[4] = {a1.x, a1.y, a1.z, a1.w}, w2[4] = {a2.x, a2.y, a2.z, a2.w};
  uint32_t o1[4], o2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo1 = 0, lo2 = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float2 cs = tr ? tr[2 * i + s] : make_float2(1.f, 0.f);
      uint16_t y1, y2;
      rot_pair_bf16(bf2f(uint16_t(w1[i] >> (16 * s))), bf2f(uint16_t(w2[i] >> (16 * s))), cs.x * mf, cs.y * mf, y1,
                    y2);
      lo1 |= uint32_t(y1) << (16 * s);
      lo2 |= uint32_t(y2) << (16 * s);
    }
    o1[i] = lo1;
    o2[i] = lo2;
  }
  *reinterpret_cast<uint4*>(dst + db) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  *reinterpret_cast<uint4*>(dst + db + half) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
}

// Stack rows [p0, p1) -> their tree rows: row_bytes of a (16-byte chunks)
// and lse_n floats of b per position.
__global__ __launch_bounds__(256) void path_scatter_kernel(const uint4* __restrict__ a, uint4* __restrict__ a_out,
                                                           const float* __restrict__ b, float* __restrict__ b_out,
                                                           const int32_t* __restrict__ srow, int32_t p0, int32_t n,
                                                           int32_t a_chunks, int32_t b_n, int64_t a_src0) {
  const int per_row = a_chunks + b_n;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n) * per_row) return;
  const int r = int(idx / per_row), c = int(idx - int64_t(r) * per_row);
  const int64_t row = srow[p0 + r];
  if (c < a_chunks)
    a_out[row * a_chunks + c] = a[(a_src0 + r) * a_chunks + c];
  else
    b_out[row * b_n + (c - a_chunks)] = b[int64_t(p0 + r) * b_n + (c - a_chunks)];
}

// The dO blocks and D of the backward chunks of one launch (blockIdx.y =
// chunk): for block row i (position qo + i), dO_blk[i] = dO[srow[qo + i]]
// (zeros below c0, the 64-row alignment pad) and D[i, h] = sum_c dO_blk[i, h,
// c] * O_stack[qo + i, h, c], summed as the preprocess kernel sums (L = d/8
// lanes of 8 products, then a butterfly), so D has the same bits as from the
// copied block.
template <int L>
__global__ __launch_bounds__(256) void path_dout_pre_kernel(const uint16_t* __restrict__ Op,
                                                            const uint16_t* __restrict__ d_o,
                                                            const int32_t* __restrict__ srow, PathChunks C,
                                                            int32_t hq) {
  const PathChunk& ch = C.c[blockIdx.y];
  uint16_t* __restrict__ dob = static_cast<uint16_t*>(ch.dob);
  const int32_t qo = ch.qo, c0 = ch.c0;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rh = t / L;  // (block row, head)
  const int sub = int(t % L);
  const int64_t rows = int64_t(ch.c1 - qo) * hq;
  float a = 0.f;
  if (rh < rows) {
    const int i = int(rh / hq), h = int(rh - int64_t(i) * hq);
    uint4 y = make_uint4(0u, 0u, 0u, 0u);
    if (qo + i >= c0) y = *reinterpret_cast<const uint4*>(d_o + (int64_t(srow[qo + i]) * hq + h) * (8 * L) + 8 * sub);
    *reinterpret_cast<uint4*>(dob + rh * (8 * L) + 8 * sub) = y;
    const uint4 x = *reinterpret_cast<const uint4*>(Op + (int64_t(qo) * hq + rh) * (8 * L) + 8 * sub);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += __uint_as_float(xs[e] << 16) * __uint_as_float(ys[e] << 16);
      a += __uint_as_float(xs[e] & 0xFFFF0000u) * __uint_as_float(ys[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) a += __shfl_xor(a, m, kWave);
  if (rh < rows && sub == 0) ch.D[rh] = a;
}

// The dQ rows of the backward chunks of one launch (blockIdx.y = chunk) to
// their tree rows: position p in [c0, c1) is row p - qo of the chunk's block.
__global__ __launch_bounds__(256) void path_dq_scatter_kernel(uint4* __restrict__ d_q,
                                                              const int32_t* __restrict__ srow, PathChunks C,
                                                              int32_t chunks_per_row) {
  const PathChunk& ch = C.c[blockIdx.y];
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(ch.c1 - ch.c0) * chunks_per_row) return;
  const int r = int(idx / chunks_per_row), c = int(idx - int64_t(r) * chunks_per_row);
  d_q[int64_t(srow[ch.c0 + r]) * chunks_per_row + c] =
      static_cast<const uint4*>(ch.dq_blk)[int64_t(ch.c0 - ch.qo + r) * chunks_per_row + c];
}

}  // namespace

int launch_path_push(const void* q, const void* k, const void* v, void* Qp, void* Kp, void* Vp, int32_t* srow,
                     const float2* tab, int32_t row0, int32_t pos0, int32_t n_rows, int32_t hq, int32_t hk,
                     int32_t d, float qmul, hipStream_t st) {
  if (n_rows <= 0) return 0;
  if (d % 16 != 0) return -1;
  const int64_t n = int64_t(n_rows) * (hq + 2 * hk) * (d / 16);
  path_push_kernel<<<dim3(blocks_for(n, 256)), dim3(256), 0, st>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<uint16_t*>(Qp), static_cast<uint16_t*>(Kp), static_cast<uint16_t*>(Vp), srow, tab, row0, pos0,
      n_rows, hq, hk, d, qmul);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_path_scatter(const void* a, void* a_out, int64_t a_row_bytes, int64_t a_src0, const float* b,
                        float* b_out, int32_t b_n, const int32_t* srow, int32_t p0, int32_t p1, hipStream_t st) {
  const int32_t n = p1 - p0;
  if (n <= 0) return 0;
  if (a_row_bytes % 16 != 0 || (b_n > 0 && (!b || !b_out))) return -1;
  const int32_t a_chunks = int32_t(a_row_bytes / 16);
  const int64_t tot = int64_t(n) * (a_chunks + b_n);
  path_scatter_kernel<<<dim3(blocks_for(tot, 256)), dim3(256), 0, st>>>(
      static_cast<const uint4*>(a), static_cast<uint4*>(a_out), b, b_out, srow, p0, n, a_chunks, b_n, a_src0);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_path_dout_pre(const void* Op, const void* d_o, const int32_t* srow, const PathChunks& C, int32_t hq,
                         int32_t d, hipStream_t st) {
  if (C.n <= 0) return 0;
  if (d != 128 || C.n > kMaxBwdCalls) return -1;
  constexpr int L = 16;
  int64_t rows = 0;
  for (int u = 0; u < C.n; ++u) rows = std::max<int64_t>(rows, C.c[u].c1 - C.c[u].qo);
  if (rows <= 0) return 0;
  path_dout_pre_kernel<L><<<dim3(blocks_for(rows * hq * L, 256), unsigned(C.n)), dim3(256), 0, st>>>(
      static_cast<const uint16_t*>(Op), static_cast<const uint16_t*>(d_o), srow, C, hq);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_path_dq_scatter(void* d_q, int64_t row_bytes, const int32_t* srow, const PathChunks& C, hipStream_t st) {
  if (C.n <= 0) return 0;
  if (row_bytes % 16 != 0 || C.n > kMaxBwdCalls) return -1;
  const int32_t cpr = int32_t(row_bytes / 16);
  int64_t rows = 0;
  for (int u = 0; u < C.n; ++u) rows = std::max<int64_t>(rows, C.c[u].c1 - C.c[u].c0);
  if (rows <= 0) return 0;
  path_dq_scatter_kernel<<<dim3(blocks_for(rows * cpr, 256), unsigned(C.n)), dim3(256), 0, st>>>(
      static_cast<uint4*>(d_q), srow, C, cpr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
