// Generic tree-attention kernels: any head dim (multiple of 16, <= 256), fp32 or
// bf16 storage, fp32 arithmetic.  They serve the fp32 configurations and every
// shape the MFMA kernels do not take; they are also the rotation and
// preprocessing kernels the MFMA path shares.
//
// Visibility: key row j is seen by query row i iff j <= i < end[j] (j is i or
// an ancestor of i in DFS order); positions are depths, so each row's result
// equals its per-branch causal-attention result (Tree Training, Abstract).
#include <algorithm>

#include "device.h"
#include "kernels.h"

using namespace ttd;

namespace {

// ---------------------------------------------------------------- RoPE (K1/K5)
// y = mul R(depth * theta) x (or mul R^T x), theta_k = base^(-2k/d), pairs
// (k, k+d/2); mul is 1 except for the query copy of the matrix-core kernels,
// which carries the softmax scale times log2(e).  One thread per (row, k);
// the angle is formed and rotated in fp64, rounded once to the output type.
template <typename Tin, typename Tout, bool ACC>
__global__ __launch_bounds__(256) void rope_kernel(const Tin* __restrict__ x, Tout* __restrict__ y, PlanPtrs P,
                                                   int32_t row0, int32_t n_rows, int32_t heads, int32_t d,
                                                   double base, double sign, double mul) {
  if (!plan_matches(P)) return;
  const int32_t* __restrict__ depth = P.depth;
  const int half = d >> 1;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n_rows) * half) return;
  const int64_t r = idx / half;
  const int k = int(idx - r * half);
  double c = 1.0, s = 0.0;
  if (base != 0.0) {
    const double theta = pow(base, -2.0 * double(k) / double(d));
    sincos(double(depth[row0 + r]) * theta, &s, &c);
    s *= sign;
  }
  c *= mul;
  s *= mul;
  for (int h = 0; h < heads; ++h) {
    const int64_t b = (r * heads + h) * d;
    const double x1 = Elem<Tin>::load(x, b + k), x2 = Elem<Tin>::load(x, b + k + half);
    const float y1 = float(x1 * c - x2 * s), y2 = float(x2 * c + x1 * s);
    if (ACC) {
      Elem<Tout>::store(y, b + k, Elem<Tout>::load(y, b + k) + y1);
      Elem<Tout>::store(y, b + k + half, Elem<Tout>::load(y, b + k + half) + y2);
    } else {
      Elem<Tout>::store(y, b + k, y1);
      Elem<Tout>::store(y, b + k + half, y2);
    }
  }
}

// The bf16 -> bf16 rotation of rope_kernel with 16-byte accesses: one thread
// per (row, 8 consecutive pairs, group of hpt heads), looping over its heads.
// Few rows (a path segment) split the heads over more threads so the grid
// still fills the chip.  With tab, the (cos, sin) table of rope_table_kernel
// (fp64 angles rounded once to fp32, row = depth), or with base 0 (no
// rotation, only the factor mul): rot_pair_bf16 in fp32, the arithmetic the
// matrix-core forward uses when it rotates its own query copy.  Otherwise
// the same fp64 angles and arithmetic as rope_kernel (bit-identical results).
// Needs half % 8 == 0, 16-byte aligned rows and hpt | heads.
__global__ __launch_bounds__(256) void rope_bf16x8_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                          PlanPtrs P, int32_t row0, int32_t n_rows, int32_t heads,
                                                          int32_t d, double base, double sign, double mul,
                                                          int32_t hpt, const float2* __restrict__ tab) {
  if (!plan_matches(P)) return;
  const int half = d >> 1, oct = half >> 3, hgroups = heads / hpt;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n_rows) * oct * hgroups) return;
  const int64_t rh = idx / oct;  // consecutive threads: consecutive octets of one head
  const int k0 = int(idx - rh * oct) * 8;
  const int64_t r = rh / hgroups;
  const int h0 = int(rh - r * hgroups) * hpt;
  if (tab || base == 0.0) {
    const float2* t = tab ? tab + int64_t(P.depth[row0 + r]) * half + k0 : nullptr;
    const float mf = float(mul), sf = float(sign * mul);
    float cf[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float2 cs = t ? t[e] : make_float2(1.f, 0.f);
      cf[e] = cs.x * mf;
      sn[e] = cs.y * sf;
    }
#pragma unroll 2
    for (int h = h0; h < h0 + hpt; ++h) {
      const int64_t b = (r * heads + h) * d + k0;
      const uint4 a1 = *reinterpret_cast<const uint4*>(x + b);
      const uint4 a2 = *reinterpret_cast<const uint4*>(x + b + half);
      const uint32_t w1[4] = {a1.x, a1.y, a1.z, a1.w}, w2[4] = {a2.x, a2.y, a2.z, a2.w};
      uint32_t o1[4], o2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t lo1 = 0, lo2 = 0;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int e = 2 * u + tt;
          uint16_t y1, y2;
          rot_pair_bf16(bf2f(uint16_t(w1[u] >> (16 * tt))), bf2f(uint16_t(w2[u] >> (16 * tt))), cf[e], sn[e], y1, y2);
          lo1 |= uint32_t(y1) << (16 * tt);
          lo2 |= uint32_t(y2) << (16 * tt);
        }
        o1[u] = lo1;
        o2[u] = lo2;
      }
      *reinterpret_cast<uint4*>(y + b) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
      *reinterpret_cast<uint4*>(y + b + half) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
    }
    return;
  }
  double c[8], sn[8];
  const double pos = double(P.depth[row0 + r]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = 1.0;
    sn[e] = 0.0;
    if (base != 0.0) {
      const double theta = pow(base, -2.0 * double(k0 + e) / double(d));
      sincos(pos * theta, &sn[e], &c[e]);
      sn[e] *= sign;
    }
    c[e] *= mul;
    sn[e] *= mul;
  }
#pragma unroll 2
  for (int h = h0; h < h0 + hpt; ++h) {
    const int64_t b = (r * heads + h) * d + k0;
    const uint4 a1 = *reinterpret_cast<const uint4*>(x + b);
    const uint4 a2 = *reinterpret_cast<const uint4*>(x + b + half);
    const uint32_t w1[4] = {a1.x, a1.y, a1.z, a1.w}, w2[4] = {a2.x, a2.y, a2.z, a2.w};
    uint32_t o1[4], o2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t lo1 = 0, lo2 = 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int e = 2 * u + t;
        const double x1 = bf2f(uint16_t(w1[u] >> (16 * t))), x2 = bf2f(uint16_t(w2[u] >> (16 * t)));
        const float y1 = float(x1 * c[e] - x2 * sn[e]), y2 = float(x2 * c[e] + x1 * sn[e]);
        lo1 |= uint32_t(f2bf(y1)) << (16 * t);
        lo2 |= uint32_t(f2bf(y2)) << (16 * t);
      }
      o1[u] = lo1;
      o2[u] = lo2;
    }
    *reinterpret_cast<uint4*>(y + b) = make_uint4(o1[0], o1[1], o1[2], o1[3]);
    *reinterpret_cast<uint4*>(y + b + half) = make_uint4(o2[0], o2[1], o2[2], o2[3]);
  }
}

// (cos, sin) of p * theta_k for every position p < n_pos and pair k < half,
// in fp64, rounded once to fp32 (the table the dK/dV epilogue rotates with).
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int32_t n_pos, int32_t half,
                                                         double base) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n_pos) * half) return;
  const int64_t p = idx / half;
  const int k = int(idx - p * half);
  const double theta = pow(base, -2.0 * double(k) / double(2 * half));
  double sn, cs;
  sincos(double(p) * theta, &sn, &cs);
  tab[idx] = make_float2(float(cs), float(sn));
}

// ---------------------------------------------------------------- forward
// One wave per (query row, query head).  Keys are visited tile by tile
// through the q-block's list of non-empty k-blocks; lane = key.
template <typename T, int DMAX>
__global__ __launch_bounds__(256) void fwd_generic(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, T* __restrict__ o,
                                                   float* __restrict__ lse, PlanPtrs P, AttnGeom g) {
  if (!plan_matches(P)) return;
  constexpr int NT = DMAX / kWave;
  __shared__ float qs[4][DMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + wave;
  const bool valid = pair < int64_t(g.n_q) * g.h_q;
  const int il = valid ? int(pair / g.h_q) : 0;
  const int h = valid ? int(pair % g.h_q) : 0;
  const int i = g.q_off + il;
  const int kvh = h / (g.h_q / g.h_kv);
  const int d = g.d;
  if (valid)
    for (int c = lane; c < d; c += kWave) qs[wave][c] = Elem<T>::load(q, (int64_t(il) * g.h_q + h) * d + c);
  __syncthreads();
  if (!valid) return;
  float m = -INFINITY, l = 0.f;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  const int qb = i / P.bq;
  for (int e = P.qb_ptr[qb]; e < P.qb_ptr[qb + 1]; ++e) {
    const int kb = P.qb_tiles[e] & 0x3FFFFFFF;
    for (int j0 = kb * P.bk; j0 < kb * P.bk + P.bk; j0 += kWave) {
      const int j = j0 + lane;
      const bool vis = j < kb * P.bk + P.bk && j < g.n_k && j <= i && i < P.end[j];
      float s = -INFINITY;
      if (vis) {
        const T* kr = k + (int64_t(j) * g.h_kv + kvh) * d;
        float a = 0.f;
        for (int c = 0; c < d; ++c) a += qs[wave][c] * Elem<T>::load(kr, c);
        s = a * g.scale;
      }
      const float mt = wave_max(s);
      if (mt == -INFINITY) continue;
      const float mn = fmaxf(m, mt);
      const float alpha = expf(m - mn);
      const float p = vis ? expf(s - mn) : 0.f;
      l = l * alpha + wave_sum(p);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
      for (int jj = 0; jj < kWave; ++jj) {
        const float pj = __shfl(p, jj, kWave);
        if (pj != 0.f) {
          const T* vr = v + (int64_t(j0 + jj) * g.h_kv + kvh) * d;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int c = lane + t * kWave;
            if (c < d) acc[t] += pj * Elem<T>::load(vr, c);
          }
        }
      }
      m = mn;
    }
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = lane + t * kWave;
    if (c < d) Elem<T>::store(o, (int64_t(il) * g.h_q + h) * d + c, acc[t] * inv);
  }
  if (lane == 0) lse[int64_t(il) * g.h_q + h] = m + logf(l);
}

// ---------------------------------------------------------------- backward pre (K3)
// D[i,h] = sum_c dO[i,h,c] * O[i,h,c]; one wave per (row, head).
template <typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ d_o,
                                                      float* __restrict__ D, int64_t rows, int d) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = int64_t(blockIdx.x) * 4 + wave;
  if (r >= rows) return;
  float a = 0.f;
  for (int c = lane; c < d; c += kWave) a += Elem<T>::load(o, r * d + c) * Elem<T>::load(d_o, r * d + c);
  a = wave_sum(a);
  if (lane == 0) D[r] = a;
}

// bf16 rows of length d = 8 L (L a power of two, at most 64): L lanes per
// row, each with one 16-byte load of O and of dO, then a reduction over the
// row's L lanes.  Rows start 16-byte aligned (checked by the launcher).
template <int L>
__global__ __launch_bounds__(256) void bwd_pre_vec_kernel(const uint16_t* __restrict__ o,
                                                          const uint16_t* __restrict__ d_o, float* __restrict__ D,
                                                          int64_t rows) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r = t / L;
  const int sub = int(t % L);
  float a = 0.f;
  if (r < rows) {
    const uint4 x = *reinterpret_cast<const uint4*>(o + r * (8 * L) + 8 * sub);
    const uint4 y = *reinterpret_cast<const uint4*>(d_o + r * (8 * L) + 8 * sub);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += __uint_as_float(xs[e] << 16) * __uint_as_float(ys[e] << 16);
      a += __uint_as_float(xs[e] & 0xFFFF0000u) * __uint_as_float(ys[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) a += __shfl_xor(a, m, kWave);
  if (r < rows && sub == 0) D[r] = a;
}

// ---------------------------------------------------------------- dQ
// One wave per (query row, head); writes scale * sum_j dS_ij k'_j (rotated
// frame, fp32) into dq_acc.
template <typename T, int DMAX>
__global__ __launch_bounds__(256) void dq_generic(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const T* __restrict__ d_o,
                                                  const float* __restrict__ lse, const float* __restrict__ D,
                                                  float* __restrict__ dq_acc, PlanPtrs P, AttnGeom g) {
  if (!plan_matches(P)) return;
  constexpr int NT = DMAX / kWave;
  __shared__ float qs[4][DMAX];
  __shared__ float ds_[4][DMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + wave;
  const bool valid = pair < int64_t(g.n_q) * g.h_q;
  const int il = valid ? int(pair / g.h_q) : 0;
  const int h = valid ? int(pair % g.h_q) : 0;
  const int i = g.q_off + il;
  const int kvh = h / (g.h_q / g.h_kv);
  const int d = g.d;
  const int64_t row = int64_t(il) * g.h_q + h;
  if (valid)
    for (int c = lane; c < d; c += kWave) {
      qs[wave][c] = Elem<T>::load(q, row * d + c);
      ds_[wave][c] = Elem<T>::load(d_o, row * d + c);
    }
  __syncthreads();
  if (!valid) return;
  const float Li = lse[row], Di = D[row];
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  const int qb = i / P.bq;
  for (int e = P.qb_ptr[qb]; e < P.qb_ptr[qb + 1]; ++e) {
    const int kb = P.qb_tiles[e] & 0x3FFFFFFF;
    for (int j0 = kb * P.bk; j0 < kb * P.bk + P.bk; j0 += kWave) {
      const int j = j0 + lane;
      const bool vis = j < kb * P.bk + P.bk && j < g.n_k && j <= i && i < P.end[j];
      float dsj = 0.f;
      if (vis) {
        const T* kr = k + (int64_t(j) * g.h_kv + kvh) * d;
        const T* vr = v + (int64_t(j) * g.h_kv + kvh) * d;
        float s = 0.f, dp = 0.f;
        for (int c = 0; c < d; ++c) {
          s += qs[wave][c] * Elem<T>::load(kr, c);
          dp += ds_[wave][c] * Elem<T>::load(vr, c);
        }
        const float p = expf(s * g.scale - Li);
        dsj = p * (dp - Di);
      }
      for (int jj = 0; jj < kWave; ++jj) {
        const float x = __shfl(dsj, jj, kWave);
        if (x != 0.f) {
          const T* kr = k + (int64_t(j0 + jj) * g.h_kv + kvh) * d;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int c = lane + t * kWave;
            if (c < d) acc[t] += x * Elem<T>::load(kr, c);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = lane + t * kWave;
    if (c < d) dq_acc[row * d + c] = acc[t] * g.scale;
  }
}

// ---------------------------------------------------------------- dK, dV
// One wave per (key row, kv head).  Key j is seen by the query rows
// [max(j, q_off), min(end[j], q_off + n_q)); lane = query.  dK is rotated
// back (R^T at the key's depth) before it is stored.
template <typename T, typename TG, bool ACC, int DMAX>
__global__ __launch_bounds__(256) void dkdv_generic(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const T* __restrict__ d_o,
                                                    const float* __restrict__ lse, const float* __restrict__ D,
                                                    TG* __restrict__ d_k, TG* __restrict__ d_v, PlanPtrs P,
                                                    AttnGeom g) {
  if (!plan_matches(P)) return;
  constexpr int NT = DMAX / kWave;
  __shared__ float ks[4][DMAX];
  __shared__ float vs[4][DMAX];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = int64_t(blockIdx.x) * 4 + wave;
  const bool valid = pair < int64_t(g.n_k) * g.h_kv;
  const int j = valid ? int(pair / g.h_kv) : 0;
  const int kvh = valid ? int(pair % g.h_kv) : 0;
  const int d = g.d;
  const int64_t krow = int64_t(j) * g.h_kv + kvh;
  if (valid)
    for (int c = lane; c < d; c += kWave) {
      ks[wave][c] = Elem<T>::load(k, krow * d + c);
      vs[wave][c] = Elem<T>::load(v, krow * d + c);
    }
  __syncthreads();
  float dk[NT], dv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) dk[t] = dv[t] = 0.f;
  const int G = g.h_q / g.h_kv;
  const int lo = valid ? max(j, g.q_off) : 0;
  const int hi = valid ? min(P.end[j], g.q_off + g.n_q) : 0;
  for (int hh = 0; hh < G && valid; ++hh) {
    const int h = kvh * G + hh;
    for (int i0 = lo; i0 < hi; i0 += kWave) {
      const int i = i0 + lane;
      float p = 0.f, dsi = 0.f;
      if (i < hi) {
        const int64_t row = int64_t(i - g.q_off) * g.h_q + h;
        const T* qr = q + row * d;
        const T* dor = d_o + row * d;
        float s = 0.f, dp = 0.f;
        for (int c = 0; c < d; ++c) {
          s += Elem<T>::load(qr, c) * ks[wave][c];
          dp += Elem<T>::load(dor, c) * vs[wave][c];
        }
        p = expf(s * g.scale - lse[row]);
        dsi = p * (dp - D[row]);
      }
      const int cnt = min(kWave, hi - i0);
      for (int ii = 0; ii < cnt; ++ii) {
        const float pi = __shfl(p, ii, kWave);
        const float x = __shfl(dsi, ii, kWave);
        const int64_t row = int64_t(i0 + ii - g.q_off) * g.h_q + h;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int c = lane + t * kWave;
          if (c < d) {
            dv[t] += pi * Elem<T>::load(d_o, row * d + c);
            dk[t] += x * Elem<T>::load(q, row * d + c);
          }
        }
      }
    }
  }
  // rotate dK back: stage in LDS (reuse ks), then each lane reads its pair partner
  __syncthreads();
  if (valid)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = lane + t * kWave;
      if (c < d) ks[wave][c] = dk[t] * g.scale;
    }
  __syncthreads();
  if (!valid) return;
  const int half = d >> 1;
  double cs = 1.0, sn = 0.0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int c = lane + t * kWave;
    if (c >= d) continue;
    const int kk = c < half ? c : c - half;
    if (g.rope_base != 0.f) {
      const double theta = pow(double(g.rope_base), -2.0 * double(kk) / double(d));
      sincos(double(P.depth[j]) * theta, &sn, &cs);
    }
    // R^T: x'_k = x_k cos + x_{k+h} sin ; x'_{k+h} = x_{k+h} cos - x_k sin
    float val;
    if (c < half)
      val = float(double(ks[wave][c]) * cs + double(ks[wave][c + half]) * sn);
    else
      val = float(double(ks[wave][c]) * cs - double(ks[wave][c - half]) * sn);
    const int64_t off = krow * d + c;
    if (ACC) {
      Elem<TG>::store(d_k, off, Elem<TG>::load(d_k, off) + val);
      Elem<TG>::store(d_v, off, Elem<TG>::load(d_v, off) + dv[t]);
    } else {
      Elem<TG>::store(d_k, off, val);
      Elem<TG>::store(d_v, off, dv[t]);
    }
  }
}

inline unsigned blocks_for(int64_t n, int per) { return unsigned((n + per - 1) / per); }

}  // namespace

// ---------------------------------------------------------------- launchers
int launch_rope(const void* x, void* y, tt_dtype tin, tt_dtype tout, bool acc, const PlanPtrs& P, int32_t row0,
                int32_t n_rows, int32_t heads, int32_t d, float base, bool inverse, hipStream_t st, double mul,
                const float2* tab) {
  const int64_t n = int64_t(n_rows) * (d / 2);
  if (n == 0) return 0;
  const dim3 grid(blocks_for(n, 256)), block(256);
  const double sg = inverse ? -1.0 : 1.0;
  const double b = double(base);
  if (tin == TT_F32 && tout == TT_F32 && !acc)
    rope_kernel<float, float, false><<<grid, block, 0, st>>>((const float*)x, (float*)y, P, row0, n_rows, heads, d, b, sg, mul);
  else if (tin == TT_F32 && tout == TT_F32 && acc)
    rope_kernel<float, float, true><<<grid, block, 0, st>>>((const float*)x, (float*)y, P, row0, n_rows, heads, d, b, sg, mul);
  else if (tin == TT_BF16 && tout == TT_BF16 && !acc && (d % 16) == 0 &&
           ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0) {
    // heads per thread: all of them, halved while the grid has fewer than
    // 2^18 threads (1024 per CU) and the count stays a divisor
    const int64_t nv = int64_t(n_rows) * (d / 16);
    int hpt = heads;
    while (hpt % 2 == 0 && nv * (heads / hpt) < (int64_t(1) << 18)) hpt /= 2;
    rope_bf16x8_kernel<<<dim3(blocks_for(nv * (heads / hpt), 256)), block, 0, st>>>(
        (const uint16_t*)x, (uint16_t*)y, P, row0, n_rows, heads, d, b, sg, mul, hpt, base != 0.f ? tab : nullptr);
  } else if (tin == TT_BF16 && tout == TT_BF16 && !acc)
    rope_kernel<uint16_t, uint16_t, false><<<grid, block, 0, st>>>((const uint16_t*)x, (uint16_t*)y, P, row0, n_rows, heads, d, b, sg, mul);
  else if (tin == TT_F32 && tout == TT_BF16 && !acc)
    rope_kernel<float, uint16_t, false><<<grid, block, 0, st>>>((const float*)x, (uint16_t*)y, P, row0, n_rows, heads, d, b, sg, mul);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rope_table(float2* tab, int32_t n_pos, int32_t half, float base, hipStream_t st) {
  const int64_t n = int64_t(n_pos) * half;
  if (n == 0) return 0;
  rope_table_kernel<<<dim3(blocks_for(n, 256)), dim3(256), 0, st>>>(tab, n_pos, half, double(base));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

#define TT_DMAX_DISPATCH(d, FN) \
  ((d) <= 64 ? FN(64) : (d) <= 128 ? FN(128) : FN(256))

int launch_fwd_generic(tt_dtype dt, const void* q, const void* k, const void* v, void* o, float* lse,
                       const PlanPtrs& P, const AttnGeom& g, hipStream_t st) {
  const int64_t pairs = int64_t(g.n_q) * g.h_q;
  if (pairs == 0) return 0;
  const dim3 grid(blocks_for(pairs, 4)), block(256);
#define FWD(DM)                                                                                                 \
  (dt == TT_F32 ? (fwd_generic<float, DM><<<grid, block, 0, st>>>((const float*)q, (const float*)k,             \
                                                                   (const float*)v, (float*)o, lse, P, g), 0)   \
                : (fwd_generic<uint16_t, DM><<<grid, block, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,    \
                                                                      (const uint16_t*)v, (uint16_t*)o, lse, P, g), 0))
  TT_DMAX_DISPATCH(g.d, FWD);
#undef FWD
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_bwd_pre(tt_dtype dt, const void* o, const void* d_o, float* D, int64_t rows, int d, hipStream_t st) {
  if (rows == 0) return 0;
  const int L = d / 8;
  const bool vec = dt == TT_BF16 && d % 8 == 0 && L <= 64 && (L & (L - 1)) == 0 &&
                   (reinterpret_cast<uintptr_t>(o) & 15u) == 0 && (reinterpret_cast<uintptr_t>(d_o) & 15u) == 0;
  if (vec) {
    const dim3 vgrid(blocks_for(rows * L, 256)), vblock(256);
    const uint16_t *ob = static_cast<const uint16_t*>(o), *db = static_cast<const uint16_t*>(d_o);
    switch (L) {
#define PRE(LL) \
  case LL: bwd_pre_vec_kernel<LL><<<vgrid, vblock, 0, st>>>(ob, db, D, rows); break;
      PRE(1) PRE(2) PRE(4) PRE(8) PRE(16) PRE(32) PRE(64)
#undef PRE
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const dim3 grid(blocks_for(rows, 4)), block(256);
  if (dt == TT_F32)
    bwd_pre_kernel<float><<<grid, block, 0, st>>>((const float*)o, (const float*)d_o, D, rows, d);
  else
    bwd_pre_kernel<uint16_t><<<grid, block, 0, st>>>((const uint16_t*)o, (const uint16_t*)d_o, D, rows, d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dq_generic(tt_dtype dt, const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                      const float* D, float* dq_acc, const PlanPtrs& P, const AttnGeom& g, hipStream_t st) {
  const int64_t pairs = int64_t(g.n_q) * g.h_q;
  if (pairs == 0) return 0;
  const dim3 grid(blocks_for(pairs, 4)), block(256);
#define DQ(DM)                                                                                                   \
  (dt == TT_F32 ? (dq_generic<float, DM><<<grid, block, 0, st>>>((const float*)q, (const float*)k,               \
                                                                  (const float*)v, (const float*)d_o, lse, D,    \
                                                                  dq_acc, P, g), 0)                              \
                : (dq_generic<uint16_t, DM><<<grid, block, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,      \
                                                                     (const uint16_t*)v, (const uint16_t*)d_o,   \
                                                                     lse, D, dq_acc, P, g), 0))
  TT_DMAX_DISPATCH(g.d, DQ);
#undef DQ
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dkdv_generic(tt_dtype dt, bool acc, const void* q, const void* k, const void* v, const void* d_o,
                        const float* lse, const float* D, void* d_k, void* d_v, const PlanPtrs& P,
                        const AttnGeom& g, hipStream_t st) {
  const int64_t pairs = int64_t(g.n_k) * g.h_kv;
  if (pairs == 0) return 0;
  const dim3 grid(blocks_for(pairs, 4)), block(256);
#define KV(DM)                                                                                                   \
  (dt == TT_F32                                                                                                  \
       ? (acc ? (dkdv_generic<float, float, true, DM><<<grid, block, 0, st>>>(                                   \
                     (const float*)q, (const float*)k, (const float*)v, (const float*)d_o, lse, D, (float*)d_k,  \
                     (float*)d_v, P, g), 0)                                                                      \
              : (dkdv_generic<float, float, false, DM><<<grid, block, 0, st>>>(                                  \
                     (const float*)q, (const float*)k, (const float*)v, (const float*)d_o, lse, D, (float*)d_k,  \
                     (float*)d_v, P, g), 0))                                                                     \
       : (acc ? (dkdv_generic<uint16_t, float, true, DM><<<grid, block, 0, st>>>(                                \
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse, D,   \
                     (float*)d_k, (float*)d_v, P, g), 0)                                                         \
              : (dkdv_generic<uint16_t, uint16_t, false, DM><<<grid, block, 0, st>>>(                            \
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse, D,   \
                     (uint16_t*)d_k, (uint16_t*)d_v, P, g), 0)))
  TT_DMAX_DISPATCH(g.d, KV);
#undef KV
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------- accumulator pop
// dK (y = 0) and dV (y = 1) rows leaving the path stack: the sum of nslot
// fp32 accumulators (slot u at acc + u * slot_stride), rounded to bf16; the
// accumulators' rows are cleared for the next segment at these positions.
__global__ __launch_bounds__(256) void acc_pop_kernel(float* __restrict__ acc_k, float* __restrict__ acc_v,
                                                      int64_t slot_stride, int nslot, uint16_t* __restrict__ out_k,
                                                      uint16_t* __restrict__ out_v, int64_t n4) {
  float* a = blockIdx.y ? acc_v : acc_k;
  uint2* o = reinterpret_cast<uint2*>(blockIdx.y ? out_v : out_k);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += int64_t(gridDim.x) * blockDim.x) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int u = 0; u < nslot; ++u) {
      float4* p = reinterpret_cast<float4*>(a + u * slot_stride) + i;
      const float4 x = *p;
      t.x += x.x;
      t.y += x.y;
      t.z += x.z;
      t.w += x.w;
      *p = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    o[i] = make_uint2(uint32_t(f2bf(t.x)) | (uint32_t(f2bf(t.y)) << 16),
                      uint32_t(f2bf(t.z)) | (uint32_t(f2bf(t.w)) << 16));
  }
}

int launch_acc_pop(float* acc_k, float* acc_v, int64_t slot_stride, int nslot, void* out_k, void* out_v, int64_t n,
                   hipStream_t st) {
  if (n <= 0) return 0;
  if (n % 4 != 0 || slot_stride % 4 != 0 || nslot < 1) return -1;
  const int64_t n4 = n / 4;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 2048);
  acc_pop_kernel<<<dim3(unsigned(blocks), 2), dim3(256), 0, st>>>(acc_k, acc_v, slot_stride, nslot,
                                                                   static_cast<uint16_t*>(out_k),
                                                                   static_cast<uint16_t*>(out_v), n4);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------- fill
// Zeroes a device buffer (bytes a multiple of 4) with plain vector stores, so
// that code a caller may capture into a graph records no memset node.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t n = int64_t(bytes / 4);
  if (n == 0) return 0;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  fill_zero_kernel<<<dim3(unsigned(blocks)), dim3(256), 0, st>>>(static_cast<uint32_t*>(p), n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
