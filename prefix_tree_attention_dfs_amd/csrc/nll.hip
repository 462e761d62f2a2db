// Weighted log-softmax NLL over the tree's logits rows (Tree Training, Abstract:
// the branch-averaged loss equals the per-token loss weighted by the fraction
// of branches through the token).  Row r predicts the tokens of its children:
//   loss_r = sum_t w_t (lse_r - z_r[x_t]),  logp_t = z_r[x_t] - lse_r,
//   dZ_r   = W_r softmax(z_r) - sum_t w_t e_{x_t},  W_r = sum_t w_t.
// dZ may overwrite z (in place): target positions are kept intact until their
// own value is written, so every dZ element is rounded exactly once.
#include "device.h"
#include "kernels.h"

using namespace ttd;

namespace {

constexpr int kThreads = 256;
constexpr int kMaxVocab = 1 << 18;  // LDS bitmap of target positions: 32 KB

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mn = fmaxf(m, m2);
  s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
  m = mn;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void nll_rows_kernel(const T* z, T* dz, int32_t vocab,
                                                            int64_t ldz, const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ tgt_id,
                                                            const float* __restrict__ tgt_w, int32_t n_tgt,
                                                            float* __restrict__ logp, float* __restrict__ row_loss) {
  __shared__ uint32_t bitmap[kMaxVocab / 32];
  __shared__ float red_m[kThreads / kWave], red_s[kThreads / kWave];
  __shared__ float red_a[kThreads / kWave], red_b[kThreads / kWave];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const T* zr = z + int64_t(r) * ldz;
  // pass 1: max and sum of exp (online, per thread, then merged)
  float m = -INFINITY, s = 0.f;
  for (int v = tid; v < vocab; v += kThreads) {
    const float x = Elem<T>::load(zr, v);
    if (x > m) {
      s = s * __expf(m - x) + 1.f;
      m = x;
    } else {
      s += __expf(x - m);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
    merge_ms(m, s, m2, s2);
  }
  if (lane == 0) {
    red_m[wv] = m;
    red_s[wv] = s;
  }
  const int words = (vocab + 31) / 32;
  for (int w = tid; w < words; w += kThreads) bitmap[w] = 0u;
  __syncthreads();
  m = red_m[0];
  s = red_s[0];
  for (int w = 1; w < kThreads / kWave; ++w) merge_ms(m, s, red_m[w], red_s[w]);
  const float lse = m + logf(s);
  // pass 2: targets -> logp, loss, row weight; mark target positions
  // targets outside [0, n_tgt) or ids outside [0, vocab) are ignored (logp = NaN)
  const int t0 = min(max(row_ptr[r], 0), n_tgt), t1 = min(max(row_ptr[r + 1], t0), n_tgt);
  float loss = 0.f, W = 0.f;
  for (int t = t0 + tid; t < t1; t += kThreads) {
    const int x = tgt_id[t];
    if (x < 0 || x >= vocab) {
      if (logp) logp[t] = NAN;
      continue;
    }
    const float w = tgt_w[t];
    const float lp = Elem<T>::load(zr, x) - lse;
    if (logp) logp[t] = lp;
    loss -= w * lp;
    W += w;
    atomicOr(&bitmap[x >> 5], 1u << (x & 31));
  }
  loss = wave_sum(loss);
  W = wave_sum(W);
  if (lane == 0) {
    red_a[wv] = loss;
    red_b[wv] = W;
  }
  __syncthreads();
  loss = 0.f;
  W = 0.f;
  for (int w = 0; w < kThreads / kWave; ++w) {
    loss += red_a[w];
    W += red_b[w];
  }
  if (tid == 0) row_loss[r] = loss;
  if (dz == nullptr) return;
  T* dr = dz + int64_t(r) * ldz;
  // pass 3a: every non-target position
  for (int v = tid; v < vocab; v += kThreads) {
    if (bitmap[v >> 5] & (1u << (v & 31))) continue;
    Elem<T>::store(dr, v, W * __expf(Elem<T>::load(zr, v) - lse));
  }
  __syncthreads();
  // pass 3b: each distinct target position, claimed by the first thread to clear its bit
  for (int t = t0 + tid; t < t1; t += kThreads) {
    const int x = tgt_id[t];
    if (x < 0 || x >= vocab) continue;
    const uint32_t bit = 1u << (x & 31);
    if (!(atomicAnd(&bitmap[x >> 5], ~bit) & bit)) continue;
    float ws = 0.f;
    for (int u = t0; u < t1; ++u)
      if (tgt_id[u] == x) ws += tgt_w[u];
    Elem<T>::store(dr, x, W * __expf(Elem<T>::load(zr, x) - lse) - ws);
  }
}

// bf16 rows that fit in registers (vocab <= 8 * kRegThreads * kRegChunks,
// vocab and ldz multiples of 8): 1024 threads hold the whole row as 16-byte
// chunks, so Z is read once and dZ written once, both 16 bytes per lane.
// Same arithmetic as nll_rows_kernel (max, sum of exp, targets, one rounding
// per dZ element, targets written last from their original logits).
constexpr int kRegThreads = 1024;
constexpr int kRegChunks = 19;  // 8 * 1024 * 19 = 155,648 logits per row
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16x8 __attribute__((ext_vector_type(8)));
constexpr float kL2e = 1.4426950408889634f;
// exp(x - c) as one FMA and v_exp_f32: 2^(x log2 e - c log2 e), cl = c log2 e
__device__ __forceinline__ float exp_shift(float x, float cl) { return __builtin_amdgcn_exp2f(fmaf(x, kL2e, -cl)); }

__global__ __launch_bounds__(kRegThreads) void nll_rows_reg_kernel(const uint16_t* z, uint16_t* dz, int32_t vocab,
                                                                   int64_t ldz, const int32_t* __restrict__ row_ptr,
                                                                   const int32_t* __restrict__ tgt_id,
                                                                   const float* __restrict__ tgt_w, int32_t n_tgt,
                                                                   float* __restrict__ logp,
                                                                   float* __restrict__ row_loss) {
  __shared__ uint32_t bitmap[kMaxVocab / 32];
  __shared__ float red_a[kRegThreads / kWave], red_b[kRegThreads / kWave];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint16_t* zr = z + int64_t(r) * ldz;
  const int nchunk = vocab >> 3;
  u16x8 x[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int ch = c * kRegThreads + tid;
    if (ch < nchunk) x[c] = *reinterpret_cast<const u16x8*>(zr + 8 * int64_t(ch));
  }
  const int words = (vocab + 31) / 32;
  for (int w = tid; w < words; w += kRegThreads) bitmap[w] = 0u;
  // pass 1: row max, then sum of exp
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (c * kRegThreads + tid < nchunk)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, bf2f(x[c][e]));
  m = wave_max(m);
  if (lane == 0) red_a[wv] = m;
  __syncthreads();
  m = red_a[0];
  for (int w = 1; w < kRegThreads / kWave; ++w) m = fmaxf(m, red_a[w]);
  float s = 0.f;
  const float ml = m * kL2e;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (c * kRegThreads + tid < nchunk)
#pragma unroll
      for (int e = 0; e < 8; ++e) s += exp_shift(bf2f(x[c][e]), ml);
  s = wave_sum(s);
  __syncthreads();  // red_a reused
  if (lane == 0) red_b[wv] = s;
  __syncthreads();
  s = 0.f;
  for (int w = 0; w < kRegThreads / kWave; ++w) s += red_b[w];
  const float lse = m + logf(s);
  // pass 2: targets -> logp, loss, row weight; mark target positions
  const int t0 = min(max(row_ptr[r], 0), n_tgt), t1 = min(max(row_ptr[r + 1], t0), n_tgt);
  float loss = 0.f, W = 0.f;
  for (int t = t0 + tid; t < t1; t += kRegThreads) {
    const int xi = tgt_id[t];
    if (xi < 0 || xi >= vocab) {
      if (logp) logp[t] = NAN;
      continue;
    }
    const float w = tgt_w[t];
    const float lp = bf2f(zr[xi]) - lse;
    if (logp) logp[t] = lp;
    loss -= w * lp;
    W += w;
    atomicOr(&bitmap[xi >> 5], 1u << (xi & 31));
  }
  loss = wave_sum(loss);
  W = wave_sum(W);
  __syncthreads();  // red_b read above
  if (lane == 0) {
    red_a[wv] = loss;
    red_b[wv] = W;
  }
  __syncthreads();
  loss = 0.f;
  W = 0.f;
  for (int w = 0; w < kRegThreads / kWave; ++w) {
    loss += red_a[w];
    W += red_b[w];
  }
  if (tid == 0) row_loss[r] = loss;
  if (dz == nullptr) return;
  uint16_t* dr = dz + int64_t(r) * ldz;
  const float lsel = lse * kL2e;
  // pass 3a: every non-target position, 16 bytes at a time where a chunk holds
  // no target; rounded to bf16 (nearest even) two at a time by the hardware
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int ch = c * kRegThreads + tid;
    if (ch >= nchunk) continue;
    const uint32_t bits = (bitmap[ch >> 2] >> ((ch & 3) * 8)) & 0xFFu;  // the chunk's 8 target bits
    b16x8 yb;
#pragma unroll
    for (int e = 0; e < 8; ++e) yb[e] = __bf16(W * exp_shift(bf2f(x[c][e]), lsel));
    const u16x8 y = __builtin_bit_cast(u16x8, yb);
    if (bits == 0u) {
      *reinterpret_cast<u16x8*>(dr + 8 * int64_t(ch)) = y;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(bits & (1u << e))) dr[8 * int64_t(ch) + e] = y[e];
    }
  }
  __syncthreads();
  // pass 3b: each distinct target position, claimed by the first thread to clear its bit
  for (int t = t0 + tid; t < t1; t += kRegThreads) {
    const int xi = tgt_id[t];
    if (xi < 0 || xi >= vocab) continue;
    const uint32_t bit = 1u << (xi & 31);
    if (!(atomicAnd(&bitmap[xi >> 5], ~bit) & bit)) continue;
    float ws = 0.f;
    for (int u = t0; u < t1; ++u)
      if (tgt_id[u] == xi) ws += tgt_w[u];
    dr[xi] = f2bf(W * exp_shift(bf2f(zr[xi]), lsel) - ws);
  }
}

__global__ __launch_bounds__(kThreads) void sum_loss_kernel(const float* __restrict__ row_loss, int32_t n,
                                                            float* __restrict__ loss) {
  __shared__ double red[kThreads / kWave];
  double a = 0.0;
  for (int i = threadIdx.x; i < n; i += kThreads) a += double(row_loss[i]);
  a = wave_sum(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
    *loss = float(t);
  }
}

}  // namespace

int launch_nll_rows(tt_dtype zt, const void* z, void* dz, int32_t n_rows, int32_t vocab, int64_t ldz,
                    const int32_t* row_ptr, const int32_t* tgt_id, const float* tgt_w, int32_t n_tgt, float* logp,
                    float* row_loss, hipStream_t st) {
  if (vocab > kMaxVocab) return -1;
  if (n_rows == 0) return 0;
  if (zt == TT_F32)
    nll_rows_kernel<float><<<n_rows, kThreads, 0, st>>>((const float*)z, (float*)dz, vocab, ldz, row_ptr, tgt_id,
                                                        tgt_w, n_tgt, logp, row_loss);
  else if (vocab % 8 == 0 && ldz % 8 == 0 && vocab <= 8 * kRegThreads * kRegChunks &&
           (reinterpret_cast<uintptr_t>(z) & 15) == 0 && (reinterpret_cast<uintptr_t>(dz) & 15) == 0)
    nll_rows_reg_kernel<<<n_rows, kRegThreads, 0, st>>>((const uint16_t*)z, (uint16_t*)dz, vocab, ldz, row_ptr,
                                                        tgt_id, tgt_w, n_tgt, logp, row_loss);
  else
    nll_rows_kernel<uint16_t><<<n_rows, kThreads, 0, st>>>((const uint16_t*)z, (uint16_t*)dz, vocab, ldz, row_ptr,
                                                           tgt_id, tgt_w, n_tgt, logp, row_loss);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_sum_loss(const float* row_loss, int32_t n, float* loss, hipStream_t st) {
  sum_loss_kernel<<<1, kThreads, 0, st>>>(row_loss, n, loss);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------- no-allocation entry point
// tree_weighted_nll_noalloc: the logits mode of tree_weighted_nll with its
// per-row partial losses in a static device array instead of the caller's
// workspace, for callers that cannot allocate (graph capture, tight loops).
// Every GPU the library runs on holds its own copy of the array until the
// process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device.
#include <mutex>

#include "attn_core.h"

namespace {

constexpr int32_t kNoAllocMaxRows = 1 << 20;  // 4 MiB of float32 row losses per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kNoAllocMaxRows];

std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_for_current_device(float** out, const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return tt::fail(TT_EDEVICE, std::string(fn) + ": no usable current device");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return tt::fail(TT_EDEVICE, std::string(fn) + ": hipGetSymbolAddress(scratch) failed: " + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return TT_OK;
}

}  // namespace

extern "C" int tree_weighted_nll_noalloc(const tt_nll_args* a, tt_stream stream) {
  tt::clear_error();
  const char* fn = "tree_weighted_nll_noalloc";
  int rc = ttc::nll_check(a, fn);
  if (rc) return rc;
  if (!a->logits)
    return tt::fail(TT_EUNSUPPORTED, std::string(fn) + ": logits mode only (the fused mode needs a rows x vocab "
                                                       "workspace; use tree_weighted_nll)");
  if (a->n_rows > kNoAllocMaxRows)
    return tt::fail(TT_EWORKSPACE, std::string(fn) + ": n_rows " + std::to_string(a->n_rows) + " exceeds the " +
                                       std::to_string(kNoAllocMaxRows) + " rows of the static scratch");
  float* row_loss = nullptr;
  if ((rc = scratch_for_current_device(&row_loss, fn))) return rc;
  hipStream_t st = (hipStream_t)stream;
  {
    ttc::KTimer t("nll_rows", st);
    if (launch_nll_rows(a->logits_dtype, a->logits, a->d_logits, a->n_rows, a->vocab, a->vocab, a->tgt_row_ptr,
                        a->tgt_id, a->tgt_w, a->n_tgt, a->logp, row_loss, st))
      return ttc::dev_fail(fn, "nll kernel launch");
  }
  ttc::KTimer t("nll_sum", st);
  if (launch_sum_loss(row_loss, a->n_rows, a->loss, st)) return ttc::dev_fail(fn, "loss reduction");
  return TT_OK;
}
