// bf16 MFMA GEMMs of the fused lm-head (gfx950): C[M][N] = sum_k A(m,k) B(k,n).
//
// Tree Training (arXiv 2511.00413), Abstract: the branch-averaged loss is a
// per-token weighted loss, so the lm-head runs once per unique tree token:
//   Z  = H W           (NN: A = H [M][K],  B = W [K][N])
//   dH = dZ W^T        (NT: A = dZ [M][K'], B stored [N][K'] = W)
//   dW = H^T dZ        (TN: A stored [K][M] = H, B = dZ [K][N])
//
// Block tile 256 x 256, k-step 64, 16 waves of 64 x 64 (2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, 64 accumulator registers, at most 128 VGPRs), so
// that four waves share each SIMD and some issue products while others wait
// on loads, the barrier or the epilogue; double-buffered LDS.  Operands whose reduction
// index is contiguous in memory are read with ds_read_b128 (or two b64 reads
// matching the permuted reduction order below); operands stored with the
// reduction index strided are read with ds_read_tr16_b64, which returns rows
// k0 + {4h..4h+3, 8+4h..8+4h+3} for lane half h -- when one operand is read
// that way, the other is read in the same reduction order.
#include "device.h"
#include "kernels.h"
#include "mfma_common.h"

using namespace ttm;

namespace {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GTHREADS = 1024;  // 16 waves: 4 (m) x 4 (n), each 64 x 64
constexpr int WTN = 2;          // 32-column tiles per wave
constexpr int WTM = 2;          // 32-row tiles per wave
// LDS row strides (elements), chosen for gfx950's 64 banks: 16-byte reads are
// served 16 lanes per cycle, 8-byte and transposed reads 32 lanes per cycle.
constexpr int KROW = GBK + 8;    // rows along k, read 16 bytes per lane (144-byte rows)
constexpr int KROW8 = GBK + 4;   // rows along k, read 8 bytes per lane (136 bytes: 32 rows on distinct banks)
constexpr int XROW = GBN + 32;   // rows along m or n, read transposed (576 bytes: 4 rows x 64 bytes on distinct banks)

template <bool A_T, bool B_T>
struct GemmLds {
  static constexpr bool PERM = A_T || !B_T;  // some operand is read transposed: permuted reduction order
  static constexpr int A_STRIDE = A_T ? XROW : (PERM ? KROW8 : KROW);
  static constexpr int B_STRIDE = B_T ? KROW : XROW;
  // A tile: [GBM][A_STRIDE] (m rows, k contiguous) or [GBK][XROW] (k rows, m contiguous)
  static constexpr int A_ELEMS = A_T ? GBK * XROW : GBM * A_STRIDE;
  static constexpr int B_ELEMS = B_T ? GBN * KROW : GBK * XROW;
};

// Loads a 256 x 64 (or 64 x 256) bf16 tile of a row-major matrix in 16-byte
// chunks; out-of-range rows/chunks read a clamped address and are zeroed.
// Every column count here is a multiple of 8 (checked by the caller), so a
// chunk is either wholly inside or wholly outside the matrix.
template <bool KROWS>  // true: tile rows are the matrix rows (k contiguous, 64 wide)
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ X, int64_t ld, int64_t r0, int64_t c0,
                                          int64_t nrows, int64_t ncols, int tid, bf16x8 (&reg)[2]) {
  // KROWS: tile = 256 rows x 64 cols (8 chunks per row); else 64 rows x 256 cols (32 chunks per row)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * GTHREADS;
    const int row = KROWS ? (c >> 3) : (c >> 5);
    const int col = KROWS ? ((c & 7) << 3) : ((c & 31) << 3);
    const int64_t gr = r0 + row, gc = c0 + col;
    const bool ok = gr < nrows && gc + 8 <= ncols;
    const int64_t cr = gr < nrows ? gr : nrows - 1;
    const int64_t cc = gc + 8 <= ncols ? gc : 0;
    const bf16x8 x = ld16(X + cr * ld + cc);
    reg[u] = ok ? x : zero8();
  }
}

template <bool KROWS, int STRIDE>
__device__ __forceinline__ void store_tile(uint16_t* s, int tid, const bf16x8 (&reg)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * GTHREADS;
    const int row = KROWS ? (c >> 3) : (c >> 5);
    const int col = KROWS ? ((c & 7) << 3) : ((c & 31) << 3);
    if constexpr (STRIDE % 8 == 0) {
      *reinterpret_cast<bf16x8*>(s + row * STRIDE + col) = reg[u];
    } else {  // rows only 8-byte aligned: two 8-byte stores
      bf16x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = reg[u][e];
        hi[e] = reg[u][4 + e];
      }
      *reinterpret_cast<bf16x4*>(s + row * STRIDE + col) = lo;
      *reinterpret_cast<bf16x4*>(s + row * STRIDE + col + 4) = hi;
    }
  }
}

// OUT: 0 = bf16 store, 1 = f32 store
template <bool A_T, bool B_T, int OUT>
__global__ __launch_bounds__(GTHREADS) void gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                        void* __restrict__ Cv, int64_t M, int64_t N, int64_t K,
                                                        int tiles_n) {
  using L = GemmLds<A_T, B_T>;
  extern __shared__ __align__(16) uint16_t smem[];
  constexpr int STAGE = L::A_ELEMS + L::B_ELEMS;  // stage s: A at s*STAGE, B right after
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;  // 4 x 4
  // block -> tile; consecutive blocks share a B column panel
  const int tm = blockIdx.x % ((M + GBM - 1) / GBM);
  const int tn = blockIdx.x / ((M + GBM - 1) / GBM);
  (void)tiles_n;
  const int64_t m0 = int64_t(tm) * GBM, n0 = int64_t(tn) * GBN;
  // leading dimensions (row-major storage)
  const int64_t lda = A_T ? M : K;  // A stored [M][K] or [K][M]
  const int64_t ldb = B_T ? K : N;  // B stored [K][N] or [N][K]

  bf16x8 ra[2], rb[2];
  auto gload = [&](int64_t k0) {
    if (A_T)
      load_tile<false>(A, lda, k0, m0, K, M, tid, ra);
    else
      load_tile<true>(A, lda, m0, k0, M, K, tid, ra);
    if (B_T)
      load_tile<true>(B, ldb, n0, k0, N, K, tid, rb);
    else
      load_tile<false>(B, ldb, k0, n0, K, N, tid, rb);
  };
  auto sstore = [&](int s) {
    uint16_t* sa = smem + s * STAGE;
    uint16_t* sb = sa + L::A_ELEMS;
    if (A_T)
      store_tile<false, XROW>(sa, tid, ra);
    else
      store_tile<true, L::A_STRIDE>(sa, tid, ra);
    if (B_T)
      store_tile<true, KROW>(sb, tid, rb);
    else
      store_tile<false, XROW>(sb, tid, rb);
  };

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = zero16();

  const int nk = int((K + GBK - 1) / GBK);
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  // reduction order: natural (8h + s) unless some operand is read transposed
  constexpr bool PERM = L::PERM;
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) gload(int64_t(kt + 1) * GBK);
    const uint16_t* a_s = smem + s * STAGE;
    const uint16_t* b_s = a_s + L::A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 af[WTM], bfr[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const int mrow = wm * 64 + i * 32;
        if (A_T) {
          af[i] = tr_frag(a_s, XROW, ks * 16, mrow, lane);
        } else if (PERM) {
          const uint16_t* p = a_s + (mrow + r) * L::A_STRIDE + ks * 16 + 4 * hh;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            af[i][e] = lo[e];
            af[i][4 + e] = hi[e];
          }
        } else {
          af[i] = lds_read16(a_s + (mrow + r) * L::A_STRIDE + ks * 16 + 8 * hh);
        }
      }
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const int ncol = wn * 64 + j * 32;
        if (B_T)
          bfr[j] = lds_read16(b_s + (ncol + r) * KROW + ks * 16 + 8 * hh);
        else
          bfr[j] = tr_frag(b_s, XROW, ks * 16, ncol, lane);
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(s ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m = 8*(e/4) + 4hh + e%4][n = r] of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (m >= M) continue;
        if (OUT == 0)
          static_cast<uint16_t*>(Cv)[m * N + n] = ttd::f2bf(acc[i][j][e]);
        else
          static_cast<float*>(Cv)[m * N + n] = acc[i][j][e];
      }
    }
}

template <bool A_T, bool B_T, int OUT>
int launch_gemm(const uint16_t* A, const uint16_t* B, void* C, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 0 || N <= 0) return 0;
  const int64_t tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
  if (tm * tn >= (int64_t(1) << 31)) return -1;
  using L = GemmLds<A_T, B_T>;
  const size_t lds = size_t(2) * (L::A_ELEMS + L::B_ELEMS) * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<A_T, B_T, OUT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
      return -1;
    attr_set = true;
  }
  gemm_kernel<A_T, B_T, OUT><<<dim3(unsigned(tm * tn)), dim3(GTHREADS), lds, st>>>(A, B, C, M, N, K, int(tn));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_gemm_nn(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N, int64_t K,
                   hipStream_t st) {
  return launch_gemm<false, false, 0>(A, B, C, M, N, K, st);
}

int launch_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N, int64_t K,
                   hipStream_t st) {
  return launch_gemm<false, true, 0>(A, B, C, M, N, K, st);
}

int launch_gemm_tn(const uint16_t* A, const uint16_t* B, void* C, bool c_f32, int64_t M, int64_t N, int64_t K,
                   hipStream_t st) {
  return c_f32 ? launch_gemm<true, false, 1>(A, B, C, M, N, K, st) : launch_gemm<true, false, 0>(A, B, C, M, N, K, st);
}
