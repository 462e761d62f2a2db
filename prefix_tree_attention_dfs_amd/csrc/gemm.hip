// bf16 MFMA GEMMs of the fused lm-head (gfx950): C[M][N] = sum_k A(m,k) B(k,n).
//
// Tree Training (arXiv 2511.00413), Abstract: the branch-averaged loss is a
// per-token weighted loss, so the lm-head runs once per unique tree token:
//   Z  = H W           (NN: A = H [M][K],  B = W [K][N])
//   dH = dZ W^T        (NT: A = dZ [M][K'], B stored [N][K'] = W)
//   dW = H^T dZ        (TN: A stored [K][M] = H, B = dZ [K][N])
//
// Block tile 256 x 256, 8 waves of 128 x 64 (4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, two waves per SIMD).  The reduction is staged 64
// at a time through two LDS buffers of 64 KB, filled by 16-byte buffer loads
// that write straight into LDS one stage ahead of the one being multiplied
// (a stage is ~2000 cycles of matrix work per SIMD).  One barrier per stage
// publishes it and frees the buffer its loads go into; 32-deep stages with
// three in flight took twice the barriers and ran 7% slower.
//
// A tile operand is stored one of two ways, each swizzled at 16-byte chunks
// so that its reads are free of LDS bank conflicts (64 banks of 4 bytes;
// 16-byte reads are served 16 lanes per cycle, 8-byte reads 32):
//   * k contiguous (rows = m or n, 64 k = 128-byte rows): chunk c of row q
//     at chunk c ^ ((q >> 1) & 7).  A fragment is a 16-byte read per lane at
//     row row0 + r, chunk 2 ks + h; 16 consecutive rows, (q & 1) choosing the
//     half of the bank space and the swizzle the chunk, cover all 16 bank
//     groups.
//   * k strided (rows = k, 256 m or n = 512-byte rows): chunk c of row k at
//     chunk c ^ ((k & 3) << 2).  A fragment is two ds_read_tr16_b64, rows
//     8h..8h+3 and 8h+4..8h+7 of the 16-row step, so every operand comes out
//     in the natural reduction order (lane (r, h) holds k = 8h .. 8h+7); the
//     32 lanes of a read cover 4 consecutive rows x 4 adjacent chunks, which
//     the swizzle spreads over all 16 bank groups.
// The buffer descriptor of a stage is built from the tile's own origin, so
// matrices above 4 GB (Z) need no 64-bit offsets; a lane whose chunk lies
// outside the matrix gets an offset past the descriptor's record count, for
// which the load writes zeros.  Every column count of a k-strided operand and
// the reduction length of a k-contiguous one are multiples of 8 (checked by
// the caller), so a chunk is either wholly inside or wholly outside.
#include "device.h"
#include "kernels.h"
#include "mfma_common.h"

using namespace ttm;

namespace {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GSTAGES = 2;
constexpr int GWAVES = 8;  // 2 (m) x 4 (n), each 128 x 64
constexpr int GTHREADS = GWAVES * 64;
constexpr int WTM = 4;  // 32-row tiles per wave
constexpr int WTN = 2;  // 32-column tiles per wave
constexpr uint32_t TILE_BYTES = 256 * GBK * 2;          // 16 KB, either layout
constexpr uint32_t STAGE_BYTES = 2 * TILE_BYTES;        // A then B
constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / GWAVES;  // 1 KB per load instruction
static_assert(LOADS_PER_WAVE == 4, "staging assumes four loads per wave per operand");
constexpr uint32_t kRecords = 0x7FFFFFF0u;  // descriptor size: every in-matrix offset is below it
constexpr uint32_t kOut = 0x80000000u;      // offset past it: the load writes zeros

// s_waitcnt with vmcnt = n (n < 16), expcnt and lgkmcnt left at their maxima
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Per-lane staging of one operand tile.  Lane l of the wave's load u fills
// LDS slot p = 64 (4 wave + u) + l; `off` is the byte offset of the global
// chunk it fetches relative to the stage's tile origin (kOut when the chunk's
// row or column is outside the matrix), `kpos` the chunk's reduction index
// within the stage (checked only in a ragged last stage).
template <bool KCONTIG>
__device__ __forceinline__ void stage_lane(int wave, int lane, int64_t ld, int64_t rc0, int64_t nrc, uint32_t (&off)[LOADS_PER_WAVE],
                                           int (&kpos)[LOADS_PER_WAVE]) {
#pragma unroll
  for (int u = 0; u < LOADS_PER_WAVE; ++u) {
    const int p = 64 * (LOADS_PER_WAVE * wave + u) + lane;
    if (KCONTIG) {  // row q (m or n) holds 8 chunks of k
      const int q = p >> 3, c = (p & 7) ^ ((q >> 1) & 7);
      off[u] = rc0 + q < nrc ? uint32_t(q * ld * 2 + 16 * c) : kOut;
      kpos[u] = 8 * c;
    } else {  // row k holds 32 chunks of m or n
      const int k = p >> 5, c = (p & 31) ^ ((k & 3) << 2);
      off[u] = rc0 + 8 * c < nrc ? uint32_t(k * ld * 2 + 16 * c) : kOut;
      kpos[u] = k;
    }
  }
}

// OUT: 0 = bf16 store, 1 = f32 store.  128 KB of LDS allows one workgroup
// per CU, i.e. two waves per SIMD: the compiler may use all 256 VGPRs to
// issue fragment reads early.
template <bool A_T, bool B_T, int OUT>
__global__ __launch_bounds__(GTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                        void* __restrict__ Cv, int64_t M, int64_t N, int64_t K) {
  // The output pointer is consumed here, so its scalar load completes in the
  // prologue: a scalar load still in flight would make every LDS wait in the
  // loop a wait for all outstanding LDS reads.
  if (Cv == nullptr) return;
  __shared__ __align__(16) uint16_t smem[GSTAGES * STAGE_BYTES / 2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  // Block -> tile.  Workgroups go to the 8 XCDs in turn (block b to XCD
  // b % 8), 32 at a time per XCD.  Z = H W: consecutive blocks share a B
  // column panel, and with 64 row tiles the 32 blocks an XCD holds span 8 row
  // and 4 column panels.  dH and dW: the grid is walked in 16 x 16-tile
  // regions, XCD x taking rows 8 (x % 2) .. +7 and columns 4 (x / 2) .. +3 of
  // each, so the 256 blocks in flight read 16 + 16 panels instead of up to 64
  // + 4 (dH) or 16 + 32 (dW); with reductions of 151936 and 16384 those
  // panels stream for the whole launch (measured 4% on each; 1.7% slower for
  // Z, whose H stays in the Infinity Cache).  Tiles outside whole regions
  // keep the plain order.
  const int tiles_m = int((M + GBM - 1) / GBM), tiles_n = int((N + GBN - 1) / GBN);
  int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  if (A_T || B_T) {
    const int rm_n = tiles_m / 16, rn_n = tiles_n / 16;
    const int full = rm_n * rn_n * 256;
    const int b = blockIdx.x;
    if (b < full) {
      const int reg = b >> 8, i = b & 255, x = i & 7, jx = i >> 3;
      tm = (reg % rm_n) * 16 + (x & 1) * 8 + (jx & 7);
      tn = (reg / rm_n) * 16 + (x >> 1) * 4 + (jx >> 3);
    } else {
      int e = b - full;
      const int right = tiles_m * (tiles_n - rn_n * 16);  // columns past the regions, every row
      if (e < right) {
        tm = e % tiles_m;
        tn = rn_n * 16 + e / tiles_m;
      } else {  // rows past the regions, the regions' columns
        e -= right;
        const int w = tiles_m - rm_n * 16;
        tm = rm_n * 16 + e % w;
        tn = e / w;
      }
    }
  }
  const int64_t m0 = int64_t(tm) * GBM, n0 = int64_t(tn) * GBN;
  const int64_t lda = A_T ? M : K;  // A stored [M][K] or [K][M]
  const int64_t ldb = B_T ? K : N;  // B stored [K][N] or [N][K]

  uint32_t offa[LOADS_PER_WAVE], offb[LOADS_PER_WAVE];
  int kpa[LOADS_PER_WAVE], kpb[LOADS_PER_WAVE];
  stage_lane<!A_T>(wave, lane, lda, m0, M, offa, kpa);
  stage_lane<B_T>(wave, lane, ldb, n0, N, offb, kpb);
  const uint32_t lds0 = lds_u32(smem);

  // loads of reduction stage kt into buffer kt % GSTAGES (eight per wave)
  const int nk = int((K + GBK - 1) / GBK);
  auto issue = [&](int kt) {
    const int64_t k0 = int64_t(kt) * GBK, krem = K - k0;
    const uint32_t la = lds0 + uint32_t(kt % GSTAGES) * STAGE_BYTES + uint32_t(LOADS_PER_WAVE * wave) * 1024u;
    const uint32_t lb = la + TILE_BYTES;
    const rsrc_t ra = make_rsrc(A_T ? A + k0 * lda + m0 : A + m0 * lda + k0, kRecords);
    const rsrc_t rb = make_rsrc(B_T ? B + n0 * ldb + k0 : B + k0 * ldb + n0, kRecords);
    if (krem >= GBK) {
#pragma unroll
      for (int u = 0; u < LOADS_PER_WAVE; ++u) dma16(ra, offa[u], 0, la + 1024u * u);
#pragma unroll
      for (int u = 0; u < LOADS_PER_WAVE; ++u) dma16(rb, offb[u], 0, lb + 1024u * u);
    } else {
#pragma unroll
      for (int u = 0; u < LOADS_PER_WAVE; ++u) dma16(ra, kpa[u] < krem ? offa[u] : kOut, 0, la + 1024u * u);
#pragma unroll
      for (int u = 0; u < LOADS_PER_WAVE; ++u) dma16(rb, kpb[u] < krem ? offb[u] : kOut, 0, lb + 1024u * u);
    }
  };

  // Fragment addresses (bytes within a tile) of this lane.  k contiguous:
  // row row0 + r, chunk 2 ks + hh; the swizzle term depends on r alone since
  // row0 is a multiple of 32.  k strided: group g = lane / 16 reads rows
  // 16 ks + 8 (g / 2) + (lane % 16) / 4 (+4 for the second half), columns
  // col0 + 16 (g % 2) + 4 (lane % 4) .. +3.
  constexpr int NKS = GBK / 16;
  const int rsw = (r >> 1) & 7;
  uint32_t rowfrag[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) rowfrag[ks] = uint32_t(r * 128 + (((2 * ks + hh) ^ rsw) << 4));
  const int g = lane >> 4, rr = lane & 15;
  const int csw = ((rr >> 2) & 3) << 2;
  const uint32_t colrow = uint32_t((8 * (g >> 1) + (rr >> 2)) * 512 + (rr & 1) * 8);
  const int clow = 2 * (g & 1) + ((rr & 3) >> 1);  // chunk within the 4-chunk group
  auto colfrag_off = [&](int col0) {  // col0: multiple of 32
    return colrow + uint32_t((((col0 >> 3) ^ csw) + clow) << 4);
  };

  f32x16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = zero16();

  // byte offsets of this wave's fragments within the A and B tiles
  uint32_t afo[WTM][NKS], bfo[WTN][NKS];
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    const int mrow = wm * 128 + i * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      afo[i][ks] = A_T ? colfrag_off(mrow) + ks * 16 * 512 : uint32_t(mrow * 128) + rowfrag[ks];
  }
#pragma unroll
  for (int j = 0; j < WTN; ++j) {
    const int ncol = wn * 64 + j * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      bfo[j][ks] = B_T ? uint32_t(ncol * 128) + rowfrag[ks] : colfrag_off(ncol) + ks * 16 * 512;
  }
  const char* lds_c = reinterpret_cast<const char*>(smem);
  auto frag = [&](bool tr, uint32_t byte) -> bf16x8 {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(lds_c + byte);
    if (!tr) return lds_read16(p);
    const bf16x4 lo = lds_tr4(p), hi = lds_tr4(p + 4 * 256);  // rows +4: same swizzle, 2 KB further
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = lo[e];
      a[4 + e] = hi[e];
    }
    return a;
  };

  // fragments of one 16-deep step of the stage in buffer b
  auto load_frags = [&](int b, int ks, bf16x8 (&af)[WTM], bf16x8 (&bfr)[WTN]) {
    const uint32_t sa = uint32_t(b) * STAGE_BYTES, sb = sa + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < WTM; ++i) af[i] = frag(A_T, sa + afo[i][ks]);
#pragma unroll
    for (int j = 0; j < WTN; ++j) bfr[j] = frag(!B_T, sb + bfo[j][ks]);
  };
  auto mma = [&](const bf16x8 (&af)[WTM], const bf16x8 (&bfr)[WTN]) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j) acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);
  };
  // Two 64-deep stages: the loads of stage kt + 1 are issued right after
  // the barrier that publishes stage kt, and the products of stage kt's last
  // 16-deep step are issued after the next barrier, behind the first reads
  // of stage kt + 1.
  bf16x8 a0[WTM], b0[WTN], a1[WTM], b1[WTN];
  if (nk > 0) {
    issue(0);
    wait_vm<0>();
    __syncthreads();
    if (1 < nk) issue(1);
    load_frags(0, 0, a0, b0);
  }
  for (int kt = 0; kt < nk - 1; ++kt) {
    const int b = kt & 1;
    load_frags(b, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    load_frags(b, 2, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
    load_frags(b, 3, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<0>();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 2 < nk) issue(kt + 2);
    load_frags(b ^ 1, 0, a0, b0);
    mma(a1, b1);
  }
  if (nk > 0) {
    const int b = (nk - 1) & 1;
    load_frags(b, 1, a1, b1);
    mma(a0, b0);
    load_frags(b, 2, a0, b0);
    mma(a1, b1);
    load_frags(b, 3, a1, b1);
    mma(a0, b0);
    mma(a1, b1);
  }

  if constexpr (OUT == 0) {
    // bf16 output through LDS: the block's 256 x 256 tile is rounded once
    // (nearest even) into the 128 KB the stages used, as rows of 512 bytes
    // whose 16-byte chunk c sits at c ^ (4 ((row >> 2) & 1)) (the two halves
    // of a wave write rows 4 apart: this puts them on disjoint banks), then
    // every thread stores 16 contiguous bytes per row it covers.
    __syncthreads();  // every wave has read its last stage
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * 128 + i * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          const int col = wn * 64 + j * 32 + r;
          const int chunk = (col >> 3) ^ (((row >> 2) & 1) << 2);
          smem[row * 256 + chunk * 8 + (col & 7)] = __builtin_bit_cast(uint16_t, __bf16(acc[i][j][e]));
        }
    __syncthreads();
    const int c = tid & 31;  // 16-byte chunk of a row: columns 8c .. 8c + 7
    const int64_t n = n0 + 8 * c;
    const bool vec = (N & 7) == 0 && (reinterpret_cast<uintptr_t>(Cv) & 15) == 0;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = it * 16 + (tid >> 5);
      const int64_t m = m0 + row;
      if (m >= M || n >= N) continue;
      const uint4 w = *reinterpret_cast<const uint4*>(&smem[row * 256 + ((c ^ (((row >> 2) & 1) << 2)) * 8)]);
      uint16_t* dst = static_cast<uint16_t*>(Cv) + m * N + n;
      if (vec) {
        *reinterpret_cast<uint4*>(dst) = w;
      } else {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (n + u < N) dst[u] = uint16_t(ws[u >> 1] >> (16 * (u & 1)));
      }
    }
    return;
  }
  // fp32 output straight from the accumulators (staging it through LDS in
  // two halves measured no faster): lane holds C[m = 8*(e/4) + 4hh + e%4][n = r]
  // of each 32 x 32 tile
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (m >= M) continue;
        static_cast<float*>(Cv)[m * N + n] = acc[i][j][e];
      }
    }
}

template <bool A_T, bool B_T, int OUT>
int launch_gemm(const uint16_t* A, const uint16_t* B, void* C, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 0 || N <= 0) return 0;
  const int64_t tm = (M + GBM - 1) / GBM, tn = (N + GBN - 1) / GBN;
  if (tm * tn >= (int64_t(1) << 31)) return -1;
  // per-lane offsets are 32-bit: 256 rows (or 32 k rows) of the widest operand
  const int64_t lda = A_T ? M : K, ldb = B_T ? K : N;
  if (int64_t(GBM) * (lda > ldb ? lda : ldb) * 2 >= int64_t(kRecords)) return -1;
  gemm_kernel<A_T, B_T, OUT><<<dim3(unsigned(tm * tn)), dim3(GTHREADS), 0, st>>>(A, B, C, M, N, K);
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
