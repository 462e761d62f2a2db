// Dense bf16 matrix-core throughput probe (gfx950).
//
// Every wave of every workgroup runs `iters` rounds of 32
// v_mfma_f32_32x32x16_bf16 on register operands, alternating between two
// independent accumulators, so the matrix pipe of each SIMD never waits on
// memory or on a dependency.  Timed by the caller on its stream, the
// FLOP count divided by the elapsed time is the rate the chip sustains under
// a pure MFMA load (its clock included), to set beside the published peak.
// One float per thread goes to `out` so that no product is dead code.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "tt.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;

__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = __bf16(1.f + 1e-3f * float(lane + s));
    b[s] = __bf16(1.f - 1e-3f * float(s));
  }
  f32x16 c0, c1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c0[i] = 0.f;
    c1[i] = 0.f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
  out[int64_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int tt_probe_mfma(int32_t n_blocks, int32_t iters, float* out, tt_stream stream, double* flops) {
  tt::clear_error();
  if (!out || !flops) return tt::fail(TT_EINVAL, "tt_probe_mfma: NULL argument");
  if (n_blocks < 1 || n_blocks > 65536 || iters < 1 || iters > (1 << 20))
    return tt::fail(TT_EINVAL, "tt_probe_mfma: n_blocks must be in [1, 65536] and iters in [1, 2^20]");
  mfma_probe_kernel<<<dim3(unsigned(n_blocks)), dim3(kThreads), 0, static_cast<hipStream_t>(stream)>>>(out, iters);
  if (hipGetLastError() != hipSuccess) return tt::fail(TT_EDEVICE, "tt_probe_mfma: launch failed");
  *flops = double(n_blocks) * (kThreads / 64) * double(iters) * 32.0 * (2.0 * 32 * 32 * 16);
  return TT_OK;
}
