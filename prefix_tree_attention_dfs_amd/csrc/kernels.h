// Host-callable launchers of the library's kernels.  Each returns 0 on success
// or -1 if the launch failed.  All take the caller's stream; none allocates.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "tt.h"

// RoPE (and its transpose) at the rows' depths; acc adds into an fp32 output.
// tab: the (cos, sin) table of launch_rope_table for these depths, or null;
// only the bf16 -> bf16 kernel uses it (fp32 rotation from the table instead
// of fp64 angles per thread).
int launch_rope(const void* x, void* y, tt_dtype tin, tt_dtype tout, bool acc, const PlanPtrs& P, int32_t row0,
                int32_t n_rows, int32_t heads, int32_t d, float base, bool inverse, hipStream_t st,
                double mul = 1.0, const float2* tab = nullptr);

// Generic (any d <= 256) path, fp32 or bf16 storage.
int launch_fwd_generic(tt_dtype dt, const void* q, const void* k, const void* v, void* o, float* lse,
                       const PlanPtrs& P, const AttnGeom& g, hipStream_t st);
int launch_bwd_pre(tt_dtype dt, const void* o, const void* d_o, float* D, int64_t rows, int d, hipStream_t st);
int launch_dq_generic(tt_dtype dt, const void* q, const void* k, const void* v, const void* d_o, const float* lse,
                      const float* D, float* dq_acc, const PlanPtrs& P, const AttnGeom& g, hipStream_t st);
int launch_dkdv_generic(tt_dtype dt, bool acc, const void* q, const void* k, const void* v, const void* d_o,
                        const float* lse, const float* D, void* d_k, void* d_v, const PlanPtrs& P,
                        const AttnGeom& g, hipStream_t st);

// bf16 MFMA path, head dim 128 (returns -2 if the geometry is not covered).
bool mfma_attn_supported(const AttnGeom& g, const PlanPtrs& P);
bool mfma_bwd_supported(const AttnGeom& g, const PlanPtrs& P);
// The forward's own query operand: q is then the caller's Q; the kernel
// rotates it at depth with tab (null: no rotation), multiplies by mul, rounds
// to bf16, uses that and stores it to out ([n_q, h_q, 128] bf16).
struct QRot {
  void* out;
  const float2* tab;
  float mul;
};
int launch_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, const PlanPtrs& P,
                    const AttnGeom& g, bool full_range, hipStream_t st, const QRot* qr = nullptr);
// dQ into dq_acc (fp32, rotated frame), or, when dq_out is set, rotated back
// with cs_tab (may be null: no rotation) and stored in bf16 to dq_out.
int launch_dq_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D,
                   float* dq_acc, void* dq_out, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                   bool full_range, hipStream_t st);
int launch_dkdv_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D,
                     void* d_k, void* d_v, bool acc, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                     hipStream_t st);
// Group sizes the one-launch backward takes: a multiple of 4 query heads per
// kv head (a dQ workgroup = one kv head's 4 heads), or 2 with an even number of
// kv heads (a dQ workgroup = two kv heads' pairs); either way 8 waves, the
// dK/dV workgroups' size.
inline bool bwd_combined_supported(int32_t h_q, int32_t h_kv) {
  if (h_kv <= 0 || h_q % h_kv != 0) return false;
  const int32_t G = h_q / h_kv;
  return G % 4 == 0 || (G == 2 && h_kv % 2 == 0);
}
// dQ (as launch_dq_mfma) and dK/dV (as launch_dkdv_mfma) in one launch;
// returns -2 (nothing launched) when the group size or output form is not
// covered (then the two launches above apply)
int launch_bwd_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D,
                    float* dq_acc, void* dq_out, void* d_k, void* d_v, bool acc, const float2* cs_tab,
                    const PlanPtrs& P, const AttnGeom& g, bool full_range, hipStream_t st);
// Several independent backward calls in one launch (as launch_bwd_mfma for
// each): every call has its own query rows (q, d_o, lse and D at the call's
// first row, g.q_off / n_q / n_k its geometry), dQ output and dK/dV outputs,
// and all share k, v, cs_tab and the plan, the head counts and the output
// form (acc, and dq_out set or not).  Calls may run in any order and side by
// side, so no two may write the same output.  Returns -2 as launch_bwd_mfma.
constexpr int kMaxBwdCalls = 4;
struct BwdCallPtrs {
  const void* q;
  const void* d_o;
  const float* lse;
  const float* D;
  float* dq_acc;
  void* dq_out;
  void* d_k;
  void* d_v;
  AttnGeom g;
};
int launch_bwd_mfma_multi(const BwdCallPtrs* calls, int n_calls, const void* k, const void* v, bool acc,
                          const float2* cs_tab, const PlanPtrs& P, bool full_range, hipStream_t st);
// (cos, sin) of p * theta_k, theta_k = base^(-2k / (2 half)), for p < n_pos and
// k < half, computed in fp64 and rounded to fp32: tab[p * half + k]
int launch_rope_table(float2* tab, int32_t n_pos, int32_t half, float base, hipStream_t st);

// bf16 out_k / out_v (n elements each, a multiple of 4) = the sum of nslot
// fp32 accumulators (slot u at acc + u * slot_stride elements); the
// accumulators' n elements are zeroed.
// Path walk data movement (bf16, d % 16 == 0; 16-byte aligned rows).
// push: tree rows [row0, row0 + n_rows) of q, k, v to stack positions
// [pos0, ...): Q rotated at the position with tab (null: not rotated) and
// multiplied by qmul, K rotated, V copied; srow[pos] = tree row.
int launch_path_push(const void* q, const void* k, const void* v, void* Qp, void* Kp, void* Vp, int32_t* srow,
                     const float2* tab, int32_t row0, int32_t pos0, int32_t n_rows, int32_t hq, int32_t hk,
                     int32_t d, float qmul, hipStream_t st);
// scatter: for positions p in [p0, p1), row srow[p] of a_out = row
// a_src0 + (p - p0) of a (a_row_bytes, a multiple of 16), and b_n floats of
// b_out = row p of b (b_n = 0: none).
int launch_path_scatter(const void* a, void* a_out, int64_t a_row_bytes, int64_t a_src0, const float* b,
                        float* b_out, int32_t b_n, const int32_t* srow, int32_t p0, int32_t p1, hipStream_t st);
// The backward chunks of one launch: chunk u's dO block dob and D (rows
// qo .. c1 - 1 of the stack; positions below c0 are the alignment pad) and
// its bf16 dQ block dq_blk (same rows).
struct PathChunk {
  void* dob;
  float* D;
  const void* dq_blk;
  int32_t qo, c0, c1;
};
struct PathChunks {
  PathChunk c[kMaxBwdCalls];
  int32_t n;
};
// dO blocks (rows of d_o via srow, zeros on the pad) and D = rowsum(dob o
// O_stack) as launch_bwd_pre computes it, for every chunk of C (d = 128).
int launch_path_dout_pre(const void* Op, const void* d_o, const int32_t* srow, const PathChunks& C, int32_t hq,
                         int32_t d, hipStream_t st);
// dQ rows [c0, c1) of every chunk of C from its block to tree rows srow[p].
int launch_path_dq_scatter(void* d_q, int64_t row_bytes, const int32_t* srow, const PathChunks& C, hipStream_t st);
int launch_acc_pop(float* acc_k, float* acc_v, int64_t slot_stride, int nslot, void* out_k, void* out_v, int64_t n,
                   hipStream_t st);

// Zeroes `bytes` (a multiple of 4) at p.
int launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// Weighted NLL.
int launch_nll_rows(tt_dtype zt, const void* z, void* dz, int32_t n_rows, int32_t vocab, int64_t ldz,
                    const int32_t* row_ptr, const int32_t* tgt_id, const float* tgt_w, int32_t n_tgt, float* logp,
                    float* row_loss, hipStream_t st);
int launch_sum_loss(const float* row_loss, int32_t n, float* loss, hipStream_t st);

// bf16 GEMMs of the fused lm-head (row-major operands).
//   Z  [M,N] = H [M,K] * W [K,N]
//   dH [M,K] = dZ [M,N] * W^T
//   dW [K,N] = H^T * dZ   (fp32 or bf16 out)
int launch_gemm_nn(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N, int64_t K,
                   hipStream_t st);
int launch_gemm_nt(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N, int64_t K,
                   hipStream_t st);
int launch_gemm_tn(const uint16_t* A, const uint16_t* B, void* C, bool c_f32, int64_t M, int64_t N, int64_t K,
                   hipStream_t st);
