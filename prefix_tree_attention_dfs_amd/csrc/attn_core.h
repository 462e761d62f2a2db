// Pieces shared by the translation units that launch attention: the device
// plan view, launch-failure reporting, optional per-launch timing, and the
// attention cores that run on already-rotated Q and K.
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "internal.h"
#include "kernels.h"

namespace ttc {

inline PlanPtrs plan_ptrs(const tt_tree* t, const void* dev_plan) {
  const int32_t* base = static_cast<const int32_t*>(dev_plan);
  const int32_t* h = t->plan.data();
  PlanPtrs P;
  P.depth = base + h[ttp::H_DEPTH];
  P.end = base + h[ttp::H_END];
  P.qb_ptr = base + h[ttp::H_QB_PTR];
  P.qb_tiles = base + h[ttp::H_QB_TILES];
  P.qb_order = base + h[ttp::H_QB_ORDER];
  P.kb_qlo = base + h[ttp::H_KB_QLO];
  P.kb_qhi = base + h[ttp::H_KB_QHI];
  P.kb_minend = base + h[ttp::H_KB_MINEND];
  P.kb_order = base + h[ttp::H_KB_ORDER];
  P.N = t->N;
  P.bq = t->bq;
  P.bk = t->bk;
  P.nqb = t->nqb;
  P.nkb = t->nkb;
  P.hdr = base;
  P.id = h[ttp::H_ID];
  return P;
}


inline int dev_fail(const char* fn, const char* what) {
  const hipError_t e = hipGetLastError();
  return tt::fail(TT_EDEVICE, std::string(fn) + ": " + what + " failed: " + hipGetErrorString(e));
}

// ---- optional per-launch timing (tt_timing_enable)
struct TimedLaunch {
  const char* name;
  hipEvent_t a, b;
};
inline thread_local bool g_timing = false;
inline thread_local std::vector<TimedLaunch> g_launches;
inline thread_local std::vector<hipEvent_t> g_pool;

inline hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with events on its stream when timing is on.
class KTimer {
 public:
  KTimer(const char* name, hipStream_t st) : name_(name), st_(st) {
    if (!g_timing) return;
    a_ = take_event();
    b_ = take_event();
    if (a_ && b_) (void)hipEventRecord(a_, st_);
  }
  ~KTimer() {
    if (!g_timing || !a_ || !b_) return;
    (void)hipEventRecord(b_, st_);
    g_launches.push_back({name_, a_, b_});
  }

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};


// Device plans the host has filled: tree_plan_upload (and the path-mode
// upload) records each buffer's address with its image's identity word, and
// every attention call checks that its plan is one of them and belongs to a
// tree of the call's shape (TT_EINVAL otherwise).  The kernels' own header
// check stays as the backstop for device memory the host cannot see.
void plan_register(const void* dev_plan, int32_t id);
int plan_check(const tt_tree* t, const void* dev_plan, const char* fn);

// Validation of tree_weighted_nll's arguments shared by its entry points
// (everything but the workspace); messages start with fn.
int nll_check(const tt_nll_args* a, const char* fn);

// Shapes the bf16 matrix-core kernels take (any GQA group, any size).
bool mfma_shape(int32_t d, int32_t bq, int32_t bk);

// Factor the query operand carries into the attention cores: the
// matrix-core kernels take q (rotated) times scale * log2(e), so that q.k is
// the score in log2 units and exp2 applies to it directly; the vector
// kernels take the rotated q itself (1).
double q_operand_scale(tt_dtype dt, const AttnGeom& g, const PlanPtrs& P);

// Forward on rotated q (times q_operand_scale) and k (no RoPE here).
int attn_fwd_core(tt_dtype dt, const PlanPtrs& P, const AttnGeom& g, const void* q, const void* k, const void* v,
                  void* o, float* lse, bool full_range, hipStream_t st);

// Backward on rotated q (times q_operand_scale) and k: D = rowsum(dO o O) into D, dQ (rotated frame,
// float32, not yet rotated back) into dq, dK and dV into d_k, d_v (float32
// and added to when acc).  When dq_final is set and the bf16 matrix-core
// kernels run, dQ is instead rotated back with cs_tab and stored in bf16 to
// dq_final, and *dq_done is set (dq is then not written).
int attn_bwd_core(tt_dtype dt, const PlanPtrs& P, const AttnGeom& g, const void* q, const void* k, const void* v,
                  const void* o, const void* d_o, const float* lse, float* D, float* dq, void* d_k, void* d_v,
                  bool acc, bool full_range, const float2* cs_tab, hipStream_t st, void* dq_final = nullptr,
                  bool* dq_done = nullptr);

}  // namespace ttc
