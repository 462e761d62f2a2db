// C ABI entry points that touch the device: plan upload, tree attention
// forward/backward, weighted NLL.  Validation happens here, before any launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "attn_core.h"
#include "internal.h"
#include "kernels.h"

using ttc::dev_fail;
using ttc::KTimer;
using ttc::plan_ptrs;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t dsize(tt_dtype t) { return t == TT_F32 ? 4 : 2; }

// Workspace carve-up, identical for the size query and the calls.
struct AttnWs {
  size_t q_rot = 0, k_rot = 0, D = 0, dq = 0, cs = 0, total = 0;
  bool rope = false;
  bool qcopy = false;  // q rotated (and, for the matrix-core kernels, scaled) into the workspace
  int32_t cs_pos = 0;  // rows of the (cos, sin) table: every depth of the tree
};

// bf16 RoPE rotates from the (cos, sin) table (fp32 per element instead of
// fp64 angles per thread); forward and backward use the same table, so the
// rotated copies the backward recomputes equal the forward's.
const float2* rope_tab(const tt_attn_args* a, const AttnWs& w, char* ws) {
  return w.rope && w.cs_pos > 0 && a->dtype == TT_BF16 ? reinterpret_cast<const float2*>(ws + w.cs) : nullptr;
}

// The matrix-core kernels take the query already multiplied by scale * log2(e)
// (their scores come out in log2 units); that copy lives in the workspace even
// without RoPE.
bool mfma_call(const tt_attn_args* a) {
  return a->dtype == TT_BF16 && ttc::mfma_shape(a->d, a->tree->bq, a->tree->bk);
}

AttnWs attn_ws(const tt_attn_args* a, bool bwd) {
  AttnWs w;
  const size_t es = dsize(a->dtype);
  w.rope = a->rope_base != 0.f;
  w.qcopy = w.rope || mfma_call(a);
  size_t off = 0;
  if (w.qcopy) {
    w.q_rot = off;
    off = align_up(off + size_t(a->n_q) * a->h_q * a->d * es);
  }
  if (w.rope) {
    w.k_rot = off;
    off = align_up(off + size_t(a->n_k) * a->h_kv * a->d * es);
    w.cs_pos = a->tree->max_depth + 1;
    w.cs = off;
    off = align_up(off + size_t(w.cs_pos) * (a->d / 2) * 8);
  }
  if (bwd) {
    w.D = off;
    off = align_up(off + size_t(a->n_q) * a->h_q * 4);
    w.dq = off;
    off = align_up(off + size_t(a->n_q) * a->h_q * a->d * 4);
  }
  w.total = off;
  return w;
}

int check_attn(const tt_attn_args* a, const char* fn) {
  using std::string;
  if (!a) return tt::fail(TT_EINVAL, string(fn) + ": args is NULL");
  if (!a->tree) return tt::fail(TT_EINVAL, string(fn) + ": tree is NULL");
  if (!a->plan) return tt::fail(TT_EINVAL, string(fn) + ": plan is NULL");
  if (a->dtype != TT_F32 && a->dtype != TT_BF16) return tt::fail(TT_EINVAL, string(fn) + ": bad dtype");
  if (a->h_q <= 0 || a->h_kv <= 0 || a->h_q % a->h_kv != 0)
    return tt::fail(TT_EINVAL, string(fn) + ": need h_q, h_kv > 0 and h_q % h_kv == 0");
  if (a->d <= 0 || a->d % 2 != 0) return tt::fail(TT_EINVAL, string(fn) + ": d must be positive and even");
  if (a->d % 16 != 0 || a->d > 256)
    return tt::fail(TT_EUNSUPPORTED, string(fn) + ": head dim must be a multiple of 16 and <= 256");
  if (a->flags & ~uint32_t(TT_ALLOW_GENERIC)) return tt::fail(TT_EINVAL, string(fn) + ": unknown flags");
  const tt_tree* t = a->tree;
  if (a->dtype == TT_BF16 && !(a->flags & TT_ALLOW_GENERIC) && !ttc::mfma_shape(a->d, t->bq, t->bk))
    return tt::fail(TT_EUNSUPPORTED, string(fn) +
                                         ": bf16 attention runs on the matrix cores for head dim 128 and 64-row "
                                         "schedule blocks only; TT_ALLOW_GENERIC selects the vector kernels");
  if (a->q_off < 0 || a->n_q < 0 || a->n_k < 0) return tt::fail(TT_EINVAL, string(fn) + ": negative q_off/n_q/n_k");
  if (int64_t(a->q_off) + a->n_q > a->n_k || a->n_k > t->N)
    return tt::fail(TT_EINVAL, string(fn) + ": need q_off + n_q <= n_k <= N");
  if (a->q_off % t->bq != 0) return tt::fail(TT_EINVAL, string(fn) + ": q_off must be a multiple of block_q");
  if (!(a->scale >= 0.f) || !std::isfinite(a->scale)) return tt::fail(TT_EINVAL, string(fn) + ": bad scale");
  if (!(a->rope_base >= 0.f) || !std::isfinite(a->rope_base))
    return tt::fail(TT_EINVAL, string(fn) + ": bad rope_base");
  const int64_t qe = int64_t(a->n_q) * a->h_q * a->d, ke = int64_t(a->n_k) * a->h_kv * a->d;
  if (qe * 4 > (int64_t(1) << 40) || ke * 4 > (int64_t(1) << 40))
    return tt::fail(TT_EOVERFLOW, string(fn) + ": tensors too large");
  if (a->n_q > 0 && (!a->q || !a->o || !a->lse))
    return tt::fail(TT_EINVAL, string(fn) + ": q, o and lse are required");
  if (a->n_k > 0 && (!a->k || !a->v)) return tt::fail(TT_EINVAL, string(fn) + ": k and v are required");
  for (const void* p : {a->q, a->k, a->v, static_cast<const void*>(a->o), static_cast<const void*>(a->lse),
                        static_cast<const void*>(a->workspace), a->plan})
    if (p && !aligned16(p)) return tt::fail(TT_EINVAL, string(fn) + ": device pointers must be 16-byte aligned");
  return TT_OK;
}

int check_ws(const tt_attn_args* a, bool bwd, const char* fn) {
  const AttnWs w = attn_ws(a, bwd);
  if (w.total > 0 && (!a->workspace || a->workspace_bytes < w.total))
    return tt::fail(TT_EWORKSPACE, std::string(fn) + ": workspace too small (need " + std::to_string(w.total) +
                                       " bytes)");
  return TT_OK;
}

AttnGeom geom(const tt_attn_args* a) {
  AttnGeom g;
  g.q_off = a->q_off;
  g.n_q = a->n_q;
  g.n_k = a->n_k;
  g.h_q = a->h_q;
  g.h_kv = a->h_kv;
  g.d = a->d;
  g.scale = a->scale == 0.f ? float(1.0 / std::sqrt(double(a->d))) : a->scale;
  g.rope_base = a->rope_base;
  return g;
}


}  // namespace

namespace ttc {

namespace {
std::mutex g_plan_mu;
std::unordered_map<uintptr_t, int32_t> g_plan_owner;  // device plan address -> identity word of its image
}  // namespace

void plan_register(const void* dev_plan, int32_t id) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  g_plan_owner[reinterpret_cast<uintptr_t>(dev_plan)] = id;
}

int plan_check(const tt_tree* t, const void* dev_plan, const char* fn) {
  int32_t id = 0;
  bool known = false;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    const auto it = g_plan_owner.find(reinterpret_cast<uintptr_t>(dev_plan));
    if (it != g_plan_owner.end()) {
      known = true;
      id = it->second;
    }
  }
  if (!known)
    return tt::fail(TT_EINVAL, std::string(fn) + ": plan was not filled by tree_plan_upload (or tree_path_plan_upload)");
  if (id != t->plan[ttp::H_ID])
    return tt::fail(TT_EINVAL, std::string(fn) + ": plan was last uploaded from a tree of another shape");
  return TT_OK;
}

bool mfma_shape(int32_t d, int32_t bq, int32_t bk) { return d == 128 && bq == 64 && bk == 64; }

double q_operand_scale(tt_dtype dt, const AttnGeom& g, const PlanPtrs& P) {
  return dt == TT_BF16 && mfma_attn_supported(g, P) ? double(g.scale) * 1.4426950408889634 : 1.0;
}

int attn_fwd_core(tt_dtype dt, const PlanPtrs& P, const AttnGeom& g, const void* q, const void* k, const void* v,
                  void* o, float* lse, bool full_range, hipStream_t st) {
  const char* fn = "attention forward";
  if (dt == TT_BF16 && mfma_attn_supported(g, P)) {
    KTimer t("attn_fwd_mfma", st);
    if (launch_fwd_mfma(q, k, v, o, lse, P, g, full_range, st)) return dev_fail(fn, "attention kernel");
  } else {
    KTimer t("attn_fwd_generic", st);
    if (launch_fwd_generic(dt, q, k, v, o, lse, P, g, st)) return dev_fail(fn, "attention kernel");
  }
  return TT_OK;
}

int attn_bwd_core(tt_dtype dt, const PlanPtrs& P, const AttnGeom& g, const void* q, const void* k, const void* v,
                  const void* o, const void* d_o, const float* lse, float* D, float* dq, void* d_k, void* d_v,
                  bool acc, bool full_range, const float2* cs_tab, hipStream_t st, void* dq_final, bool* dq_done) {
  const char* fn = "attention backward";
  if (dq_done) *dq_done = false;
  {
    KTimer t("attn_bwd_pre", st);
    if (launch_bwd_pre(dt, o, d_o, D, int64_t(g.n_q) * g.h_q, g.d, st)) return dev_fail(fn, "preprocess");
  }
  if (dt == TT_BF16 && mfma_bwd_supported(g, P)) {
    // one launch for dQ and dK/dV when the dQ workgroups have the dK/dV
    // workgroups' size (four query heads each: groups of a multiple of 4, or
    // two kv heads' pairs)
    if (bwd_combined_supported(g.h_q, g.h_kv) && (acc || dq_final)) {
      int rc = -2;
      {
        KTimer t("attn_bwd_mfma", st);
        rc = launch_bwd_mfma(q, k, v, d_o, lse, D, dq, dq_final, d_k, d_v, acc, cs_tab, P, g, full_range, st);
      }
      if (rc == -1) return dev_fail(fn, "backward kernel");
      if (rc == 0) {
        if (dq_final && dq_done) *dq_done = true;
        return TT_OK;
      }
    }
    {
      KTimer t("attn_bwd_dq_mfma", st);
      if (launch_dq_mfma(q, k, v, d_o, lse, D, dq, dq_final, cs_tab, P, g, full_range, st))
        return dev_fail(fn, "dq kernel");
      if (dq_final && dq_done) *dq_done = true;
    }
    {
      KTimer t("attn_bwd_dkdv_mfma", st);
      if (launch_dkdv_mfma(q, k, v, d_o, lse, D, d_k, d_v, acc, cs_tab, P, g, st)) return dev_fail(fn, "dk/dv kernel");
    }
  } else {
    {
      KTimer t("attn_bwd_dq_generic", st);
      if (launch_dq_generic(dt, q, k, v, d_o, lse, D, dq, P, g, st)) return dev_fail(fn, "dq kernel");
    }
    {
      KTimer t("attn_bwd_dkdv_generic", st);
      if (launch_dkdv_generic(dt, acc, q, k, v, d_o, lse, D, d_k, d_v, P, g, st)) return dev_fail(fn, "dk/dv kernel");
    }
  }
  return TT_OK;
}

}  // namespace ttc

extern "C" int tt_timing_enable(int on) {
  tt::clear_error();
  ttc::g_timing = on != 0;
  return TT_OK;
}

extern "C" int tt_timing_collect(tt_kernel_time* out, int capacity, int* count) {
  tt::clear_error();
  if (!count || (capacity > 0 && !out)) return tt::fail(TT_EINVAL, "tt_timing_collect: NULL argument");
  std::vector<tt_kernel_time> agg;
  int rc = TT_OK;
  for (const ttc::TimedLaunch& t : ttc::g_launches) {
    float ms = 0.f;
    if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&ms, t.a, t.b) != hipSuccess) {
      rc = TT_EDEVICE;
      ms = 0.f;
    }
    size_t k = 0;
    while (k < agg.size() && std::strncmp(agg[k].name, t.name, sizeof(agg[k].name)) != 0) ++k;
    if (k == agg.size()) {
      tt_kernel_time z{};
      std::strncpy(z.name, t.name, sizeof(z.name) - 1);
      agg.push_back(z);
    }
    agg[k].launches += 1;
    agg[k].total_ms += ms;
    agg[k].max_ms = std::max(agg[k].max_ms, double(ms));
    ttc::g_pool.push_back(t.a);
    ttc::g_pool.push_back(t.b);
  }
  ttc::g_launches.clear();
  *count = int(agg.size());
  for (int i = 0; i < capacity && i < int(agg.size()); ++i) out[i] = agg[size_t(i)];
  if (rc != TT_OK) return tt::fail(rc, "tt_timing_collect: event query failed");
  return TT_OK;
}

extern "C" int tree_plan_upload(const tt_tree* t, void* dev_plan, size_t bytes, tt_stream stream) {
  tt::clear_error();
  if (!t || !dev_plan) return tt::fail(TT_EINVAL, "tree_plan_upload: NULL argument");
  if (!aligned16(dev_plan)) return tt::fail(TT_EINVAL, "tree_plan_upload: plan must be 16-byte aligned");
  const size_t need = t->plan.size() * sizeof(int32_t);
  if (bytes < need) return tt::fail(TT_EWORKSPACE, "tree_plan_upload: buffer smaller than tree_plan_bytes");
  if (hipMemcpyAsync(dev_plan, t->plan.data(), need, hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess)
    return dev_fail("tree_plan_upload", "hipMemcpyAsync");
  ttc::plan_register(dev_plan, t->plan[ttp::H_ID]);
  return TT_OK;
}

extern "C" int tree_attn_workspace_bytes(const tt_attn_args* a, int for_bwd, size_t* bytes) {
  tt::clear_error();
  if (!bytes) return tt::fail(TT_EINVAL, "tree_attn_workspace_bytes: bytes is NULL");
  if (!a || !a->tree) return tt::fail(TT_EINVAL, "tree_attn_workspace_bytes: args/tree is NULL");
  if (a->n_q < 0 || a->n_k < 0 || a->h_q <= 0 || a->h_kv <= 0 || a->d <= 0)
    return tt::fail(TT_EINVAL, "tree_attn_workspace_bytes: bad geometry");
  *bytes = attn_ws(a, for_bwd != 0).total;
  return TT_OK;
}

extern "C" int tree_attn_fwd(const tt_attn_args* a, tt_stream stream) {
  tt::clear_error();
  const char* fn = "tree_attn_fwd";
  int rc = check_attn(a, fn);
  if (rc) return rc;
  if ((rc = check_ws(a, false, fn))) return rc;
  if ((rc = ttc::plan_check(a->tree, a->plan, fn))) return rc;
  if (a->n_q == 0) return TT_OK;
  hipStream_t st = (hipStream_t)stream;
  const PlanPtrs P = plan_ptrs(a->tree, a->plan);
  const AttnGeom g = geom(a);
  const AttnWs w = attn_ws(a, false);
  char* ws = static_cast<char*>(a->workspace);
  const void* q = a->q;
  const void* k = a->k;
  if (rope_tab(a, w, ws)) {  // only the bf16 kernels read the table
    KTimer t("rope_table", st);
    if (launch_rope_table(reinterpret_cast<float2*>(ws + w.cs), w.cs_pos, a->d / 2, a->rope_base, st))
      return dev_fail(fn, "rope table");
  }
  const float2* tab = rope_tab(a, w, ws);
  // the matrix-core kernel makes the query operand from the caller's Q itself
  // and leaves it at q_rot for the backward (same arithmetic as rope_q)
  const bool own_q = a->dtype == TT_BF16 && mfma_attn_supported(g, P);
  if (w.qcopy && !own_q) {
    KTimer t("rope_q", st);
    if (launch_rope(a->q, ws + w.q_rot, a->dtype, a->dtype, false, P, a->q_off, a->n_q, a->h_q, a->d,
                    a->rope_base, false, st, ttc::q_operand_scale(a->dtype, g, P), tab))
      return dev_fail(fn, "rope(q)");
    q = ws + w.q_rot;
  }
  if (w.rope) {
    KTimer t("rope_k", st);
    if (launch_rope(a->k, ws + w.k_rot, a->dtype, a->dtype, false, P, 0, a->n_k, a->h_kv, a->d,
                    a->rope_base, false, st, 1.0, tab))
      return dev_fail(fn, "rope(k)");
    k = ws + w.k_rot;
  }
  const bool full_range = a->q_off == 0 && a->n_q == P.N;
  if (own_q) {
    const QRot qr{ws + w.q_rot, tab, float(ttc::q_operand_scale(a->dtype, g, P))};
    KTimer t("attn_fwd_mfma", st);
    if (launch_fwd_mfma(a->q, k, a->v, a->o, a->lse, P, g, full_range, st, &qr))
      return dev_fail(fn, "attention kernel");
    return TT_OK;
  }
  return ttc::attn_fwd_core(a->dtype, P, g, q, k, a->v, a->o, a->lse, full_range, st);
}

extern "C" int tree_attn_bwd(const tt_attn_bwd_args* b, tt_stream stream) {
  tt::clear_error();
  const char* fn = "tree_attn_bwd";
  if (!b) return tt::fail(TT_EINVAL, "tree_attn_bwd: args is NULL");
  const tt_attn_args* a = &b->a;
  int rc = check_attn(a, fn);
  if (rc) return rc;
  if (b->flags & ~(TT_ACCUMULATE_DKDV | TT_BWD_REUSE_ROTATED))
    return tt::fail(TT_EINVAL, "tree_attn_bwd: unknown flags");
  const bool acc = (b->flags & TT_ACCUMULATE_DKDV) != 0;
  const bool reuse = (b->flags & TT_BWD_REUSE_ROTATED) != 0;
  if (a->n_q > 0 && (!b->d_o || !b->d_q)) return tt::fail(TT_EINVAL, "tree_attn_bwd: d_o and d_q are required");
  if (a->n_k > 0 && (!b->d_k || !b->d_v)) return tt::fail(TT_EINVAL, "tree_attn_bwd: d_k and d_v are required");
  for (const void* p : {b->d_o, static_cast<const void*>(b->d_q), static_cast<const void*>(b->d_k),
                        static_cast<const void*>(b->d_v)})
    if (p && !aligned16(p)) return tt::fail(TT_EINVAL, "tree_attn_bwd: device pointers must be 16-byte aligned");
  if ((rc = check_ws(a, true, fn))) return rc;
  if ((rc = ttc::plan_check(a->tree, a->plan, fn))) return rc;
  if (a->n_k == 0) return TT_OK;
  hipStream_t st = (hipStream_t)stream;
  const PlanPtrs P = plan_ptrs(a->tree, a->plan);
  const AttnGeom g = geom(a);
  const AttnWs w = attn_ws(a, true);
  char* ws = static_cast<char*>(a->workspace);
  const void* q = a->q;
  const void* k = a->k;
  // the forward wrote the rotated copies and the (cos, sin) table at the same
  // offsets (tree_attn_workspace_bytes layout)
  float2* cs_tab = nullptr;
  if (rope_tab(a, w, ws)) {
    cs_tab = reinterpret_cast<float2*>(ws + w.cs);
    if (!reuse) {
      KTimer t("rope_table", st);
      if (launch_rope_table(cs_tab, w.cs_pos, a->d / 2, a->rope_base, st)) return dev_fail(fn, "rope table");
    }
  }
  const float2* tab = rope_tab(a, w, ws);
  if (w.qcopy) {
    if (a->n_q > 0 && !reuse) {
      KTimer t("rope_q", st);
      if (launch_rope(a->q, ws + w.q_rot, a->dtype, a->dtype, false, P, a->q_off, a->n_q, a->h_q, a->d,
                      a->rope_base, false, st, ttc::q_operand_scale(a->dtype, g, P), tab))
        return dev_fail(fn, "rope(q)");
    }
    q = ws + w.q_rot;
  }
  if (w.rope) {
    if (!reuse) {
      KTimer t("rope_k", st);
      if (launch_rope(a->k, ws + w.k_rot, a->dtype, a->dtype, false, P, 0, a->n_k, a->h_kv, a->d,
                      a->rope_base, false, st, 1.0, tab))
        return dev_fail(fn, "rope(k)");
    }
    k = ws + w.k_rot;
  }
  float* D = reinterpret_cast<float*>(ws + w.D);
  float* dq = reinterpret_cast<float*>(ws + w.dq);
  const bool full_range = a->q_off == 0 && a->n_q == P.N;
  // the bf16 dQ kernel rotates back and converts in its epilogue (table
  // built above whenever RoPE is on); other paths finalize from fp32 below
  bool dq_done = false;
  void* dq_final = (a->dtype == TT_BF16 && (!w.rope || cs_tab)) ? b->d_q : nullptr;
  if ((rc = ttc::attn_bwd_core(a->dtype, P, g, q, k, a->v, a->o, b->d_o, a->lse, D, dq, b->d_k, b->d_v, acc,
                               full_range, cs_tab, st, dq_final, &dq_done)))
    return rc;
  // dQ: rotate back at the query rows' depths, convert to the output dtype
  if (a->n_q > 0 && !dq_done) {
    KTimer t("dq_finalize", st);
    if (launch_rope(dq, b->d_q, TT_F32, a->dtype, false, P, a->q_off, a->n_q, a->h_q, a->d, a->rope_base, true,
                    st))
      return dev_fail(fn, "dq finalize");
  }
  return TT_OK;
}

// ---------------------------------------------------------------- weighted NLL
namespace {

struct NllWs {
  size_t z = 0, row_loss = 0, total = 0;
  bool fused = false;
};

NllWs nll_ws(const tt_nll_args* a) {
  NllWs w;
  w.fused = a->hidden != nullptr;
  size_t off = 0;
  if (w.fused) {
    w.z = off;
    off = align_up(off + size_t(a->n_rows) * size_t(a->vocab) * 2);
  }
  w.row_loss = off;
  off = align_up(off + size_t(a->n_rows) * 4);
  w.total = off;
  return w;
}

}  // namespace

extern "C" int tree_nll_workspace_bytes(const tt_nll_args* a, size_t* bytes) {
  tt::clear_error();
  if (!a || !bytes) return tt::fail(TT_EINVAL, "tree_nll_workspace_bytes: NULL argument");
  if (a->n_rows < 0 || a->vocab <= 0) return tt::fail(TT_EINVAL, "tree_nll_workspace_bytes: bad sizes");
  *bytes = nll_ws(a).total;
  return TT_OK;
}

namespace ttc {

int nll_check(const tt_nll_args* a, const char* fn) {
  using std::string;
  const string f(fn);
  if (!a) return tt::fail(TT_EINVAL, f + ": args is NULL");
  const bool fused = a->hidden != nullptr || a->w_vocab != nullptr;
  const bool logits = a->logits != nullptr;
  if (fused == logits) return tt::fail(TT_EINVAL, f + ": give exactly one of logits or hidden+w_vocab");
  if (fused && (!a->hidden || !a->w_vocab)) return tt::fail(TT_EINVAL, f + ": fused mode needs hidden and w_vocab");
  if (a->n_rows < 0 || a->vocab <= 0 || a->n_tgt < 0) return tt::fail(TT_EINVAL, f + ": bad sizes");
  if (fused && a->d_model <= 0) return tt::fail(TT_EINVAL, f + ": bad d_model");
  if (a->vocab > (1 << 18)) return tt::fail(TT_EUNSUPPORTED, f + ": vocab > 262144");
  if (fused && (a->vocab % 8 != 0 || a->d_model % 8 != 0))
    return tt::fail(TT_EUNSUPPORTED, f + ": fused mode needs vocab and d_model multiples of 8");
  if (logits && a->logits_dtype != TT_F32 && a->logits_dtype != TT_BF16)
    return tt::fail(TT_EINVAL, f + ": bad logits dtype");
  if (fused && a->d_w_vocab && a->dw_dtype != TT_F32 && a->dw_dtype != TT_BF16)
    return tt::fail(TT_EINVAL, f + ": bad dw dtype");
  if (!a->loss || !a->tgt_row_ptr || (a->n_tgt > 0 && (!a->tgt_id || !a->tgt_w)))
    return tt::fail(TT_EINVAL, f + ": loss and the target CSR are required");
  if (logits && a->d_hidden) return tt::fail(TT_EINVAL, f + ": d_hidden needs fused mode");
  if (logits && a->d_w_vocab) return tt::fail(TT_EINVAL, f + ": d_w_vocab needs fused mode");
  if (fused && a->d_logits) return tt::fail(TT_EINVAL, f + ": d_logits needs logits mode");
  for (const void* p : {a->hidden, a->w_vocab, a->logits, static_cast<const void*>(a->tgt_row_ptr),
                        static_cast<const void*>(a->tgt_id), static_cast<const void*>(a->tgt_w),
                        static_cast<const void*>(a->loss), static_cast<const void*>(a->logp),
                        static_cast<const void*>(a->d_hidden), static_cast<const void*>(a->d_w_vocab),
                        static_cast<const void*>(a->d_logits), static_cast<const void*>(a->workspace)})
    if (p && !aligned16(p)) return tt::fail(TT_EINVAL, f + ": device pointers must be 16-byte aligned");
  return TT_OK;
}

}  // namespace ttc

extern "C" int tree_weighted_nll(const tt_nll_args* a, tt_stream stream) {
  tt::clear_error();
  const char* fn = "tree_weighted_nll";
  int rc = ttc::nll_check(a, fn);
  if (rc) return rc;
  const bool logits = a->logits != nullptr;
  const NllWs w = nll_ws(a);
  if (!a->workspace || a->workspace_bytes < w.total)
    return tt::fail(TT_EWORKSPACE, std::string(fn) + ": workspace too small (need " + std::to_string(w.total) +
                                       " bytes)");
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(a->workspace);
  float* row_loss = reinterpret_cast<float*>(ws + w.row_loss);
  if (logits) {
    KTimer t("nll_rows", st);
    if (launch_nll_rows(a->logits_dtype, a->logits, a->d_logits, a->n_rows, a->vocab, a->vocab, a->tgt_row_ptr,
                        a->tgt_id, a->tgt_w, a->n_tgt, a->logp, row_loss, st))
      return dev_fail(fn, "nll kernel launch");
  } else {
    uint16_t* z = reinterpret_cast<uint16_t*>(ws + w.z);
    const uint16_t* H = static_cast<const uint16_t*>(a->hidden);
    const uint16_t* W = static_cast<const uint16_t*>(a->w_vocab);
    {
      KTimer t("lmhead_z_gemm", st);
      if (a->n_rows > 0 && launch_gemm_nn(H, W, z, a->n_rows, a->vocab, a->d_model, st))
        return dev_fail(fn, "lm-head gemm");
    }
    {
      KTimer t("nll_rows", st);
      if (launch_nll_rows(TT_BF16, z, z, a->n_rows, a->vocab, a->vocab, a->tgt_row_ptr, a->tgt_id, a->tgt_w,
                          a->n_tgt, a->logp, row_loss, st))
        return dev_fail(fn, "nll kernel launch");
    }
    if (a->d_hidden && a->n_rows > 0) {
      KTimer t("lmhead_dh_gemm", st);
      if (launch_gemm_nt(z, W, static_cast<uint16_t*>(a->d_hidden), a->n_rows, a->d_model, a->vocab, st))
        return dev_fail(fn, "d_hidden gemm");
    }
    if (a->d_w_vocab) {
      KTimer t("lmhead_dw_gemm", st);
      if (launch_gemm_tn(H, z, a->d_w_vocab, a->dw_dtype == TT_F32, a->d_model, a->vocab, a->n_rows, st))
        return dev_fail(fn, "d_w_vocab gemm");
    }
  }
  {
    KTimer t("nll_sum", st);
    if (launch_sum_loss(row_loss, a->n_rows, a->loss, st)) return dev_fail(fn, "loss reduction");
  }
  return TT_OK;
}
