// Path mode (tree_attn_path): one attention layer walked depth-first over the
// tree's segments with a stack of the current path (AReaL-DTA, arXiv
// 2602.00482, summary page, Methodology in Plain English; Key Contributions 2
// for the right-to-left chunks).  The stack keeps Q and K already rotated at
// their positions (= depths), so every call runs the attention cores without
// RoPE; gradients are rotated back as they leave the stack.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <utility>
#include <vector>

#include "attn_core.h"
#include "internal.h"
#include "kernels.h"

using ttc::dev_fail;
using ttc::KTimer;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
size_t dsize(tt_dtype t) { return t == TT_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Backward chunk calls per launch on the matrix-core path: the calls of a
// launch run side by side (each with its own dO copy, D, dQ block and dK/dV
// accumulators), so one launch's grid holds the workgroups of several chunks
// and the launch's tail is shorter against its length.  Three for chunks of
// up to 2048 rows, two above (measured on the 8B-shape walk: three chunks of
// 2048 per launch 2% faster than two; three of 4096 3.5% slower than two).
constexpr int kPathCallsSmall = 3, kPathCallsLarge = 2, kPathSmallChunk = 2048;
static_assert(kPathCallsSmall <= kMaxBwdCalls && kPathCallsLarge <= kMaxBwdCalls,
              "one launch takes at most kMaxBwdCalls calls");

// Workspace carve-up, identical for the size query and the call.
struct PathWs {
  size_t qp = 0, kp = 0, vp = 0, op = 0, lsep = 0;  // stack of max_path positions
  size_t dka = 0, dva = 0;  // float32 dK, dV accumulators (backward), `slots` of max_path rows each
  size_t doc = 0, D = 0;    // per-call buffers, chunk + 64 rows, `slots` of each
  size_t dq = 0;            // float32 dQ of one call (vector kernels)
  size_t dqs = 0;           // matrix-core path: per-call bf16 dQ (rotated back, `slots`)
  size_t srow = 0, cs = 0;  // matrix-core path: tree row at each stack position, (cos, sin) table
  bool fused = false;       // matrix-core path: pushes, dO blocks and outputs by the walk's own kernels
  int slots = 1;            // chunk calls per backward launch
  size_t acc_slot = 0, doc_slot = 0, D_slot = 0, dqs_slot = 0;  // bytes per slot
  size_t total = 0;
};

PathWs path_ws(const tt_path_args* a, bool bwd) {
  const tt_path* p = a->path;
  const size_t L = size_t(p->max_path), C = size_t(p->chunk) + 64, es = dsize(a->dtype);
  const size_t hq = size_t(a->h_q), hk = size_t(a->h_kv), d = size_t(a->d);
  const bool mfma = a->dtype == TT_BF16 && ttc::mfma_shape(a->d, 64, 64);
  PathWs w;
  // several calls per launch where the combined matrix-core launch exists
  // (8-wave dQ workgroups: groups of a multiple of 4 heads, or of 2 with an
  // even number of kv heads)
  w.slots = !(mfma && bwd_combined_supported(a->h_q, a->h_kv)) ? 1
            : p->chunk <= kPathSmallChunk          ? kPathCallsSmall
                                                   : kPathCallsLarge;
  const size_t S = size_t(w.slots);
  w.acc_slot = align_up(L * hk * d * 4);
  w.doc_slot = align_up(C * hq * d * es);
  w.D_slot = align_up(C * hq * 4);
  w.dqs_slot = align_up(C * hq * d * 2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  w.qp = take(L * hq * d * es);
  w.kp = take(L * hk * d * es);
  w.vp = take(L * hk * d * es);
  w.op = take(L * hq * d * es);
  w.lsep = take(L * hq * 4);
  w.fused = mfma;
  if (mfma) {
    w.srow = take(L * 4);
    w.cs = take(L * (d / 2) * 8);
  }
  if (bwd) {
    w.dka = take(S * w.acc_slot);
    w.dva = take(S * w.acc_slot);
    w.doc = take(S * w.doc_slot);
    w.D = take(S * w.D_slot);
    w.dq = take(C * hq * d * 4);
    if (mfma) w.dqs = take(S * w.dqs_slot);
  }
  w.total = off;
  return w;
}

int check_path(const tt_path_args* a, const char* fn) {
  using std::string;
  if (!a) return tt::fail(TT_EINVAL, string(fn) + ": args is NULL");
  if (!a->path) return tt::fail(TT_EINVAL, string(fn) + ": path is NULL");
  if (a->dtype != TT_F32 && a->dtype != TT_BF16) return tt::fail(TT_EINVAL, string(fn) + ": bad dtype");
  if (a->h_q <= 0 || a->h_kv <= 0 || a->h_q % a->h_kv != 0)
    return tt::fail(TT_EINVAL, string(fn) + ": need h_q, h_kv > 0 and h_q % h_kv == 0");
  if (a->d <= 0 || a->d % 2 != 0) return tt::fail(TT_EINVAL, string(fn) + ": d must be positive and even");
  if (a->d % 16 != 0 || a->d > 256)
    return tt::fail(TT_EUNSUPPORTED, string(fn) + ": head dim must be a multiple of 16 and <= 256");
  if (a->flags & ~uint32_t(TT_ALLOW_GENERIC)) return tt::fail(TT_EINVAL, string(fn) + ": unknown flags");
  if (a->dtype == TT_BF16 && !(a->flags & TT_ALLOW_GENERIC) && !ttc::mfma_shape(a->d, 64, 64))
    return tt::fail(TT_EUNSUPPORTED, string(fn) +
                                         ": bf16 attention runs on the matrix cores for head dim 128 only; "
                                         "TT_ALLOW_GENERIC selects the vector kernels");
  if (!(a->scale >= 0.f) || !std::isfinite(a->scale)) return tt::fail(TT_EINVAL, string(fn) + ": bad scale");
  if (!(a->rope_base >= 0.f) || !std::isfinite(a->rope_base))
    return tt::fail(TT_EINVAL, string(fn) + ": bad rope_base");
  const int64_t N = a->path->tree->N;
  if (N * a->h_q * a->d * 4 > (int64_t(1) << 40)) return tt::fail(TT_EOVERFLOW, string(fn) + ": tensors too large");
  if (N > 0 && (!a->q || !a->k || !a->v || !a->o || !a->lse))
    return tt::fail(TT_EINVAL, string(fn) + ": q, k, v, o and lse are required");
  if (N > 0 && a->d_o && (!a->d_q || !a->d_k || !a->d_v))
    return tt::fail(TT_EINVAL, string(fn) + ": d_q, d_k and d_v are required with d_o");
  if (a->path->max_path > 0 && !a->plan) return tt::fail(TT_EINVAL, string(fn) + ": plan is NULL");
  for (const void* p : {a->q, a->k, a->v, static_cast<const void*>(a->o), static_cast<const void*>(a->lse), a->d_o,
                        static_cast<const void*>(a->d_q), static_cast<const void*>(a->d_k),
                        static_cast<const void*>(a->d_v), a->plan})
    if (p && !aligned16(p)) return tt::fail(TT_EINVAL, string(fn) + ": device pointers must be 16-byte aligned");
  if (a->workspace && (reinterpret_cast<uintptr_t>(a->workspace) & (kAlign - 1)) != 0)
    return tt::fail(TT_EINVAL, string(fn) + ": workspace must be 256-byte aligned");
  return TT_OK;
}

// Chunks of stack positions [p0, p1) (boundaries at multiples of chunk).
std::vector<std::pair<int32_t, int32_t>> chunks(int32_t p0, int32_t p1, int32_t chunk) {
  std::vector<std::pair<int32_t, int32_t>> v;
  for (int32_t c0 = p0; c0 < p1;) {
    const int32_t c1 = std::min(p1, (c0 / chunk + 1) * chunk);
    v.push_back({c0, c1});
    c0 = c1;
  }
  return v;
}

}  // namespace

extern "C" int tree_path_plan_bytes(const tt_path* p, size_t* bytes) {
  tt::clear_error();
  if (!p || !bytes) return tt::fail(TT_EINVAL, "tree_path_plan_bytes: NULL argument");
  *bytes = p->chain ? p->chain->plan.size() * sizeof(int32_t) : 0;
  return TT_OK;
}

extern "C" int tree_path_plan_upload(const tt_path* p, void* dev_plan, size_t bytes, tt_stream stream) {
  tt::clear_error();
  if (!p) return tt::fail(TT_EINVAL, "tree_path_plan_upload: path is NULL");
  if (!p->chain) return TT_OK;  // an empty tree has no calls
  return tree_plan_upload(p->chain, dev_plan, bytes, stream);
}

extern "C" int tree_path_workspace_bytes(const tt_path_args* a, size_t* bytes) {
  tt::clear_error();
  if (!bytes) return tt::fail(TT_EINVAL, "tree_path_workspace_bytes: bytes is NULL");
  if (!a || !a->path) return tt::fail(TT_EINVAL, "tree_path_workspace_bytes: args/path is NULL");
  if (a->h_q <= 0 || a->h_kv <= 0 || a->d <= 0 || (a->dtype != TT_F32 && a->dtype != TT_BF16))
    return tt::fail(TT_EINVAL, "tree_path_workspace_bytes: bad geometry");
  *bytes = path_ws(a, a->d_o != nullptr).total;
  return TT_OK;
}

extern "C" int tree_attn_path(const tt_path_args* a, tt_stream stream) {
  tt::clear_error();
  const char* fn = "tree_attn_path";
  int rc = check_path(a, fn);
  if (rc) return rc;
  const tt_path* p = a->path;
  const bool bwd = a->d_o != nullptr;
  const PathWs w = path_ws(a, bwd);
  if (w.total > 0 && (!a->workspace || a->workspace_bytes < w.total))
    return tt::fail(TT_EWORKSPACE, std::string(fn) + ": workspace too small (need " + std::to_string(w.total) +
                                       " bytes)");
  if (p->tree->N == 0) return TT_OK;
  if ((rc = ttc::plan_check(p->chain, a->plan, fn))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(a->workspace);
  const tt_dtype dt = a->dtype;
  const size_t es = dsize(dt), hq = size_t(a->h_q), hk = size_t(a->h_kv), d = size_t(a->d);
  const size_t qrow = hq * d * es, krow = hk * d * es;  // bytes per row
  const float rb = a->rope_base;

  const PlanPtrs P = ttc::plan_ptrs(p->chain, a->plan);
  AttnGeom g;
  g.h_q = a->h_q;
  g.h_kv = a->h_kv;
  g.d = a->d;
  g.scale = a->scale == 0.f ? float(1.0 / std::sqrt(double(a->d))) : a->scale;
  g.rope_base = 0.f;  // the stack holds rotated rows
  const double qmul = ttc::q_operand_scale(dt, g, P);  // and queries in the attention cores' operand form

  char *Qp = ws + w.qp, *Kp = ws + w.kp, *Vp = ws + w.vp, *Op = ws + w.op;
  float* LSEp = reinterpret_cast<float*>(ws + w.lsep);
  float* dKa = reinterpret_cast<float*>(ws + w.dka);
  float* dVa = reinterpret_cast<float*>(ws + w.dva);
  char* dOc = ws + w.doc;
  float* D = reinterpret_cast<float*>(ws + w.D);
  float* dq = reinterpret_cast<float*>(ws + w.dq);
  const char* q = static_cast<const char*>(a->q);
  const char* k = static_cast<const char*>(a->k);
  const char* v = static_cast<const char*>(a->v);
  char* o = static_cast<char*>(a->o);
  const char* d_o = static_cast<const char*>(a->d_o);
  char* d_q = static_cast<char*>(a->d_q);
  char* d_k = static_cast<char*>(a->d_k);
  char* d_v = static_cast<char*>(a->d_v);

  if (bwd) {
    KTimer t("path_clear", st);
    if (launch_fill_zero(dKa, size_t(w.slots) * w.acc_slot, st) ||
        launch_fill_zero(dVa, size_t(w.slots) * w.acc_slot, st))
      return dev_fail(fn, "clear");
  }
  // matrix-core path: pushes rotate with this table of stack positions
  // (= depths), and the dQ and dK/dV epilogues rotate back with it (dQ stored
  // as bf16 rows of the call)
  char* dqs = bwd && w.dqs ? ws + w.dqs : nullptr;
  int32_t* srow = w.fused ? reinterpret_cast<int32_t*>(ws + w.srow) : nullptr;
  float2* cs_tab = nullptr;
  if (w.fused && rb != 0.f) {
    cs_tab = reinterpret_cast<float2*>(ws + w.cs);
    KTimer t("rope_table", st);
    if (launch_rope_table(cs_tab, p->max_path, a->d / 2, rb, st)) return dev_fail(fn, "rope table");
  }
  // the segments of a round and the part of [c0, c1) each one holds
  const auto seg_of = [&](const tt_path::Round& rd, int32_t i) -> const tt_path::Seg& {
    return p->segs[size_t(rd.bwd ? -1 - p->events[size_t(i)] : p->events[size_t(i)])];
  };
  for (const tt_path::Round& rd : p->rounds) {
    if (!rd.bwd) {
      // enter: push each segment's rows, then one chunked forward over the
      // round's positions against the stack
      for (int32_t i = rd.ev0; i < rd.ev1; ++i) {
        const tt_path::Seg& s = seg_of(rd, i);
        const size_t r0 = size_t(s.row0), n = size_t(s.len), d0 = size_t(s.depth0);
        KTimer t("path_push", st);
        if (w.fused) {
          // Q rotated and scaled, K rotated, V copied, srow set: one launch
          if (launch_path_push(q, k, v, Qp, Kp, Vp, srow, cs_tab, s.row0, s.depth0, s.len, a->h_q, a->h_kv, a->d,
                               float(qmul), st))
            return dev_fail(fn, "push");
          continue;
        }
        if (launch_rope(q + r0 * qrow, Qp + d0 * qrow, dt, dt, false, P, s.depth0, s.len, a->h_q, a->d, rb, false,
                        st, qmul) ||
            launch_rope(k + r0 * krow, Kp + d0 * krow, dt, dt, false, P, s.depth0, s.len, a->h_kv, a->d, rb, false,
                        st) ||
            hipMemcpyAsync(Vp + d0 * krow, v + r0 * krow, n * krow, hipMemcpyDeviceToDevice, st) != hipSuccess)
          return dev_fail(fn, "push");
      }
      {
        // one call over the whole round: the visibility rule keeps each query
        // to the positions at or below it (only the backward is chunked)
        const int32_t qo = rd.p0 & ~63;
        g.q_off = qo;
        g.n_q = rd.p1 - qo;
        g.n_k = rd.p1;
        if ((rc = ttc::attn_fwd_core(dt, P, g, Qp + size_t(qo) * qrow, Kp, Vp, Op + size_t(qo) * qrow,
                                     LSEp + size_t(qo) * hq, false, st)))
          return rc;
      }
      if (w.fused) {
        // the round's segments are stacked one on the next: positions [p0, p1)
        KTimer t("path_out", st);
        if (launch_path_scatter(Op, o, int64_t(qrow), rd.p0, LSEp, a->lse, a->h_q, srow, rd.p0, rd.p1, st))
          return dev_fail(fn, "forward outputs");
        continue;
      }
      for (int32_t i = rd.ev0; i < rd.ev1; ++i) {
        const tt_path::Seg& s = seg_of(rd, i);
        const size_t r0 = size_t(s.row0), n = size_t(s.len), d0 = size_t(s.depth0);
        KTimer t("path_out", st);
        if (hipMemcpyAsync(o + r0 * qrow, Op + d0 * qrow, n * qrow, hipMemcpyDeviceToDevice, st) != hipSuccess ||
            hipMemcpyAsync(a->lse + r0 * hq, LSEp + d0 * hq, n * hq * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
          return dev_fail(fn, "forward outputs");
      }
    } else if (bwd) {
      // leave: one backward over the round's positions, chunks right to left
      // (every descendant's gradient has arrived), then pop each segment.
      // With several slots, consecutive chunks share a launch, each adding
      // into its own accumulators (no two writers per key); the pops sum them.
      const auto cs = chunks(rd.p0, rd.p1, p->chunk);
      const size_t nch = cs.size(), S = size_t(w.slots);
      for (size_t i0 = 0; i0 < nch; i0 += S) {
        const size_t nc = std::min(S, nch - i0);
        BwdCallPtrs calls[kMaxBwdCalls];
        float* Ds[kMaxBwdCalls];
        PathChunks pc{};  // the launch's chunks, for the walk's own kernels
        pc.n = int32_t(nc);
        for (size_t u = 0; u < nc; ++u) {
          const int32_t c0 = cs[nch - 1 - i0 - u].first, c1 = cs[nch - 1 - i0 - u].second, qo = c0 & ~63;
          const size_t pad = size_t(c0 - qo);
          char* dOu = dOc + u * w.doc_slot;
          Ds[u] = reinterpret_cast<float*>(reinterpret_cast<char*>(D) + u * w.D_slot);
          pc.c[u] = PathChunk{dOu, Ds[u], dqs ? dqs + u * w.dqs_slot : nullptr, qo, c0, c1};
          if (!w.fused) {
            KTimer t("path_dout", st);
            if (launch_fill_zero(dOu, pad * qrow, st)) return dev_fail(fn, "upstream gradient");
            for (int32_t i = rd.ev0; i < rd.ev1; ++i) {
              const tt_path::Seg& s = seg_of(rd, i);
              const int32_t lo = std::max(c0, s.depth0), hi = std::min(c1, s.depth0 + s.len);
              if (lo >= hi) continue;
              const size_t row = size_t(s.row0) + size_t(lo - s.depth0);
              if (hipMemcpyAsync(dOu + size_t(lo - qo) * qrow, d_o + row * qrow, size_t(hi - lo) * qrow,
                                 hipMemcpyDeviceToDevice, st) != hipSuccess)
                return dev_fail(fn, "upstream gradient");
            }
          }
          g.q_off = qo;
          g.n_q = c1 - qo;
          g.n_k = c1;
          calls[u] = BwdCallPtrs{Qp + size_t(qo) * qrow, dOu, LSEp + size_t(qo) * hq, Ds[u], nullptr,
                                 dqs ? dqs + u * w.dqs_slot : nullptr,
                                 reinterpret_cast<char*>(dKa) + u * w.acc_slot,
                                 reinterpret_cast<char*>(dVa) + u * w.acc_slot, g};
        }
        if (w.fused) {
          // every chunk's dO rows gathered through srow (zeros on the pad
          // rows) and D = rowsum(dO o O): one launch
          KTimer t("path_dout", st);
          if (launch_path_dout_pre(Op, d_o, srow, pc, a->h_q, a->d, st)) return dev_fail(fn, "upstream gradient");
        }
        bool dq_done = false;
        if (S > 1) {
          for (size_t u = 0; u < nc && !w.fused; ++u) {
            KTimer t("attn_bwd_pre", st);
            const AttnGeom& gu = calls[u].g;
            if (launch_bwd_pre(dt, Op + size_t(gu.q_off) * qrow, calls[u].d_o, Ds[u], int64_t(gu.n_q) * gu.h_q, gu.d,
                               st))
              return dev_fail(fn, "backward preprocess");
          }
          KTimer t("attn_bwd_mfma", st);
          if (launch_bwd_mfma_multi(calls, int(nc), Kp, Vp, true, cs_tab, P, false, st))
            return dev_fail(fn, "backward kernel");
          dq_done = true;
        } else if ((rc = ttc::attn_bwd_core(dt, P, calls[0].g, calls[0].q, Kp, Vp,
                                            Op + size_t(calls[0].g.q_off) * qrow, calls[0].d_o, calls[0].lse, D,
                                            dq, dKa, dVa, true, false, cs_tab, st, dqs, &dq_done))) {
          return rc;
        }
        // dQ rows of each chunk to their tree rows: from the bf16 blocks the
        // kernel rotated back, through srow in one launch; otherwise segment
        // by segment, copied, or rotated back here from the fp32 block
        // (vector kernels)
        if (w.fused && dq_done) {
          KTimer t("dq_finalize", st);
          if (launch_path_dq_scatter(d_q, int64_t(qrow), srow, pc, st)) return dev_fail(fn, "dq finalize");
          continue;
        }
        for (size_t u = 0; u < nc; ++u) {
          const int32_t c0 = cs[nch - 1 - i0 - u].first, c1 = cs[nch - 1 - i0 - u].second, qo = c0 & ~63;
          const char* dqu = dqs ? dqs + u * w.dqs_slot : nullptr;
          KTimer t("dq_finalize", st);
          for (int32_t i = rd.ev0; i < rd.ev1; ++i) {
            const tt_path::Seg& s = seg_of(rd, i);
            const int32_t lo = std::max(c0, s.depth0), hi = std::min(c1, s.depth0 + s.len);
            if (lo >= hi) continue;
            const size_t row = size_t(s.row0) + size_t(lo - s.depth0);
            if (dq_done ? hipMemcpyAsync(d_q + row * qrow, dqu + size_t(lo - qo) * qrow, size_t(hi - lo) * qrow,
                                         hipMemcpyDeviceToDevice, st) != hipSuccess
                        : launch_rope(dq + size_t(lo - qo) * hq * d, d_q + row * qrow, TT_F32, dt, false, P, lo,
                                      hi - lo, a->h_q, a->d, rb, true, st) != 0)
              return dev_fail(fn, "dq finalize");
          }
        }
      }
      for (int32_t i = rd.ev0; i < rd.ev1; ++i) {
        const tt_path::Seg& s = seg_of(rd, i);
        const size_t r0 = size_t(s.row0), n = size_t(s.len), d0 = size_t(s.depth0);
        KTimer t("path_pop", st);
        if (w.slots > 1) {
          // the matrix-core kernel rotated each contribution back at the
          // key's depth (when there is RoPE): sum the slots and convert
          if (launch_acc_pop(dKa + d0 * hk * d, dVa + d0 * hk * d, w.acc_slot / 4, w.slots, d_k + r0 * krow,
                             d_v + r0 * krow, int64_t(n) * int64_t(hk * d), st))
            return dev_fail(fn, "pop");
          continue;
        }
        // with the table, the matrix-core dK/dV kernel already rotated each
        // contribution back at the key's depth (rotation is linear, so the
        // sums are in the output frame): convert only
        if (launch_rope(dKa + d0 * hk * d, d_k + r0 * krow, TT_F32, dt, false, P, s.depth0, s.len, a->h_kv, a->d,
                        cs_tab ? 0.f : rb, true, st) ||
            launch_rope(dVa + d0 * hk * d, d_v + r0 * krow, TT_F32, dt, false, P, s.depth0, s.len, a->h_kv, a->d,
                        0.f, false, st) ||
            launch_fill_zero(dKa + d0 * hk * d, n * hk * d * 4, st) ||
            launch_fill_zero(dVa + d0 * hk * d, n * hk * d * 4, st))
          return dev_fail(fn, "pop");
      }
    }
  }
  return TT_OK;
}
