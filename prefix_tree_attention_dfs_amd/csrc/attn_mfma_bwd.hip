// bf16 MFMA tree attention backward, head dim 128 (gfx950).
//
// Gradients of sum(dO * O) with the probabilities recomputed from the
// forward's LSE; a shared prefix key collects the gradient of every query in
// its subtree (AReaL-DTA summary, Key Contributions 1 and Methodology:
// shared segments are backpropagated once with the gradients of all
// descendant leaves accumulated).
//
// Two kernels, neither uses atomics:
//   dq_mfma_kernel   query-stationary (the forward's walk over the block's
//                    non-empty key tiles):  S^T = K Q^T, P^T, dP^T = V dO^T,
//                    dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// Q comes multiplied by scale * log2(e), so S is in log2 units; S's
// accumulators start at -LSE log2(e) and dP's at -D, so P = exp2(S) and
// dS = P dP come straight from the products.
//   dkdv_mfma_kernel key-stationary: one workgroup per 256 keys x kv head,
//                    each of its 8 waves owning 32 keys (K in registers, V
//                    in LDS, both loaded once).  It streams 64-row
//                    Q / dO tiles of every query head of the group over the
//                    contiguous range of query rows that see its keys, top
//                    down, loaded straight from global memory into LDS (no
//                    staging registers):  S = Q K^T, P, dP = dO V^T, dS,
//                    dV^T += dO^T P, dK^T += Q^T dS.
// Recomputing S and dP in both kernels costs 14 d MFMA flops per visible pair
// instead of 10 d, in exchange for no fp32 atomic traffic on dQ.
// Where both kinds of workgroup have 8 waves (groups of a multiple of 4 query
// heads; groups of 2 over an even number of kv heads, a dQ workgroup then
// taking two kv heads) they run as one launch, bwd_mfma_kernel (or, for
// several independent calls, bwd_multi_mfma_kernel), the kind with the
// longest workgroups first.
#include <algorithm>

#include "device.h"
#include "kernels.h"
#include "mfma_common.h"

using namespace ttm;
using ttd::Elem;

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ dQ
template <int G>
struct DqCfg {
  static constexpr int WAVES = 2 * G;  // each wave: 32 query rows of one head
  static constexpr int THREADS = WAVES * 64;
  static constexpr int CH = (BK * D / 8) / THREADS;
};

struct __align__(16) DqStage {
  uint16_t K[BK * D];  // swizzled: row reads (S^T) and transposed reads (dQ^T)
  uint16_t V[BK * D];  // swizzled: row reads (dP^T)
  int32_t end[BK];
};

// FIN: the epilogue rotates dQ back at the query's depth (R^T with the
// caller's (cos, sin) table; none: no rotation) and stores it in bf16 to
// dq_out; otherwise it stores the rotated-frame dQ in fp32 to dq_acc.
// WIDE: K/V of 2 GiB or more (each tile's descriptors start at the tile).
// The body of the dQ kernel for workgroup `bid` (the kernel below, or the
// dQ part of the combined backward launch).
// KVP: key/value heads per workgroup.  With KVP = 2 the workgroup runs the
// same query block for two kv heads (2 G waves each, each set staging its own
// head's K/V tiles: st[2 * buffer + set]); both sets walk the block's one tile
// list, so they meet at every barrier.  That gives GQA-2 workgroups of 8
// waves, the size the combined launch needs.
template <int G, bool FIN, bool WIDE, int KVP = 1>
__device__ __forceinline__ void dq_body(
    DqStage* __restrict__ st, const int bid, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ Dv, float* __restrict__ dq_acc, uint16_t* __restrict__ dq_out,
    const float2* __restrict__ cs_tab, const PlanPtrs& P, const AttnGeom& g, int full_range, int qb_first, int n_qb,
    int nsub) {
  static_assert(KVP == 1 || KVP == 2, "one or two kv heads per workgroup");
  constexpr int KW = DqCfg<G>::WAVES;  // waves per kv head
  if (!plan_matches(P)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int kvs = KVP == 1 ? 0 : wave / KW, kw = KVP == 1 ? wave : wave % KW;  // kv set, wave within it
  const int kvh = (bid % (g.h_kv / KVP)) * KVP + kvs;
  const int rest = bid / (g.h_kv / KVP);
  const int sub = rest % nsub, idx = rest / nsub;
  const int qb = full_range ? ld_uniform(P.qb_order, idx) : (qb_first + n_qb - 1 - idx);
  const int head = (kvh * nsub + sub) * G + (kw >> 1);
  const int pos0 = (wave & 1) * 32;
  const int row = qb * BQ - g.q_off + pos0 + r;  // q-buffer row of this lane's query
  const bool rok = row < g.n_q;
  const int qpos = qb * BQ + pos0 + r;

  bf16x8 qf[8], of[8];
#pragma unroll
  for (int dc = 0; dc < 8; ++dc) {
    const int64_t off = (int64_t(row) * g.h_q + head) * D + dc * 16 + 8 * hh;
    qf[dc] = rok ? ld16(q + off) : zero8();
    of[dc] = rok ? ld16(d_o + off) : zero8();
  }
  const float neg_lse2 = rok ? -lse[int64_t(row) * g.h_q + head] * kLog2e : 0.f;
  const float neg_D = rok ? -Dv[int64_t(row) * g.h_q + head] : 0.f;

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = zero16();

  // tile staging: buffer loads, zero past n_k keys (end = 0 there: invisible)
  const int64_t kv_elems = int64_t(g.n_k) * g.h_kv * D;
  const int64_t tile_elems = int64_t(BK) * g.h_kv * D;
  const rsrc_t re = make_rsrc(P.end, uint32_t(g.n_k) * 4);
  const rsrc_t rk0 = make_rsrc(k, WIDE ? 0u : uint32_t(kv_elems * 2)), rv0 = make_rsrc(v, WIDE ? 0u : uint32_t(kv_elems * 2));
  // K and V tiles go from global memory straight into LDS in the swizzled
  // layout, NL loads of 1 KB per wave each, as in the forward (each kv set
  // loads its own head's tiles)
  constexpr int NL = (BK * D * 2 / 1024) / KW;
  static_assert(NL * KW * 1024 == BK * D * 2, "the waves' 1 KB loads cover a tile");
  uint32_t dvoff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (kw * NL + i) * 64 + lane;
    const int key = p >> 4, c = (p & 15) ^ swz(p >> 4);
    dvoff[i] = (uint32_t(key * g.h_kv + kvh) * D + c * 8) * 2;
  }
  int32_t ereg = 0;
  auto load_tile = [&](int kb, DqStage& s) {
    const uint32_t kbase = lds_u32(s.K) + kw * NL * 1024, vbase = lds_u32(s.V) + kw * NL * 1024;
    if constexpr (WIDE) {
      const int64_t t0 = int64_t(kb) * tile_elems;
      const uint32_t bytes = tile_rec_bytes(kv_elems - t0);
      const rsrc_t rk = make_rsrc(k + t0, bytes), rv = make_rsrc(v + t0, bytes);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        dma16(rk, dvoff[i], 0, kbase + i * 1024);
        dma16(rv, dvoff[i], 0, vbase + i * 1024);
      }
    } else {
      const uint32_t so = uint32_t(kb) * uint32_t(tile_elems * 2);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        dma16(rk0, dvoff[i], so, kbase + i * 1024);
        dma16(rv0, dvoff[i], so, vbase + i * 1024);
      }
    }
    if (tid < BK) ereg = bloadi(re, uint32_t(tid) * 4, uint32_t(kb) * BK * 4);
  };
  auto store_end = [&](DqStage& s) {
    if (tid < BK) s.end[tid] = ereg;
  };

  // tile-list entries two ahead, as in the forward
  const int e0 = ld_uniform(P.qb_ptr, qb), e1 = ld_uniform(P.qb_ptr, qb + 1);
  int cur = e0 < e1 ? ld_uniform(P.qb_tiles, e0) : 0;
  int nxt = e0 + 1 < e1 ? ld_uniform(P.qb_tiles, e0 + 1) : 0;
  // the tile's end[] (the same for every kv head) goes to set 0's stage only
  if (e0 < e1) {
    load_tile(cur & kKbMask, st[kvs]);
    store_end(st[0]);
  }
  wait_vmem();  // also the direct-to-LDS loads, which the compiler does not track
  __syncthreads();
  for (int e = e0; e < e1; ++e) {
    const int sidx = (e - e0) & 1;
    const int ent = cur;
    const int kb = ent & kKbMask;
    const bool full = (ent & kFull) != 0;
    cur = nxt;
    if (e + 2 < e1) nxt = ld_uniform(P.qb_tiles, e + 2);
    // the other buffer was last read in the previous tile
    if (e + 1 < e1) load_tile(cur & kKbMask, st[(sidx ^ 1) * KVP + kvs]);
    const DqStage& S = st[sidx * KVP + kvs];
    const int32_t* __restrict__ S_end = st[sidx * KVP].end;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 s = splat16_here(neg_lse2), dp = splat16_here(neg_D);
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const bf16x8 a = lds_read16(&S.K[soff(kt * 32 + r, dc * 16 + 8 * hh)]);
        s = mfma(a, qf[dc], s);
        const bf16x8 b = lds_read16(&S.V[soff(kt * 32 + r, dc * 16 + 8 * hh)]);
        dp = mfma(b, of[dc], dp);
      }
      // dS is computed at raised wave priority, as in the dK/dV kernel, so the
      // wave's own dQ products start sooner (measured 0.6% on this kernel)
      __builtin_amdgcn_s_setprio(1);
      if (full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = exp2_fast(s[i]) * dp[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool vis = (kb * BK + kl <= qpos) & (qpos < S_end[kl]);
          s[i] = vis ? exp2_fast(s[i]) * dp[i] : 0.f;
        }
      }
      const bf16x8 d0 = c_to_b(s, 0), d1 = c_to_b(s, 1);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        acc[dt] = mfma(tr_frag_swz(S.K, kt * 32, dt * 32, lane), d0, acc[dt]);
        acc[dt] = mfma(tr_frag_swz(S.K, kt * 32 + 16, dt * 32, lane), d1, acc[dt]);
      }
    }
    if (e + 1 < e1) store_end(st[(sidx ^ 1) * KVP]);
    wait_vmem();  // this wave's direct-to-LDS loads of the next tile have landed
    __syncthreads();
  }
  if (!rok) return;
  if (FIN) {
    // coordinates (c, c+64) of a rotation pair are the same register of
    // blocks dt and dt+2: dQ = R^T (scale * dQ') in registers, one bf16 rounding
    const float2* __restrict__ cs_row = cs_tab ? cs_tab + int64_t(P.depth[qpos]) * (D / 2) : nullptr;
    uint16_t* orow = dq_out + (int64_t(row) * g.h_q + head) * D;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int c0 = dt * 32 + 8 * i4 + 4 * hh;
        bf16x4 lo4, hi4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x1 = acc[dt][4 * i4 + e] * g.scale, x2 = acc[dt + 2][4 * i4 + e] * g.scale;
          float cs = 1.f, sn = 0.f;
          if (cs_row) {
            const float2 t = cs_row[c0 + e];
            cs = t.x;
            sn = t.y;
          }
          lo4[e] = __bf16(x1 * cs + x2 * sn);
          hi4[e] = __bf16(x2 * cs - x1 * sn);
        }
        *reinterpret_cast<bf16x4*>(orow + c0) = lo4;
        *reinterpret_cast<bf16x4*>(orow + c0 + 64) = hi4;
      }
    return;
  }
  float* out = dq_acc + (int64_t(row) * g.h_q + head) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = acc[dt][4 * i4 + e] * g.scale;
      *reinterpret_cast<f32x4*>(out + dt * 32 + 8 * i4 + 4 * hh) = w;
    }
}

// ------------------------------------------------------------------ dK, dV
// One workgroup per 256 keys x kv head, 8 waves (two per SIMD); wave w owns
// keys 32 w .. +32 for the whole kernel: its K fragments (B operands of S)
// sit in registers, loaded once from global memory, and V of the 256 keys in
// LDS.  Query tiles of 64 rows (Q, dO, LSE, D of one head) stream through a
// double-buffered stage; every wave runs both 32-row halves of each staged
// tile, so a stage (32 KB) feeds 512 MFMAs and each wave's dK, dV are
// complete at the end (no exchange between waves).
constexpr int KV_WAVES = 8;
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_KEYS = 32 * KV_WAVES;             // keys per workgroup
constexpr int QT = 64;                             // query rows per staged tile
constexpr int VCH = (KV_KEYS * D / 8) / KV_THREADS;  // 16-byte chunks of V per thread

struct __align__(16) KvStage {
  uint16_t Q[QT * D];  // swizzled (row reads for S, transposed reads for dK^T)
  uint16_t O[QT * D];  // dO, swizzled (row reads for dP, transposed reads for dV^T)
  float s0[QT];  // -LSE log2(e): start value of the S accumulator (Q carries scale log2(e)), so P = exp2(S)
  float d0[QT];  // -D: start value of the dP accumulator, so that dS = P dP
};

struct __align__(16) KvLds {
  uint16_t V[KV_KEYS * KSTR];  // padded: row reads only
  KvStage st[2];
  int32_t red[KV_WAVES];
};
// After the tile loop of an accumulating call the whole KvLds is reused:
// each wave's 32 x 128 fp32 dK (then dV) block, rows EST floats apart.
constexpr int EST = 132;
static_assert(KV_WAVES * 32 * EST * 4 <= int(sizeof(KvLds)), "the epilogue blocks fit in the LDS");

// The body of the dK/dV kernel for workgroup `bid` (the kernel below, or the
// dK/dV part of the combined backward launch).
// G: query heads per kv head (0: any group size, read from g at run time).
// WIDE: Q / dO of 2 GiB or more (each tile's descriptors start at the tile).
template <int G, bool ACC, typename TG, bool WIDE>
__device__ __forceinline__ void dkdv_body(
    KvLds& L, const int bid, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ Dv, TG* __restrict__ d_k, TG* __restrict__ d_v, const float2* __restrict__ cs_tab,
    const PlanPtrs& P, const AttnGeom& g) {
  if (!plan_matches(P)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int kvh = bid % g.h_kv;
  // a whole-tree call takes its key groups in the plan's launch order (latest
  // query-range end first); a chunk call in key order
  const bool whole = g.q_off == 0 && g.n_q == P.N && g.n_k == P.N;
  const int kb2 = whole ? ld_uniform(P.kb_order, bid / g.h_kv) : bid / g.h_kv;
  const int kbase = kb2 * KV_KEYS;
  const int j = kbase + wave * 32 + r;  // this lane's key (lane column of S, dP, dK^T, dV^T)
  const bool jok = j < g.n_k;

  // V of the workgroup's keys -> LDS (rows past n_k are zero)
#pragma unroll
  for (int u = 0; u < VCH; ++u) {
    const int c = tid + u * KV_THREADS;
    const int key = c >> 4, dch = c & 15;
    const int jj = kbase + key;
    const bool ok = jj < g.n_k;
    const bf16x8 vx = ld16(v + (int64_t(ok ? jj : g.n_k - 1) * g.h_kv + kvh) * D + dch * 8);
    *reinterpret_cast<bf16x8*>(&L.V[key * KSTR + dch * 8]) = ok ? vx : zero8();
  }
  // this wave's 32 keys as B operands of S = Q K^T, straight from global
  // memory: lane (r, hh) holds K[j][16 dc + 8 hh .. +8]
  bf16x8 kf[8];
  {
    const uint16_t* krow = k + (int64_t(jok ? j : 0) * g.h_kv + kvh) * D + 8 * hh;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) kf[dc] = jok ? ld16(krow + dc * 16) : zero8();
  }
  const int endj = jok ? P.end[j] : -1;

  // query rows seen by this workgroup's keys: [kbase, max end) within the call's query range
  int mx = jok ? endj : 0, mn = jok ? endj : 0x7FFFFFFF;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = max(mx, __shfl_xor(mx, o, 64));
    mn = min(mn, __shfl_xor(mn, o, 64));
  }
  if (lane == 0) L.red[wave] = mx;
  __syncthreads();
  int hi = 0;
#pragma unroll
  for (int w = 0; w < KV_WAVES; ++w) hi = max(hi, L.red[w]);
  const int wave_min_end = __builtin_amdgcn_readfirstlane(mn);
  const int lo = max(kbase, g.q_off);
  hi = min(hi, g.q_off + g.n_q);
  const int wave_kmax = kbase + wave * 32 + 31;

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  const int qt_first = lo / QT;  // query tiles are aligned to 64 tree rows
  const int n_qt = hi > lo ? (hi - 1) / QT - qt_first + 1 : 0;
  const int GG = G > 0 ? G : g.h_q / g.h_kv;
  const int n_steps = n_qt * GG;

  float lreg = 0.f, dreg = 0.f;
  // query rows past n_q read zeros (tiles start at or after q_off, which is
  // a multiple of 64, so rows are never below the buffer)
  const int64_t q_elems = int64_t(g.n_q) * g.h_q * D, r_elems = int64_t(g.n_q) * g.h_q;
  const uint32_t qb0 = WIDE ? 0u : uint32_t(q_elems * 2), rb0 = WIDE ? 0u : uint32_t(r_elems * 4);
  const rsrc_t rq0 = make_rsrc(q, qb0), ro0 = make_rsrc(d_o, qb0), rl0 = make_rsrc(lse, rb0), rd0 = make_rsrc(Dv, rb0);
  // Q and dO tiles (64 rows x 128 bf16 = 16 KB each) go from global memory
  // straight into LDS: 16 loads of 1 KB per tile, two per wave.  Lane l of
  // load j fills LDS slot 64 j + l = (row, stored chunk) = ((64 j + l) / 16,
  // (64 j + l) % 16), so it fetches global chunk (stored chunk ^ swz(row)) of
  // that row and the tile lands in the swizzled layout the reads expect.
  uint32_t dvoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;
    const int row = p >> 4, c = (p & 15) ^ swz(p >> 4);
    dvoff[i] = (uint32_t(row) * g.h_q * D + c * 8) * 2;
  }
  auto load_tile = [&](int step, KvStage& s) {
    // query tiles from the top down: workgroups over a shared prefix have the
    // same upper end, so they walk the same tiles together and share them in L2
    const int rev = n_steps - 1 - step;
    const int qt = qt_first + rev / GG, head = kvh * GG + rev % GG;
    const int64_t rowh = int64_t(qt * QT - g.q_off) * g.h_q + head;  // (row, head) of the tile's first row
    const uint32_t qb = lds_u32(s.Q) + wave * 2048, ob = lds_u32(s.O) + wave * 2048;
    if constexpr (WIDE) {
      const uint32_t qbytes = tile_rec_bytes(q_elems - rowh * D);
      const uint32_t rbytes = tile_rec_bytes(2 * (r_elems - rowh));  // float32 entries
      const rsrc_t rq = make_rsrc(q + rowh * D, qbytes), ro = make_rsrc(d_o + rowh * D, qbytes);
      const rsrc_t rl = make_rsrc(lse + rowh, rbytes), rd = make_rsrc(Dv + rowh, rbytes);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16(rq, dvoff[i], 0, qb + i * 1024);
        dma16(ro, dvoff[i], 0, ob + i * 1024);
      }
      if (tid < QT) {
        lreg = bloadf(rl, uint32_t(tid) * g.h_q * 4, 0);
        dreg = bloadf(rd, uint32_t(tid) * g.h_q * 4, 0);
      }
    } else {
      const uint32_t rh = uint32_t(rowh);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16(rq0, dvoff[i], rh * D * 2, qb + i * 1024);
        dma16(ro0, dvoff[i], rh * D * 2, ob + i * 1024);
      }
      if (tid < QT) {
        lreg = bloadf(rl0, uint32_t(tid) * g.h_q * 4, rh * 4);
        dreg = bloadf(rd0, uint32_t(tid) * g.h_q * 4, rh * 4);
      }
    }
  };
  auto store_rows = [&](KvStage& s) {
    if (tid < QT) {
      s.s0[tid] = -lreg * kLog2e;
      s.d0[tid] = -dreg;
    }
  };

  if (n_steps > 0) {
    load_tile(0, L.st[0]);
    store_rows(L.st[0]);
  }
  wait_vmem();  // also the direct-to-LDS loads, which the compiler does not track
  __syncthreads();
  const uint16_t* Vt = L.V + (wave * 32 + r) * KSTR + 8 * hh;
  for (int step = 0; step < n_steps; ++step) {
    const int sidx = step & 1;
    const int qt = qt_first + (n_steps - 1 - step) / GG;
    if (step + 1 < n_steps) load_tile(step + 1, L.st[sidx ^ 1]);  // that stage was last read in the previous step
    const KvStage& S = L.st[sidx];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int q0 = qt * QT + mt * 32;  // tree row of this half's first query
      // every (query, key) pair of this wave's 32 x 32 block visible and in range?
      const bool full =
          __builtin_amdgcn_readfirstlane(wave_kmax <= q0 && wave_min_end > q0 + 31 && q0 >= lo && q0 + 31 < hi);
      // S starts at -LSE log2(e) and dP at -D (both per query = per register), so
      // that the products below give S - LSE log2(e) (log2 units) and dP - D directly
      f32x16 s, dp;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int ql = mt * 32 + 8 * i4 + 4 * hh;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&S.s0[ql]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&S.d0[ql]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * i4 + e] = l4[e];
          dp[4 * i4 + e] = d4[e];
        }
      }
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        s = mfma(lds_read16(&S.Q[soff(mt * 32 + r, dc * 16 + 8 * hh)]), kf[dc], s);
        dp = mfma(lds_read16(&S.O[soff(mt * 32 + r, dc * 16 + 8 * hh)]), lds_read16(Vt + dc * 16), dp);
      }
      // schedule: the start values and the first two steps' operands, then
      // each step's two products followed by the reads two steps ahead (the
      // compiler's own order reads one step ahead and waits before almost
      // every product; measured 1.1-1.8% on the backward launch)
      __builtin_amdgcn_sched_group_barrier(0x100, 14, 0);
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      f32x16 ds;
      // the softmax step runs at raised wave priority: the SIMD's other wave,
      // usually issuing MFMAs, yields issue slots to it, which shortens the gap
      // before this wave's own dV/dK products
      __builtin_amdgcn_s_setprio(1);
      // PARTIAL blocks: invisible pairs get S = -inf in place (exp2 gives 0),
      // so both kinds of block share one exponential step and the branch
      // leaves no values to merge
      if (!full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = qt * QT + mt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool vis = (j <= qq) & (qq < endj) & (qq >= lo) & (qq < hi);
          s[i] = vis ? s[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_fast(s[i]);
        s[i] = p;
        ds[i] = p * dp[i];
      }
      const bf16x8 p0 = c_to_b(s, 0), p1 = c_to_b(s, 1);
      const bf16x8 s0 = c_to_b(ds, 0), s1 = c_to_b(ds, 1);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        dv[dt] = mfma(tr_frag_swz(S.O, mt * 32, dt * 32, lane), p0, dv[dt]);
        dv[dt] = mfma(tr_frag_swz(S.O, mt * 32 + 16, dt * 32, lane), p1, dv[dt]);
        dk[dt] = mfma(tr_frag_swz(S.Q, mt * 32, dt * 32, lane), s0, dk[dt]);
        dk[dt] = mfma(tr_frag_swz(S.Q, mt * 32 + 16, dt * 32, lane), s1, dk[dt]);
      }
    }
    if (step + 1 < n_steps) store_rows(L.st[sidx ^ 1]);
    wait_vmem();  // this wave's direct-to-LDS loads of the next tile have landed
    __syncthreads();
  }
  if constexpr (ACC) {
    // Accumulating (chunk) calls: each wave passes its 32 keys' dK (rotated
    // back) and dV through its own part of the LDS, which is free after the
    // loop's last barrier, so that the read-add-write of the fp32 accumulators
    // goes by whole rows (32 lanes cover a key's 128 values in 16-byte pieces)
    // instead of each lane reading and writing its own key's row 16 bytes at
    // a time.
    float* E = reinterpret_cast<float*>(&L) + wave * (32 * EST);
    const auto put_rows = [&](TG* __restrict__ out) {
      // two passes of 8 pieces per lane: all loads of a pass are in flight together
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 x[8];
        int64_t o[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int f = (8 * h + u) * 64 + lane, jj = kbase + wave * 32 + (f >> 5);
          x[u] = *reinterpret_cast<const float4*>(&E[(f >> 5) * EST + (f & 31) * 4]);
          ok[u] = jj < g.n_k;
          o[u] = (int64_t(ok[u] ? jj : 0) * g.h_kv + kvh) * D + (f & 31) * 4;
        }
        float4 y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[u]) y[u] = *reinterpret_cast<const float4*>(out + o[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (ok[u])
            *reinterpret_cast<float4*>(out + o[u]) =
                make_float4(y[u].x + x[u].x, y[u].y + x[u].y, y[u].z + x[u].z, y[u].w + x[u].w);
      }
    };

    // dK = R^T (scale * dK') at the key's depth, with (cos, sin) of depth *
    // theta_c from the caller's table (none: no rotation); coordinates (c, c+64)
    // are the same register of blocks dt and dt+2.  The Q operand carried
    // scale * log2(e), so scale * dK' is the accumulator times ln 2.
    const float2* __restrict__ cs_row = cs_tab && jok ? cs_tab + int64_t(P.depth[j]) * (D / 2) : nullptr;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float lo4[4], hi4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = dt * 32 + 8 * i4 + 4 * hh + e;
          const float x1 = dk[dt][4 * i4 + e] * kLn2, x2 = dk[dt + 2][4 * i4 + e] * kLn2;
          float cs = 1.f, sn = 0.f;
          if (cs_row) {
            const float2 t = cs_row[c];
            cs = t.x;
            sn = t.y;
          }
          lo4[e] = x1 * cs + x2 * sn;
          hi4[e] = x2 * cs - x1 * sn;
        }
        const int c0 = dt * 32 + 8 * i4 + 4 * hh;
        *reinterpret_cast<float4*>(&E[r * EST + c0]) = make_float4(lo4[0], lo4[1], lo4[2], lo4[3]);
        *reinterpret_cast<float4*>(&E[r * EST + c0 + 64]) = make_float4(hi4[0], hi4[1], hi4[2], hi4[3]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    put_rows(d_k);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(&E[r * EST + dt * 32 + 8 * i4 + 4 * hh]) =
            make_float4(dv[dt][4 * i4], dv[dt][4 * i4 + 1], dv[dt][4 * i4 + 2], dv[dt][4 * i4 + 3]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    put_rows(d_v);
  } else {
    // whole-tree calls: bf16 stores straight from the accumulators (staging
    // them through LDS measured 0.6% slower here: the extra code spills)
    if (!jok) return;

    // dK = R^T (scale * dK') at the key's depth, with (cos, sin) of depth *
    // theta_c from the caller's table (none: no rotation); coordinates (c, c+64)
    // are the same register of blocks dt and dt+2.  The Q operand carried
    // scale * log2(e), so scale * dK' is the accumulator times ln 2.
    const float2* __restrict__ cs_row = cs_tab ? cs_tab + int64_t(P.depth[j]) * (D / 2) : nullptr;
    const int64_t base = (int64_t(j) * g.h_kv + kvh) * D;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float lo4[4], hi4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = dt * 32 + 8 * i4 + 4 * hh + e;
          const float x1 = dk[dt][4 * i4 + e] * kLn2, x2 = dk[dt + 2][4 * i4 + e] * kLn2;
          float cs = 1.f, sn = 0.f;
          if (cs_row) {
            const float2 t = cs_row[c];
            cs = t.x;
            sn = t.y;
          }
          lo4[e] = x1 * cs + x2 * sn;
          hi4[e] = x2 * cs - x1 * sn;
        }
        const int c0 = dt * 32 + 8 * i4 + 4 * hh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Elem<TG>::store(d_k, base + c0 + e, lo4[e]);
          Elem<TG>::store(d_k, base + c0 + 64 + e, hi4[e]);
        }
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = dt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        Elem<TG>::store(d_v, base + c, dv[dt][i]);
      }
  }
}

// two waves per SIMD, except at G = 1, where the LDS stages of 2-wave
// workgroups hold one
template <int G, bool FIN, bool WIDE>
__global__ __launch_bounds__(DqCfg<G>::THREADS, G >= 2 ? 2 : 1) void dq_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dq_out, const float2* __restrict__ cs_tab, PlanPtrs P,
    AttnGeom g, int full_range, int qb_first, int n_qb, int nsub) {
  __shared__ DqStage st[2];
  dq_body<G, FIN, WIDE>(st, blockIdx.x, q, k, v, d_o, lse, Dv, dq_acc, dq_out, cs_tab, P, g, full_range, qb_first,
                        n_qb, nsub);
}

template <int G, bool ACC, typename TG, bool WIDE>
__global__ __launch_bounds__(KV_THREADS, 2) void dkdv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ Dv,
    TG* __restrict__ d_k, TG* __restrict__ d_v, const float2* __restrict__ cs_tab, PlanPtrs P, AttnGeom g) {
  __shared__ KvLds L;
  dkdv_body<G, ACC, TG, WIDE>(L, blockIdx.x, q, k, v, d_o, lse, Dv, d_k, d_v, cs_tab, P, g);
}

// dQ and dK/dV in one launch, for one backward call or several independent
// ones (each with its own query rows, dQ output and dK/dV accumulators; they
// share K, V and the plan).  The grid is a list of segments, each the dQ or
// the dK/dV workgroups of one call, ordered so that the segments with the
// longest workgroups go first (dK/dV in tree mode, where a shared root's keys
// walk every query; dQ for a short chunk of queries against a long prefix);
// the rest fill the CUs the first leave idle.  Every workgroup has 8 waves
// (four query heads per dQ workgroup: one kv head's group of 4, or two kv
// heads' groups of 2); the two kinds share one LDS allocation.
// GK: the dK/dV body's group size (0: a multiple of 4 read at run time).
template <int GK>
struct DqOf {
  static constexpr int G = GK == 2 ? 2 : 4;    // query heads per kv head in a dQ workgroup
  static constexpr int KVP = GK == 2 ? 2 : 1;  // kv heads per dQ workgroup
};
static_assert(sizeof(KvLds) >= 2 * 2 * sizeof(DqStage), "the dK/dV workgroups' LDS holds the dQ stages");
static_assert(DqCfg<4>::THREADS == KV_THREADS && 2 * DqCfg<2>::THREADS == KV_THREADS,
              "the combined launch needs equal workgroup sizes");

struct BwdCall {
  const uint16_t* q;
  const uint16_t* d_o;
  const float* lse;
  const float* Dv;
  float* dq_acc;
  uint16_t* dq_out;
  void* d_k;
  void* d_v;
  AttnGeom g;
  int32_t qb_first, n_qb;
};
struct BwdGrid {
  BwdCall c[kMaxBwdCalls];
  int32_t b0[2 * kMaxBwdCalls + 1];  // segment s holds workgroups [b0[s], b0[s + 1])
  int32_t what[2 * kMaxBwdCalls];    // 2 * call + (1: dK/dV, 0: dQ)
  int32_t n_seg;
};

// One call: the segment order reduces to which kind goes first.
template <int GK, bool ACC, typename TG, bool WQ, bool FIN, bool WKV>
__global__ __launch_bounds__(KV_THREADS, 2) void bwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_o, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dq_out, TG* __restrict__ d_k, TG* __restrict__ d_v,
    const float2* __restrict__ cs_tab, PlanPtrs P, AttnGeom g, int full_range, int qb_first, int n_qb, int nsub,
    int n_kv, int n_dq, int dq_first) {
  __shared__ __align__(16) unsigned char smem[sizeof(KvLds)];
  const int b = blockIdx.x;
  const bool kv = dq_first ? b >= n_dq : b < n_kv;
  if (kv)
    dkdv_body<GK, ACC, TG, WQ>(*reinterpret_cast<KvLds*>(smem), dq_first ? b - n_dq : b, q, k, v, d_o, lse, Dv,
                               d_k, d_v, cs_tab, P, g);
  else
    dq_body<DqOf<GK>::G, FIN, WKV, DqOf<GK>::KVP>(reinterpret_cast<DqStage*>(smem), dq_first ? b : b - n_kv, q, k,
                                                  v, d_o, lse, Dv, dq_acc, dq_out, cs_tab, P, g, full_range,
                                                  qb_first, n_qb, nsub);
}

// Several calls (a separate kernel: the per-call selection costs the
// one-call case registers and about 1% of its time).
template <int GK, bool ACC, typename TG, bool WQ, bool FIN, bool WKV>
__global__ __launch_bounds__(KV_THREADS, 2) void bwd_multi_mfma_kernel(const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 const float2* __restrict__ cs_tab, PlanPtrs P,
                                                                 int full_range, int nsub, BwdGrid G) {
  __shared__ __align__(16) unsigned char smem[sizeof(KvLds)];
  const int b = blockIdx.x;
  int s = 0;
  for (int i = 1; i < G.n_seg; ++i) s += b >= G.b0[i] ? 1 : 0;
  const BwdCall& c = G.c[G.what[s] >> 1];
  const int lb = b - G.b0[s];
  if (G.what[s] & 1)
    dkdv_body<GK, ACC, TG, WQ>(*reinterpret_cast<KvLds*>(smem), lb, c.q, k, v, c.d_o, c.lse, c.Dv,
                               static_cast<TG*>(c.d_k), static_cast<TG*>(c.d_v), cs_tab, P, c.g);
  else
    dq_body<DqOf<GK>::G, FIN, WKV, DqOf<GK>::KVP>(reinterpret_cast<DqStage*>(smem), lb, c.q, k, v, c.d_o, c.lse,
                                                  c.Dv, c.dq_acc, c.dq_out, cs_tab, P, c.g, full_range, c.qb_first,
                                                  c.n_qb, nsub);
}

template <int G>
int launch_dq_g(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D_,
                float* dq_acc, void* dq_out, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                bool full_range, hipStream_t st) {
  const int qb_first = g.q_off / BQ;
  const int qb_end = (g.q_off + g.n_q + BQ - 1) / BQ;
  const int n_qb = qb_end - qb_first;
  if (n_qb <= 0) return 0;
  const int nsub = (g.h_q / g.h_kv) / G;
  const dim3 grid(unsigned(n_qb) * unsigned(g.h_kv) * unsigned(nsub)), block(DqCfg<G>::THREADS);
  const bool wide = int64_t(g.n_k) * g.h_kv * D * 2 >= (int64_t(1) << 31);
#define TT_DQ(FIN, WIDE)                                                                                          \
  dq_mfma_kernel<G, FIN, WIDE><<<grid, block, 0, st>>>(                                                           \
      (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o, lse, D_,                  \
      FIN ? nullptr : dq_acc, FIN ? (uint16_t*)dq_out : nullptr, FIN ? cs_tab : nullptr, P, g, full_range ? 1 : 0, \
      qb_first, n_qb, nsub)
  if (dq_out) {
    if (wide) TT_DQ(true, true); else TT_DQ(true, false);
  } else {
    if (wide) TT_DQ(false, true); else TT_DQ(false, false);
  }
#undef TT_DQ
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int G>
int launch_dkdv_g(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D_,
                  void* d_k, void* d_v, bool acc, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                  hipStream_t st) {
  const int nkb2 = (g.n_k + KV_KEYS - 1) / KV_KEYS;
  if (nkb2 <= 0) return 0;
  const dim3 grid(unsigned(nkb2) * unsigned(g.h_kv)), block(KV_THREADS);
  const bool wide = int64_t(g.n_q) * g.h_q * D * 2 >= (int64_t(1) << 31);
#define TT_KV(ACC, TG, WIDE)                                                                                    \
  dkdv_mfma_kernel<G, ACC, TG, WIDE><<<grid, block, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,             \
                                                             (const uint16_t*)v, (const uint16_t*)d_o, lse, D_, \
                                                             (TG*)d_k, (TG*)d_v, cs_tab, P, g)
  if (acc) {
    if (wide) TT_KV(true, float, true); else TT_KV(true, float, false);
  } else {
    if (wide) TT_KV(false, uint16_t, true); else TT_KV(false, uint16_t, false);
  }
#undef TT_KV
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int GK, bool ACC, typename TG, bool FIN>
int launch_bwd_g(const BwdCallPtrs* calls, int n_calls, const void* k, const void* v, const float2* cs_tab,
                 const PlanPtrs& P, bool full_range, bool wide, hipStream_t st) {
  BwdGrid G{};
  struct Seg {
    int64_t len;  // longest workgroup of the segment, in MFMAs per wave / 16
    int32_t what, count;
  } seg[2 * kMaxBwdCalls];
  int ns = 0;
  // dQ workgroups: one per q-block and kv head (groups of a multiple of 4
  // heads, nsub per kv head) or per q-block and pair of kv heads (groups of 2)
  constexpr int KVP = DqOf<GK>::KVP;
  const int nsub = (calls[0].g.h_q / calls[0].g.h_kv) / DqOf<GK>::G;
  for (int i = 0; i < n_calls; ++i) {
    const AttnGeom& g = calls[i].g;
    BwdCall& c = G.c[i];
    c.q = static_cast<const uint16_t*>(calls[i].q);
    c.d_o = static_cast<const uint16_t*>(calls[i].d_o);
    c.lse = calls[i].lse;
    c.Dv = calls[i].D;
    c.dq_acc = FIN ? nullptr : calls[i].dq_acc;
    c.dq_out = FIN ? static_cast<uint16_t*>(calls[i].dq_out) : nullptr;
    c.d_k = calls[i].d_k;
    c.d_v = calls[i].d_v;
    c.g = g;
    c.qb_first = g.q_off / BQ;
    c.n_qb = (g.q_off + g.n_q + BQ - 1) / BQ - c.qb_first;
    const int n_kv = (g.n_k + KV_KEYS - 1) / KV_KEYS * g.h_kv;
    const int n_dq = c.n_qb > 0 ? c.n_qb * (g.h_kv / KVP) * nsub : 0;
    // a dK/dV workgroup walks up to n_q query rows x the group's heads (64
    // MFMAs per wave per 64 rows and head), a dQ one up to n_k keys (48 MFMAs
    // per wave per 64 keys); dK/dV is listed first, so it leads on a tie
    if (n_kv > 0) seg[ns++] = {4 * int64_t(g.n_q) * (g.h_q / g.h_kv), 2 * i + 1, n_kv};
    if (n_dq > 0) seg[ns++] = {3 * int64_t(g.n_k), 2 * i, n_dq};
  }
  std::stable_sort(seg, seg + ns, [](const Seg& x, const Seg& y) { return x.len > y.len; });
  int64_t nb = 0;
  for (int s = 0; s < ns; ++s) {
    G.b0[s] = int32_t(nb);
    G.what[s] = seg[s].what;
    nb += seg[s].count;
  }
  G.b0[ns] = int32_t(nb);
  G.n_seg = ns;
  if (nb <= 0) return 0;
  if (nb >= (int64_t(1) << 31)) return -1;
  const dim3 grid(static_cast<unsigned>(nb)), block(KV_THREADS);
  if (n_calls == 1) {
    const BwdCall& c = G.c[0];
    const int n_kv = (c.g.n_k + KV_KEYS - 1) / KV_KEYS * c.g.h_kv;
    const int n_dq = int(nb) - n_kv, dq_first = ns > 0 && (G.what[0] & 1) == 0 ? 1 : 0;
#define TT_BWD(WIDE)                                                                                          \
  bwd_mfma_kernel<GK, ACC, TG, WIDE, FIN, WIDE><<<grid, block, 0, st>>>(                                      \
      c.q, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), c.d_o, c.lse, c.Dv, c.dq_acc,     \
      c.dq_out, static_cast<TG*>(c.d_k), static_cast<TG*>(c.d_v), cs_tab, P, c.g, full_range ? 1 : 0,          \
      c.qb_first, c.n_qb, nsub, n_kv, n_dq, dq_first)
    if (wide)
      TT_BWD(true);
    else
      TT_BWD(false);
#undef TT_BWD
  } else {
#define TT_BWD(WIDE)                                                                          \
  bwd_multi_mfma_kernel<GK, ACC, TG, WIDE, FIN, WIDE><<<grid, block, 0, st>>>(                \
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), cs_tab, P, full_range ? 1 : 0, nsub, G)
    if (wide)
      TT_BWD(true);
    else
      TT_BWD(false);
#undef TT_BWD
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_bwd_mfma_multi(const BwdCallPtrs* calls, int n_calls, const void* k, const void* v, bool acc,
                          const float2* cs_tab, const PlanPtrs& P, bool full_range, hipStream_t st) {
  if (n_calls < 1 || n_calls > kMaxBwdCalls) return -1;
  const AttnGeom& g0 = calls[0].g;
  const int G = g0.h_q / g0.h_kv;
  // the dQ workgroups of other groups have fewer waves than the dK/dV ones
  if (!bwd_combined_supported(g0.h_q, g0.h_kv)) return -2;
  const bool fin = calls[0].dq_out != nullptr;
  if (!acc && !fin) return -2;
  bool wide = false;
  for (int i = 0; i < n_calls; ++i) {
    const AttnGeom& g = calls[i].g;
    if (g.h_q != g0.h_q || g.h_kv != g0.h_kv || g.d != g0.d || (calls[i].dq_out != nullptr) != fin) return -1;
    wide = wide || int64_t(g.n_k) * g.h_kv * D * 2 >= (int64_t(1) << 31) ||
           int64_t(g.n_q) * g.h_q * D * 2 >= (int64_t(1) << 31);
  }
#define TT_B(GK, ACC, TG, FIN) launch_bwd_g<GK, ACC, TG, FIN>(calls, n_calls, k, v, cs_tab, P, full_range, wide, st)
  if (G == 2) {
    if (!acc) return TT_B(2, false, uint16_t, true);
    return fin ? TT_B(2, true, float, true) : TT_B(2, true, float, false);
  }
  if (G == 4) {
    if (!acc) return TT_B(4, false, uint16_t, true);
    return fin ? TT_B(4, true, float, true) : TT_B(4, true, float, false);
  }
  if (!acc) return TT_B(0, false, uint16_t, true);
  return fin ? TT_B(0, true, float, true) : TT_B(0, true, float, false);
#undef TT_B
}

int launch_bwd_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D_,
                    float* dq_acc, void* dq_out, void* d_k, void* d_v, bool acc, const float2* cs_tab,
                    const PlanPtrs& P, const AttnGeom& g, bool full_range, hipStream_t st) {
  const BwdCallPtrs c{q, d_o, lse, D_, dq_acc, dq_out, d_k, d_v, g};
  return launch_bwd_mfma_multi(&c, 1, k, v, acc, cs_tab, P, full_range, st);
}

bool mfma_bwd_supported(const AttnGeom& g, const PlanPtrs& P) {
  return g.d == D && P.bq == BQ && P.bk == BK && g.h_kv > 0 && g.h_q % g.h_kv == 0;
}

int launch_dq_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D_,
                   float* dq_acc, void* dq_out, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                   bool full_range, hipStream_t st) {
  switch (group_split(g.h_q / g.h_kv)) {
    case 1: return launch_dq_g<1>(q, k, v, d_o, lse, D_, dq_acc, dq_out, cs_tab, P, g, full_range, st);
    case 2: return launch_dq_g<2>(q, k, v, d_o, lse, D_, dq_acc, dq_out, cs_tab, P, g, full_range, st);
    case 4: return launch_dq_g<4>(q, k, v, d_o, lse, D_, dq_acc, dq_out, cs_tab, P, g, full_range, st);
    default: return -1;
  }
}

int launch_dkdv_mfma(const void* q, const void* k, const void* v, const void* d_o, const float* lse, const float* D_,
                     void* d_k, void* d_v, bool acc, const float2* cs_tab, const PlanPtrs& P, const AttnGeom& g,
                     hipStream_t st) {
  switch (g.h_q / g.h_kv) {
    case 1: return launch_dkdv_g<1>(q, k, v, d_o, lse, D_, d_k, d_v, acc, cs_tab, P, g, st);
    case 2: return launch_dkdv_g<2>(q, k, v, d_o, lse, D_, d_k, d_v, acc, cs_tab, P, g, st);
    case 4: return launch_dkdv_g<4>(q, k, v, d_o, lse, D_, d_k, d_v, acc, cs_tab, P, g, st);
    case 8: return launch_dkdv_g<8>(q, k, v, d_o, lse, D_, d_k, d_v, acc, cs_tab, P, g, st);
    default: return launch_dkdv_g<0>(q, k, v, d_o, lse, D_, d_k, d_v, acc, cs_tab, P, g, st);
  }
}
