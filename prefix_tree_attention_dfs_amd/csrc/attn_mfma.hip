// bf16 MFMA tree attention forward, head dim 128 (gfx950).
//
// Tree Training (arXiv 2511.00413), Abstract: each unique token is computed
// once and must get exactly its per-branch result; row i attends to row j iff
// j <= i < end[j] (j is i or an ancestor of i in DFS order).
//
// One workgroup = one 64-row query block x G query heads of one key/value
// head's group (GQA; a group of more than 4 heads is split over several
// workgroups, nsub per block, which read the same K/V tiles).  It walks the block's list of
// non-empty 64-key tiles (the plan's CSR); FULL tiles skip the mask.  K and V
// tiles go from global memory straight into LDS (swizzled layout), double
// buffered, one barrier per tile.  Per wave: NT sub-tiles of 32 query rows of one head, Q held in
// registers as B operands.
//   S^T  = K Q^T        (A = K rows from LDS, B = Q; Q carries scale * log2(e),
//                        so scores are in log2 units, and the accumulators
//                        start at minus the running max: no per-score FMA)
//   online softmax over keys (columns are lanes: row statistics are per lane;
//                        no per-tile max unless a row's sum says it grew)
//   O^T += V^T P^T      (A = V^T via ds_read_tr16_b64, B = P^T straight from
//                        the S^T accumulator registers)
// With PRO the kernel makes the query operand itself: it reads the caller's
// Q, rotates each row at its depth from the (cos, sin) table, multiplies by
// scale * log2(e), rounds to bf16 (rot_pair_bf16, the RoPE kernel's
// arithmetic) and stores that copy for the backward, so no separate pass
// over Q runs before the forward.
#include "device.h"
#include "kernels.h"
#include "mfma_common.h"

using namespace ttm;

namespace {

template <int G>
struct FwdCfg {
  static constexpr int NT = 1;                          // 32-row query sub-tiles per wave
  static constexpr int WAVES = (G * BQ) / (32 * NT);     // waves per workgroup
  static constexpr int THREADS = WAVES * 64;
  static constexpr int CH = (BK * D / 8) / THREADS;      // 16-byte chunks per thread per K (or V) tile
  static constexpr int WPH = 2 / NT;                     // waves per head
  // waves per SIMD the register budget is set for: two, except at G = 1, where
  // the LDS (two 33 KB stages per 2-wave workgroup) holds one wave per SIMD
  static constexpr int MINB = G >= 2 ? 2 : 1;
};

struct __align__(16) FwdStage {
  uint16_t K[BK * D];  // swizzled (soff): row reads for S^T
  uint16_t V[BK * D];  // swizzled: transposed reads for O^T
  int32_t end[BK];
};

// WIDE: K/V of 2 GiB or more; each tile's descriptors then start at the tile
// (64-bit base) instead of one descriptor with a 32-bit tile offset.
template <int G, bool WIDE, bool PRO>
__global__ __launch_bounds__(FwdCfg<G>::THREADS, FwdCfg<G>::MINB) void fwd_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, PlanPtrs P, AttnGeom g, int full_range, int qb_first,
    int n_qb, int nsub, uint16_t* __restrict__ q_out, const float2* __restrict__ qtab, float qmul) {
  using C = FwdCfg<G>;
  constexpr int NT = C::NT;
  __shared__ FwdStage st[2];
  if (!plan_matches(P)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, hh = lane >> 5;
  const int kvh = blockIdx.x % g.h_kv;
  const int rest = blockIdx.x / g.h_kv;
  const int sub = rest % nsub, idx = rest / nsub;
  const int qb = full_range ? ld_uniform(P.qb_order, idx) : (qb_first + n_qb - 1 - idx);
  const int head = (kvh * nsub + sub) * G + wave / C::WPH;
  const int pos0 = (wave % C::WPH) * 32 * NT;
  const int qrow0 = qb * BQ - g.q_off;  // q-buffer row of the block's first position
  // the exponentials run against the running max (log2 units) without a tile
  // max: a lane's 16 values of each 32-key half are accepted while their sum
  // is at most tsum (so every p <= 2^8, which the fp32 sums and the bf16 P
  // operand carry without loss of relative precision); otherwise, and for a
  // row with no max yet, the tile is redone with the max moved to the exact
  // running max.  Any max gives the same softmax: O and l share it, and the
  // LSE adds it back.
  constexpr float tsum = 256.f;

  // Q fragments (B operands): lane holds Q[row][dc*16 + 8hh .. +8]
  bf16x8 qf[NT][8];
  int32_t qdep[NT];  // PRO: the rows' depths (table rows)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = qrow0 + pos0 + nt * 32 + r;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[nt][dc] = row < g.n_q ? ld16(q + (int64_t(row) * g.h_q + head) * D + dc * 16 + 8 * hh) : zero8();
    if constexpr (PRO) qdep[nt] = row < g.n_q ? P.depth[g.q_off + row] : 0;
  }

  f32x16 oacc[NT][4];
  float m[NT], lpart[NT];  // running max (log2 units, -inf before any visible key), partial row sum
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lpart[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[nt][dt] = zero16();
  }

  // tile staging: buffer loads, zero past n_k keys (end = 0 there: invisible)
  const int64_t kv_elems = int64_t(g.n_k) * g.h_kv * D;
  const int64_t tile_elems = int64_t(BK) * g.h_kv * D;  // one 64-key tile of K (or V)
  const rsrc_t re = make_rsrc(P.end, uint32_t(g.n_k) * 4);
  const rsrc_t rk0 = make_rsrc(k, WIDE ? 0u : uint32_t(kv_elems * 2)), rv0 = make_rsrc(v, WIDE ? 0u : uint32_t(kv_elems * 2));
  // K and V tiles (64 keys x 128 bf16 = 16 KB each) go from global memory
  // straight into LDS: 16 loads of 1 KB per tile, NL per wave.  Lane l of
  // load j fills LDS slot 64 j + l = (key, stored chunk) = ((64 j + l) / 16,
  // (64 j + l) % 16) and fetches global chunk (stored chunk ^ swz(key)), so
  // the tile lands in the swizzled layout.
  constexpr int NL = (BK * D * 2 / 1024) / C::WAVES;  // 1 KB loads per wave per tile
  static_assert(NL * C::WAVES * 1024 == BK * D * 2, "the waves' 1 KB loads cover a tile");
  uint32_t dvoff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (wave * NL + i) * 64 + lane;
    const int key = p >> 4, c = (p & 15) ^ swz(p >> 4);
    dvoff[i] = (uint32_t(key * g.h_kv + kvh) * D + c * 8) * 2;
  }
  int32_t ereg = 0;
  auto load_tile = [&](int kb, FwdStage& s) {
    const uint32_t kbase = lds_u32(s.K) + wave * NL * 1024, vbase = lds_u32(s.V) + wave * NL * 1024;
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
  auto store_end = [&](FwdStage& s) {
    if (tid < BK) s.end[tid] = ereg;
  };

  // tile-list entries run two ahead of the tile being computed: cur is the
  // next tile's (prefetched this iteration), nxt the one after
  const int e0 = ld_uniform(P.qb_ptr, qb), e1 = ld_uniform(P.qb_ptr, qb + 1);
  int cur = e0 < e1 ? ld_uniform(P.qb_tiles, e0) : 0;
  int nxt = e0 + 1 < e1 ? ld_uniform(P.qb_tiles, e0 + 1) : 0;
  if (e0 < e1) load_tile(cur & kKbMask, st[0]);
  if constexpr (PRO) {
    // make the query operand while the first tile is in flight (stored to
    // q_out in the epilogue): the pair (c, c + 64) of coordinate
    // c = dc*16 + 8hh + e sits in this lane's qf[dc] and qf[dc + 4]; the
    // table row holds pairs 0..63
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int row = qrow0 + pos0 + nt * 32 + r;
      if (row >= g.n_q) continue;
      // all table loads in flight together, then the rotations
      float4 cs[4][4];  // cs[dc][i]: (cos, sin) of pairs dc*16 + 8hh + 2i, + 2i + 1
      if (qtab) {
        const float4* t = reinterpret_cast<const float4*>(qtab + int64_t(qdep[nt]) * (D / 2) + 8 * hh);
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[dc][i] = t[dc * 8 + i];
      } else {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
#pragma unroll
          for (int i = 0; i < 4; ++i) cs[dc][i] = make_float4(1.f, 0.f, 1.f, 0.f);
      }
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        uint16_t y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float4 c4 = cs[dc][e >> 1];
          const float c = (e & 1) ? c4.z : c4.x, sn = (e & 1) ? c4.w : c4.y;
          ttd::rot_pair_bf16(float(qf[nt][dc][e]), float(qf[nt][dc + 4][e]), c * qmul, sn * qmul, y1[e], y2[e]);
        }
        qf[nt][dc] = __builtin_bit_cast(bf16x8, y1);
        qf[nt][dc + 4] = __builtin_bit_cast(bf16x8, y2);
      }
    }
  }
  if (e0 < e1) store_end(st[0]);
  wait_vmem();  // also the direct-to-LDS loads, which the compiler does not track
  __syncthreads();

  for (int e = e0; e < e1; ++e) {
    const int sidx = (e - e0) & 1;
    const int ent = cur;
    const int kb = ent & kKbMask;
    const bool full = (ent & kFull) != 0;
    // the next tile's loads, without a branch: on the block's last tile cur is
    // that tile again (the list entry two ahead is clamped to the last one;
    // tile 0 for a one-tile block), so the spare stage receives a copy nobody
    // reads, and the wait before the barrier below still covers it (a uniform
    // branch here cost 0.6%)
    cur = nxt;
    nxt = ld_uniform(P.qb_tiles, min(e + 2, e1 - 1));
    load_tile(cur & kKbMask, st[sidx ^ 1]);  // that stage was last read in the previous tile
    const FwdStage& S = st[sidx];

    // S^T = K Q^T - m for both 32-key halves (scores in log2 units relative to
    // the running max), mask, exponentials of both halves against the running
    // max, one vote for the rare case above (a row without a max yet, or a
    // lane's half whose sum exceeds tsum), then O^T += V^T P^T.
    f32x16 sv[2][NT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float neg = m[nt] == -INFINITY ? 0.f : -m[nt];
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[kt][nt][i] = neg;
      }
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const bf16x8 a = lds_read16(&S.K[soff(kt * 32 + r, dc * 16 + 8 * hh)]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sv[kt][nt] = mfma(a, qf[nt][dc], sv[kt][nt]);
      }
    }
    auto mask_half = [&](int kt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int qpos = qb * BQ + pos0 + nt * 32 + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kt * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool vis = (kb * BK + kl <= qpos) & (qpos < S.end[kl]);
          sv[kt][nt][i] = vis ? sv[kt][nt][i] : -INFINITY;
        }
      }
    };
    if (!full) {
      mask_half(0);
      mask_half(1);
    }
    bf16x8 pf[2][2][NT];
    float ls[2][NT];
    bool redo = false;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ls[kt][nt] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(sv[kt][nt][i]);
          sv[kt][nt][i] = p;
          ls[kt][nt] += p;
        }
        redo |= (m[nt] == -INFINITY) | !(ls[kt][nt] <= tsum);
      }
    if (__any(redo)) {
      // rare: raw scores of both halves again (the K tile is still staged),
      // the max moved to the exact running max (O and l rescaled), the
      // exponentials against it
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sv[kt][nt] = zero16();
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) {
          const bf16x8 a = lds_read16(&S.K[soff(kt * 32 + r, dc * 16 + 8 * hh)]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sv[kt][nt] = mfma(a, qf[nt][dc], sv[kt][nt]);
        }
        if (!full) mask_half(kt);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sv[kt][nt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = m[nt] == -INFINITY ? mx : fmaxf(m[nt], mx);
        if (m[nt] != -INFINITY && mn > m[nt]) {
          const float alpha = exp2_fast(m[nt] - mn);
          lpart[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[nt][dt][i] *= alpha;
        }
        m[nt] = mn;
        const float neg = mn == -INFINITY ? 0.f : -mn;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          ls[kt][nt] = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = exp2_fast(sv[kt][nt][i] + neg);
            sv[kt][nt][i] = p;
            ls[kt][nt] += p;
          }
        }
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        lpart[nt] += ls[kt][nt];
#pragma unroll
        for (int c = 0; c < 2; ++c) pf[kt][c][nt] = c_to_b(sv[kt][nt], c);
      }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bf16x8 a = tr_frag_swz(S.V, kt * 32 + 16 * c, dt * 32, lane);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) oacc[nt][dt] = mfma(a, pf[kt][c][nt], oacc[nt][dt]);
        }

    store_end(st[sidx ^ 1]);
    wait_vmem();  // this wave's direct-to-LDS loads of the next tile have landed
    __syncthreads();
  }

  // epilogue: O = O^T / l (lane = query row, registers = head-dim entries), LSE
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = lpart[nt] + __shfl_xor(lpart[nt], 32, 64);
    const int row = qrow0 + pos0 + nt * 32 + r;
    if (row >= g.n_q) continue;
    const float inv = 1.f / lt;
    uint16_t* orow = o + (int64_t(row) * g.h_q + head) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __bf16(oacc[nt][dt][4 * i4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * i4 + 4 * hh) = w;
      }
    // natural-log LSE from the log2-unit max: ln 2 (m + log2 sum 2^(s' - m))
    if (hh == 0) lse[int64_t(row) * g.h_q + head] = (m[nt] + __log2f(lt)) * 0.6931471805599453f;
    if constexpr (PRO) {
      uint16_t* dst = q_out + (int64_t(row) * g.h_q + head) * D + 8 * hh;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) *reinterpret_cast<bf16x8*>(dst + dc * 16) = qf[nt][dc];
    }
  }
}

template <int G>
int launch_fwd_g(const void* q, const void* k, const void* v, void* o, float* lse, const PlanPtrs& P,
                 const AttnGeom& g, bool full_range, hipStream_t st, const QRot* qr) {
  const int qb_first = g.q_off / BQ;
  const int qb_end = (g.q_off + g.n_q + BQ - 1) / BQ;
  const int n_qb = qb_end - qb_first;
  if (n_qb <= 0) return 0;
  const int nsub = (g.h_q / g.h_kv) / G;
  const dim3 grid(unsigned(n_qb) * unsigned(g.h_kv) * unsigned(nsub)), block(FwdCfg<G>::THREADS);
  const bool wide = int64_t(g.n_k) * g.h_kv * D * 2 >= (int64_t(1) << 31);
  uint16_t* q_out = qr ? static_cast<uint16_t*>(qr->out) : nullptr;
  const float2* qtab = qr ? qr->tab : nullptr;
  const float qmul = qr ? qr->mul : 1.f;
#define TT_FWD(WIDE, PRO)                                                                                    \
  fwd_mfma_kernel<G, WIDE, PRO><<<grid, block, 0, st>>>((const uint16_t*)q, (const uint16_t*)k,              \
                                                        (const uint16_t*)v, (uint16_t*)o, lse, P, g,         \
                                                        full_range ? 1 : 0, qb_first, n_qb, nsub, q_out, qtab, \
                                                        qmul)
  if (qr) {
    if (wide) TT_FWD(true, true); else TT_FWD(false, true);
  } else {
    if (wide) TT_FWD(true, false); else TT_FWD(false, false);
  }
#undef TT_FWD
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

bool mfma_attn_supported(const AttnGeom& g, const PlanPtrs& P) {
  return g.d == D && P.bq == BQ && P.bk == BK && g.h_kv > 0 && g.h_q % g.h_kv == 0;
}

int launch_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, const PlanPtrs& P,
                    const AttnGeom& g, bool full_range, hipStream_t st, const QRot* qr) {
  switch (group_split(g.h_q / g.h_kv)) {
    case 1: return launch_fwd_g<1>(q, k, v, o, lse, P, g, full_range, st, qr);
    case 2: return launch_fwd_g<2>(q, k, v, o, lse, P, g, full_range, st, qr);
    case 4: return launch_fwd_g<4>(q, k, v, o, lse, P, g, full_range, st, qr);
    default: return -1;
  }
}
