// Host-side prefix tree: trie insertion, lexicographic DFS serialization,
// per-row arrays, and the tile schedule of the tree attention.  No HIP calls.
//
// Tree Training (arXiv 2511.00413), Abstract: the tokens of a task form a tree
// with shared prefixes; DFS serialization visits each token once; each
// token's loss weight is the fraction of branches through it.
// AReaL-DTA (arXiv 2602.00482) summary, Key Contributions 3: rollouts are
// sorted into one prefix tree in lexicographic DFS order.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <new>

#include "internal.h"

namespace tt {
static thread_local std::string g_err;
int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
void clear_error() { g_err.clear(); }
const char* last_error() { return g_err.c_str(); }
}  // namespace tt

extern "C" const char* tt_last_error(void) { return tt::last_error(); }

namespace {

// Open-addressing map (parent node, token) -> child node.
class ChildMap {
 public:
  explicit ChildMap(size_t expect) {
    size_t cap = 16;
    while (cap < expect * 2 + 16) cap <<= 1;
    keys_.assign(cap, kEmpty);
    vals_.assign(cap, -1);
    mask_ = cap - 1;
  }
  // Returns the child id, inserting `fresh` if absent (then *inserted = true).
  int32_t find_or_insert(int32_t parent, int32_t tok, int32_t fresh, bool* inserted) {
    const uint64_t key = (uint64_t(uint32_t(parent + 1)) << 32) | uint32_t(tok);
    size_t h = mix(key) & mask_;
    while (true) {
      if (keys_[h] == key) {
        *inserted = false;
        return vals_[h];
      }
      if (keys_[h] == kEmpty) {
        keys_[h] = key;
        vals_[h] = fresh;
        *inserted = true;
        return fresh;
      }
      h = (h + 1) & mask_;
    }
  }

 private:
  static constexpr uint64_t kEmpty = ~uint64_t(0);
  static uint64_t mix(uint64_t x) {  // splitmix64 finalizer
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ULL;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebULL;
    x ^= x >> 31;
    return x;
  }
  std::vector<uint64_t> keys_;
  std::vector<int32_t> vals_;
  size_t mask_;
};

bool pow2_in(int32_t b, int32_t lo, int32_t hi) { return b >= lo && b <= hi && (b & (b - 1)) == 0; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Keys per workgroup of the matrix-core dK/dV kernel: the unit of the key
// launch order.
constexpr int32_t kKeyGroup = 256;

// Tile schedule (visibility j <= i < end[j]).  For a key block the rows that
// see some key in it form the contiguous range [first key, max end): each
// key j is seen by [j, end[j]) and consecutive keys' ranges touch.
void build_schedule(tt_tree* t) {
  const int32_t N = t->N, bq = t->bq, bk = t->bk;
  t->nqb = (N + bq - 1) / bq;
  t->nkb = (N + bk - 1) / bk;
  std::vector<int32_t> qlo(t->nkb), qhi(t->nkb), minend(t->nkb);
  for (int32_t kb = 0; kb < t->nkb; ++kb) {
    const int32_t j0 = kb * bk, j1 = std::min(N, j0 + bk);
    int32_t mx = 0, mn = std::numeric_limits<int32_t>::max();
    for (int32_t j = j0; j < j1; ++j) {
      mx = std::max(mx, t->end[j]);
      mn = std::min(mn, t->end[j]);
    }
    qlo[kb] = j0;
    qhi[kb] = mx;
    minend[kb] = mn;
  }
  // per-q-block tile lists, k-blocks ascending
  std::vector<int32_t> cnt(t->nqb + 1, 0);
  for (int32_t kb = 0; kb < t->nkb; ++kb)
    for (int32_t qb = qlo[kb] / bq; qb <= (qhi[kb] - 1) / bq; ++qb) cnt[qb + 1]++;
  for (int32_t qb = 0; qb < t->nqb; ++qb) cnt[qb + 1] += cnt[qb];
  const int64_t ntiles = cnt[t->nqb];
  std::vector<int32_t> tiles(ntiles), fill(cnt.begin(), cnt.end() - 1);
  int64_t nfull = 0;
  for (int32_t kb = 0; kb < t->nkb; ++kb) {
    const int32_t j0 = kb * bk, j1 = std::min(N, j0 + bk);
    const bool complete = (j1 - j0) == bk;
    for (int32_t qb = qlo[kb] / bq; qb <= (qhi[kb] - 1) / bq; ++qb) {
      const int32_t i0 = qb * bq, i1 = std::min(N, i0 + bq);
      const bool full = complete && (j1 - 1 <= i0) && (minend[kb] >= i1);
      nfull += full;
      tiles[fill[qb]++] = kb | (full ? ttp::kFullBit : 0);
    }
  }
  t->n_tiles = ntiles;
  t->n_full = nfull;
  // launch orders.  q-blocks from the last row up: the workgroups an XCD runs
  // together are then DFS neighbours, which read nearly the same ancestor K/V
  // tiles (one L2 fetch serves them all), and the root's blocks, whose tile
  // lists are the shortest, come last.  Measured against largest-first on the
  // 8B-shape tree: forward HBM reads 7.9 -> 3.3 GB, backward 37 -> 19 GB, both
  // kernels ~1.8% faster.  Key groups (kKeyGroup keys, the backward's dK/dV
  // workgroup) by the end of the rows that see them, latest first, ties in key
  // order: groups that run together then walk the same query tiles from the
  // same top row (a chain segment's keys share one end), and the shared
  // root's groups, whose walks are the longest, start first.
  std::vector<int32_t> qorder(t->nqb);
  for (int32_t i = 0; i < t->nqb; ++i) qorder[i] = t->nqb - 1 - i;
  const int32_t gb = std::max(1, kKeyGroup / bk), ng = (t->nkb + gb - 1) / gb;
  std::vector<int32_t> korder(ng), gend(ng, 0);
  for (int32_t kb = 0; kb < t->nkb; ++kb) gend[kb / gb] = std::max(gend[kb / gb], qhi[kb]);
  for (int32_t i = 0; i < ng; ++i) korder[i] = i;
  std::stable_sort(korder.begin(), korder.end(), [&](int32_t a, int32_t b) { return gend[a] > gend[b]; });

  // plan image
  int64_t w = ttp::H_WORDS;
  auto place = [&](int64_t n) {
    const int64_t at = w;
    w = round_up(w + std::max<int64_t>(n, 1), 64);
    return at;
  };
  const int64_t o_depth = place(N), o_end = place(N), o_qptr = place(t->nqb + 1),
                o_qtiles = place(ntiles), o_qorder = place(t->nqb), o_qlo = place(t->nkb),
                o_qhi = place(t->nkb), o_minend = place(t->nkb), o_korder = place(ng);
  t->plan.assign(size_t(w), 0);
  int32_t* p = t->plan.data();
  p[ttp::H_MAGIC] = ttp::kMagic;
  p[ttp::H_N] = N;
  p[ttp::H_BQ] = bq;
  p[ttp::H_BK] = bk;
  p[ttp::H_NQB] = t->nqb;
  p[ttp::H_NKB] = t->nkb;
  p[ttp::H_NTILES] = int32_t(ntiles);
  p[ttp::H_BYTES] = int32_t(w * 4);
  p[ttp::H_DEPTH] = int32_t(o_depth);
  p[ttp::H_END] = int32_t(o_end);
  p[ttp::H_QB_PTR] = int32_t(o_qptr);
  p[ttp::H_QB_TILES] = int32_t(o_qtiles);
  p[ttp::H_QB_ORDER] = int32_t(o_qorder);
  p[ttp::H_KB_QLO] = int32_t(o_qlo);
  p[ttp::H_KB_QHI] = int32_t(o_qhi);
  p[ttp::H_KB_MINEND] = int32_t(o_minend);
  p[ttp::H_KB_ORDER] = int32_t(o_korder);
  std::copy(t->depth.begin(), t->depth.end(), p + o_depth);
  std::copy(t->end.begin(), t->end.end(), p + o_end);
  std::copy(cnt.begin(), cnt.end(), p + o_qptr);
  std::copy(tiles.begin(), tiles.end(), p + o_qtiles);
  std::copy(qorder.begin(), qorder.end(), p + o_qorder);
  std::copy(qlo.begin(), qlo.end(), p + o_qlo);
  std::copy(qhi.begin(), qhi.end(), p + o_qhi);
  std::copy(minend.begin(), minend.end(), p + o_minend);
  std::copy(korder.begin(), korder.end(), p + o_korder);
  uint32_t h = 2166136261u;  // FNV-1a over every byte of the image
  for (const int32_t x : t->plan)
    for (int b = 0; b < 4; ++b) h = (h ^ ((uint32_t(x) >> (8 * b)) & 0xFFu)) * 16777619u;
  p[ttp::H_ID] = int32_t(h);
}

int build(const int32_t* tokens, const int64_t* offs, int32_t B, tt_tree* t) {
  const int64_t total = offs[B];
  t->B = B;
  t->seq_tokens = total;
  t->seq_off.assign(offs, offs + B + 1);
  // 1. trie insertion, nodes numbered in insertion order
  ChildMap map(static_cast<size_t>(total));
  std::vector<int32_t> ntok, npar, nterm;
  ntok.reserve(size_t(total));
  npar.reserve(size_t(total));
  std::vector<int32_t> pos_node(static_cast<size_t>(total));
  for (int32_t s = 0; s < B; ++s) {
    int32_t cur = -1;
    for (int64_t k = offs[s]; k < offs[s + 1]; ++k) {
      bool ins = false;
      const int32_t id = map.find_or_insert(cur, tokens[k], int32_t(ntok.size()), &ins);
      if (ins) {
        ntok.push_back(tokens[k]);
        npar.push_back(cur);
      }
      pos_node[size_t(k)] = id;
      cur = id;
    }
  }
  const int32_t N = int32_t(ntok.size());
  t->N = N;
  nterm.assign(size_t(N), 0);
  for (int32_t s = 0; s < B; ++s)
    if (offs[s + 1] > offs[s]) nterm[size_t(pos_node[size_t(offs[s + 1] - 1)])]++;

  // 2. children lists (CSR over node ids), sorted by token; roots likewise
  std::vector<int32_t> cptr(size_t(N) + 2, 0), clist(static_cast<size_t>(N));
  for (int32_t u = 0; u < N; ++u) cptr[size_t(npar[u] + 1) + 1]++;  // slot 0 = roots
  for (int32_t u = 0; u < N + 1; ++u) cptr[size_t(u) + 1] += cptr[size_t(u)];
  {
    std::vector<int32_t> f(cptr.begin(), cptr.end() - 1);
    for (int32_t u = 0; u < N; ++u) clist[size_t(f[size_t(npar[u] + 1)]++)] = u;
  }
  for (int32_t g = 0; g < N + 1; ++g)
    std::sort(clist.begin() + cptr[size_t(g)], clist.begin() + cptr[size_t(g) + 1],
              [&](int32_t a, int32_t b) { return ntok[size_t(a)] < ntok[size_t(b)]; });

  // 3. iterative preorder DFS (chains can be tens of thousands deep)
  std::vector<int32_t> dfs_of(static_cast<size_t>(N)), ndepth(static_cast<size_t>(N));
  std::vector<int32_t> stack;
  stack.reserve(size_t(N));
  for (int32_t c = cptr[1] - 1; c >= cptr[0]; --c) {
    stack.push_back(clist[size_t(c)]);
    ndepth[size_t(clist[size_t(c)])] = 0;
  }
  int32_t next = 0;
  while (!stack.empty()) {
    const int32_t u = stack.back();
    stack.pop_back();
    dfs_of[size_t(u)] = next++;
    const int32_t g = u + 1;
    for (int32_t c = cptr[size_t(g) + 1] - 1; c >= cptr[size_t(g)]; --c) {
      const int32_t v = clist[size_t(c)];
      ndepth[size_t(v)] = ndepth[size_t(u)] + 1;
      stack.push_back(v);
    }
  }

  // 4. per-row arrays in DFS order
  t->token.assign(size_t(N), 0);
  t->depth.assign(size_t(N), 0);
  t->parent.assign(size_t(N), -1);
  t->n_pass.assign(size_t(N), 0);
  for (int32_t u = 0; u < N; ++u) {
    const int32_t p = dfs_of[size_t(u)];
    t->token[size_t(p)] = ntok[size_t(u)];
    t->depth[size_t(p)] = ndepth[size_t(u)];
    t->parent[size_t(p)] = npar[size_t(u)] < 0 ? -1 : dfs_of[size_t(npar[size_t(u)])];
    t->n_pass[size_t(p)] = nterm[size_t(u)];
  }
  std::vector<int32_t> size(static_cast<size_t>(N), 1);
  for (int32_t i = N - 1; i >= 0; --i) {
    const int32_t p = t->parent[size_t(i)];
    if (p >= 0) {
      size[size_t(p)] += size[size_t(i)];
      t->n_pass[size_t(p)] += t->n_pass[size_t(i)];
    }
  }
  t->end.resize(size_t(N));
  t->weight.resize(size_t(N));
  const float fB = float(B);
  for (int32_t i = 0; i < N; ++i) {
    t->end[size_t(i)] = i + size[size_t(i)];
    t->weight[size_t(i)] = float(t->n_pass[size_t(i)]) / fB;  // exact operands, one rounding
  }
  t->seq_pos_to_dfs.resize(size_t(total));
  for (int64_t k = 0; k < total; ++k) t->seq_pos_to_dfs[size_t(k)] = dfs_of[size_t(pos_node[size_t(k)])];

  // 5. targets CSR (children of each row, ascending) and statistics
  t->tgt_row_ptr.assign(size_t(N) + 1, 0);
  for (int32_t i = 0; i < N; ++i)
    if (t->parent[size_t(i)] >= 0) t->tgt_row_ptr[size_t(t->parent[size_t(i)]) + 1]++;
  for (int32_t i = 0; i < N; ++i) t->tgt_row_ptr[size_t(i) + 1] += t->tgt_row_ptr[size_t(i)];
  t->tgt_dfs.resize(size_t(t->tgt_row_ptr[size_t(N)]));
  {
    std::vector<int32_t> f(t->tgt_row_ptr.begin(), t->tgt_row_ptr.end() - 1);
    for (int32_t i = 0; i < N; ++i)
      if (t->parent[size_t(i)] >= 0) t->tgt_dfs[size_t(f[size_t(t->parent[size_t(i)])]++)] = i;
  }
  t->n_roots = 0;
  t->n_leaves = 0;
  t->max_depth = -1;
  t->leaf_tokens = 0;
  t->pairs = 0;
  for (int32_t i = 0; i < N; ++i) {
    t->n_roots += t->parent[size_t(i)] < 0;
    const bool leaf = t->end[size_t(i)] == i + 1;
    t->n_leaves += leaf;
    t->max_depth = std::max(t->max_depth, t->depth[size_t(i)]);
    t->pairs += int64_t(t->depth[size_t(i)]) + 1;
    if (leaf) t->leaf_tokens += int64_t(t->depth[size_t(i)]) + 1;
  }
  t->dense_pairs = 0;
  for (int32_t s = 0; s < B; ++s) {
    const int64_t L = offs[s + 1] - offs[s];
    t->dense_pairs += L * (L + 1) / 2;
  }
  build_schedule(t);
  return TT_OK;
}

}  // namespace

extern "C" int tree_build(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                          int32_t block_q, int32_t block_k, tt_tree** out) {
  tt::clear_error();
  if (!out) return tt::fail(TT_EINVAL, "tree_build: out is NULL");
  *out = nullptr;
  if (n_seqs < 0) return tt::fail(TT_EINVAL, "tree_build: n_seqs < 0");
  if (n_seqs >= (1 << 24)) return tt::fail(TT_EOVERFLOW, "tree_build: n_seqs must be < 2^24");
  if (!seq_offsets) return tt::fail(TT_EINVAL, "tree_build: seq_offsets is NULL");
  if (block_q == 0) block_q = 64;
  if (block_k == 0) block_k = 64;
  if (!pow2_in(block_q, 16, 256) || !pow2_in(block_k, 16, 256))
    return tt::fail(TT_EINVAL, "tree_build: block sizes must be powers of two in [16, 256]");
  if (seq_offsets[0] != 0) return tt::fail(TT_EINVAL, "tree_build: seq_offsets[0] != 0");
  for (int32_t s = 0; s < n_seqs; ++s)
    if (seq_offsets[s + 1] < seq_offsets[s])
      return tt::fail(TT_EINVAL, "tree_build: seq_offsets must be non-decreasing");
  const int64_t total = seq_offsets[n_seqs];
  if (total > int64_t(std::numeric_limits<int32_t>::max()) - 1)
    return tt::fail(TT_EOVERFLOW, "tree_build: more than 2^31-2 tokens");
  if (total > 0 && !tokens) return tt::fail(TT_EINVAL, "tree_build: tokens is NULL");
  for (int64_t k = 0; k < total; ++k)
    if (tokens[k] < 0) return tt::fail(TT_EINVAL, "tree_build: negative token id");
  tt_tree* t = nullptr;
  try {
    t = new tt_tree();
    t->bq = block_q;
    t->bk = block_k;
    const int rc = build(tokens, seq_offsets, n_seqs, t);
    if (rc != TT_OK) {
      delete t;
      return rc;
    }
  } catch (const std::bad_alloc&) {
    delete t;
    return tt::fail(TT_ENOMEM, "tree_build: host allocation failed");
  }
  *out = t;
  return TT_OK;
}

extern "C" void tree_free(tt_tree* tree) { delete tree; }

extern "C" int tree_info(const tt_tree* t, tt_tree_info* o) {
  tt::clear_error();
  if (!t || !o) return tt::fail(TT_EINVAL, "tree_info: NULL argument");
  o->n_nodes = t->N;
  o->n_seqs = t->B;
  o->n_roots = t->n_roots;
  o->n_leaves = t->n_leaves;
  o->max_depth = t->max_depth;
  o->seq_tokens = t->seq_tokens;
  o->leaf_tokens = t->leaf_tokens;
  o->n_targets = int64_t(t->tgt_dfs.size());
  o->pairs = t->pairs;
  o->dense_pairs = t->dense_pairs;
  o->block_q = t->bq;
  o->block_k = t->bk;
  o->n_tiles = t->n_tiles;
  o->n_full_tiles = t->n_full;
  return TT_OK;
}

extern "C" int tree_export(const tt_tree* t, const tt_tree_arrays* d) {
  tt::clear_error();
  if (!t || !d) return tt::fail(TT_EINVAL, "tree_export: NULL argument");
  auto cp = [](int32_t* dst, const std::vector<int32_t>& src) {
    if (dst && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(int32_t));
  };
  cp(d->token, t->token);
  cp(d->depth, t->depth);
  cp(d->end, t->end);
  cp(d->parent, t->parent);
  cp(d->n_pass, t->n_pass);
  if (d->weight && !t->weight.empty()) std::memcpy(d->weight, t->weight.data(), t->weight.size() * sizeof(float));
  cp(d->seq_pos_to_dfs, t->seq_pos_to_dfs);
  cp(d->tgt_row_ptr, t->tgt_row_ptr);
  cp(d->tgt_dfs, t->tgt_dfs);
  for (size_t i = 0; i < t->tgt_dfs.size(); ++i) {
    if (d->tgt_token) d->tgt_token[i] = t->token[size_t(t->tgt_dfs[i])];
    if (d->tgt_w) d->tgt_w[i] = t->weight[size_t(t->tgt_dfs[i])];
  }
  return TT_OK;
}

extern "C" int tree_target_weights(const tt_tree* t, const float* seq_scale, const uint8_t* token_mask,
                                   float* tgt_w) {
  tt::clear_error();
  if (!t || !tgt_w) return tt::fail(TT_EINVAL, "tree_target_weights: NULL argument");
  if (seq_scale)
    for (int32_t s = 0; s < t->B; ++s)
      if (!std::isfinite(seq_scale[s])) return tt::fail(TT_EINVAL, "tree_target_weights: seq_scale must be finite");
  // sums in double over sequences in input order, one division, one rounding to float
  std::vector<double> acc(size_t(t->N), 0.0);
  for (int32_t s = 0; s < t->B; ++s) {
    const double a = seq_scale ? double(seq_scale[s]) : 1.0;
    for (int64_t k = t->seq_off[size_t(s)] + 1; k < t->seq_off[size_t(s) + 1]; ++k)
      if (!token_mask || token_mask[k]) acc[size_t(t->seq_pos_to_dfs[size_t(k)])] += a;
  }
  const double B = double(t->B);
  for (size_t i = 0; i < t->tgt_dfs.size(); ++i) tgt_w[i] = float(acc[size_t(t->tgt_dfs[i])] / B);
  return TT_OK;
}

extern "C" int tree_plan_bytes(const tt_tree* t, size_t* bytes) {
  tt::clear_error();
  if (!t || !bytes) return tt::fail(TT_EINVAL, "tree_plan_bytes: NULL argument");
  *bytes = t->plan.size() * sizeof(int32_t);
  return TT_OK;
}

extern "C" int tree_plan_copy(const tt_tree* t, void* dst, size_t bytes) {
  tt::clear_error();
  if (!t || !dst) return tt::fail(TT_EINVAL, "tree_plan_copy: NULL argument");
  const size_t need = t->plan.size() * sizeof(int32_t);
  if (bytes < need) return tt::fail(TT_EWORKSPACE, "tree_plan_copy: buffer smaller than tree_plan_bytes");
  std::memcpy(dst, t->plan.data(), need);
  return TT_OK;
}
