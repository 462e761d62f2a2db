// Path-mode traversal plan: segments of the tree, the depth-first walk over
// them and the chunking of each segment's queries (AReaL-DTA, arXiv
// 2602.00482, summary page, Methodology in Plain English and Key
// Contributions 2).  Host only.
#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

tt_path::~tt_path() { tree_free(chain); }

namespace {

// Chunks of a segment occupying stack positions [p0, p1): boundaries at the
// multiples of `chunk`, so only the first chunk of a segment can start off a
// 64-row boundary.  Calls through f(c0, c1), left to right.
template <typename F>
void for_chunks(int32_t p0, int32_t p1, int32_t chunk, F f) {
  int32_t c0 = p0;
  while (c0 < p1) {
    const int32_t c1 = std::min(p1, (c0 / chunk + 1) * chunk);
    f(c0, c1);
    c0 = c1;
  }
}

}  // namespace

extern "C" int tree_path_build(const tt_tree* t, int32_t chunk, int32_t order, tt_path** out) {
  tt::clear_error();
  if (!t || !out) return tt::fail(TT_EINVAL, "tree_path_build: NULL argument");
  if (chunk <= 0 || chunk % 64 != 0) return tt::fail(TT_EINVAL, "tree_path_build: chunk must be a positive multiple of 64");
  if (order != 0 && order != 1) return tt::fail(TT_EINVAL, "tree_path_build: order must be 0 or 1");
  *out = nullptr;
  tt_path* p = new (std::nothrow) tt_path;
  if (!p) return tt::fail(TT_ENOMEM, "tree_path_build: out of memory");
  try {
    p->tree = t;
    p->chunk = chunk;
    p->order = order;
    const int32_t N = t->N;
    // segments: row i continues row i-1's segment iff i-1 is i's parent and has no other child
    std::vector<int32_t> nchild(static_cast<size_t>(N), 0), seg_of(static_cast<size_t>(N), -1);
    for (int32_t i = 0; i < N; ++i)
      if (t->parent[size_t(i)] >= 0) ++nchild[size_t(t->parent[size_t(i)])];
    for (int32_t i = 0; i < N; ++i) {
      const int32_t par = t->parent[size_t(i)];
      if (i > 0 && par == i - 1 && nchild[size_t(i - 1)] == 1) {
        seg_of[size_t(i)] = seg_of[size_t(i - 1)];
        ++p->segs.back().len;
      } else {
        seg_of[size_t(i)] = int32_t(p->segs.size());
        p->segs.push_back({i, 1, t->depth[size_t(i)], par < 0 ? -1 : seg_of[size_t(par)]});
      }
    }
    p->max_path = t->max_depth + 1;
    // children lists in DFS order, then the walk
    const int32_t S = int32_t(p->segs.size());
    std::vector<std::vector<int32_t>> kids(static_cast<size_t>(S));
    std::vector<int32_t> roots;
    for (int32_t s = 0; s < S; ++s) {
      const int32_t par = p->segs[size_t(s)].parent;
      (par < 0 ? roots : kids[size_t(par)]).push_back(s);
    }
    if (order == 1) {
      // greedy: a segment's backward round continues into its parent only
      // from the parent's last child, so the child whose own chain of last
      // descendants is shortest goes last (it lengthens the parent's round
      // instead of making a short round of its own); the others keep their
      // longer rounds.  chain(s) = len(s) + chain(last child of s), bottom up
      // (children have larger indices than their parent); ties keep DFS order.
      std::vector<int64_t> chain_len(static_cast<size_t>(S), 0);
      auto by_chain = [&](int32_t a, int32_t b) { return chain_len[size_t(a)] > chain_len[size_t(b)]; };
      for (int32_t s = S - 1; s >= 0; --s) {
        auto& k = kids[size_t(s)];
        std::stable_sort(k.begin(), k.end(), by_chain);
        chain_len[size_t(s)] = p->segs[size_t(s)].len + (k.empty() ? 0 : chain_len[size_t(k.back())]);
      }
      std::stable_sort(roots.begin(), roots.end(), by_chain);
    }
    p->events.reserve(size_t(2 * S));
    std::vector<std::pair<int32_t, size_t>> stack;  // (segment, next child index)
    for (int32_t r : roots) {
      p->events.push_back(r);
      stack.push_back({r, 0});
      while (!stack.empty()) {
        auto& top = stack.back();
        const auto& ch = kids[size_t(top.first)];
        if (top.second < ch.size()) {
          const int32_t c = ch[top.second++];
          p->events.push_back(c);
          stack.push_back({c, 0});
        } else {
          p->events.push_back(-1 - top.first);
          stack.pop_back();
        }
      }
    }
    // rounds: maximal runs of enters / of leaves; each run's segments are
    // stacked one on the next (an enter run descends, a leave run ascends)
    for (size_t e = 0; e < p->events.size();) {
      const bool bwd = p->events[e] < 0;
      size_t f = e;
      while (f < p->events.size() && (p->events[f] < 0) == bwd) ++f;
      const auto seg_at = [&](size_t i) { return p->segs[size_t(bwd ? -1 - p->events[i] : p->events[i])]; };
      const tt_path::Seg first = seg_at(e), last = seg_at(f - 1);
      tt_path::Round rd;
      rd.bwd = bwd;
      rd.ev0 = int32_t(e);
      rd.ev1 = int32_t(f);
      rd.p0 = bwd ? last.depth0 : first.depth0;
      rd.p1 = bwd ? first.depth0 + first.len : last.depth0 + last.len;
      p->rounds.push_back(rd);
      // a forward round is one call; a backward round runs in chunks
      const auto count_call = [&](int32_t c0, int32_t) {
        ++(bwd ? p->bwd_calls : p->fwd_calls);
        const int64_t qo = c0 & ~63;
        p->pad_rows += c0 - qo;
        p->pad_pairs += (int64_t(c0) * (c0 + 1) - qo * (qo + 1)) / 2;  // sum over rows r in [qo, c0) of r + 1
      };
      if (bwd)
        for_chunks(rd.p0, rd.p1, chunk, count_call);
      else
        count_call(rd.p0, rd.p1);
      e = f;
    }
    // the chain of the longest path: its plan serves every call
    if (p->max_path > 0) {
      std::vector<int32_t> tok(static_cast<size_t>(p->max_path));
      for (int32_t i = 0; i < p->max_path; ++i) tok[size_t(i)] = i;
      const int64_t off[2] = {0, p->max_path};
      const int rc = tree_build(tok.data(), off, 1, 64, 64, &p->chain);
      if (rc != TT_OK) {
        delete p;
        return rc;
      }
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return tt::fail(TT_ENOMEM, "tree_path_build: out of memory");
  }
  *out = p;
  return TT_OK;
}

extern "C" void tree_path_free(tt_path* p) { delete p; }

extern "C" int tree_path_info(const tt_path* p, tt_path_info* out) {
  tt::clear_error();
  if (!p || !out) return tt::fail(TT_EINVAL, "tree_path_info: NULL argument");
  out->n_segments = int32_t(p->segs.size());
  out->max_path = p->max_path;
  out->chunk = p->chunk;
  out->order = p->order;
  out->fwd_calls = p->fwd_calls;
  out->bwd_calls = p->bwd_calls;
  out->pad_rows = p->pad_rows;
  out->query_rows = 2 * int64_t(p->tree->N) + p->pad_rows;
  out->pad_pairs = p->pad_pairs;
  return TT_OK;
}

extern "C" int tree_path_segments(const tt_path* p, int32_t* row0, int32_t* len, int32_t* depth0, int32_t* parent,
                                  int32_t* events) {
  tt::clear_error();
  if (!p) return tt::fail(TT_EINVAL, "tree_path_segments: path is NULL");
  for (size_t s = 0; s < p->segs.size(); ++s) {
    if (row0) row0[s] = p->segs[s].row0;
    if (len) len[s] = p->segs[s].len;
    if (depth0) depth0[s] = p->segs[s].depth0;
    if (parent) parent[s] = p->segs[s].parent;
  }
  if (events) std::copy(p->events.begin(), p->events.end(), events);
  return TT_OK;
}
