// Internal host-side definitions shared by the library's translation units.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tt.h"

// Device plan image: int32 words.  Header, then sections each aligned to 64
// words (256 bytes) so every section is a naturally aligned device array.
namespace ttp {
enum : int32_t {
  kMagic = 0x31505454,  // "TTP1"
  // header word indices
  H_MAGIC = 0, H_N, H_BQ, H_BK, H_NQB, H_NKB, H_NTILES, H_BYTES,
  H_DEPTH, H_END, H_QB_PTR, H_QB_TILES, H_QB_ORDER,
  H_KB_QLO, H_KB_QHI, H_KB_MINEND, H_KB_ORDER,
  H_ID,  // FNV-1a hash of the image (this word 0 while hashing): which tree it belongs to
  H_WORDS = 64
};
constexpr int32_t kFullBit = int32_t(0x40000000);  // tile entry: kb | kFullBit if FULL
}  // namespace ttp

struct tt_tree {
  int32_t N = 0, B = 0, n_roots = 0, n_leaves = 0, max_depth = -1;
  int64_t seq_tokens = 0, leaf_tokens = 0, pairs = 0, dense_pairs = 0;
  std::vector<int32_t> token, depth, end, parent, n_pass;
  std::vector<float> weight;
  std::vector<int32_t> seq_pos_to_dfs;
  std::vector<int64_t> seq_off;  // [B+1] input sequence offsets
  std::vector<int32_t> tgt_row_ptr, tgt_dfs;
  // schedule
  int32_t bq = 64, bk = 64, nqb = 0, nkb = 0;
  int64_t n_tiles = 0, n_full = 0;
  std::vector<int32_t> plan;  // the device plan image (host copy)
};

namespace tt {
int fail(int code, const std::string& msg);  // records msg, returns code
void clear_error();
inline const int32_t* plan_section(const tt_tree* t, int hdr) { return t->plan.data() + t->plan[hdr]; }
}  // namespace tt

// Path-mode traversal plan (tree_path_build).  Segments are maximal chains of
// DFS rows; events list the walk: e >= 0 enters segment e, e < 0 leaves
// segment -1 - e.  A round is a maximal run of consecutive enters (a forward
// round) or of consecutive leaves (a backward round): its segments lie
// contiguously on the stack, positions [p0, p1), so one chunked pass serves
// them all.  `chain` is a one-sequence tree of max_path rows whose plan
// serves every attention call of the walk (stack position = depth).
struct tt_path {
  struct Seg {
    int32_t row0, len, depth0, parent;
  };
  struct Round {
    bool bwd;
    int32_t p0, p1;    // stack positions covered
    int32_t ev0, ev1;  // its events: events[ev0 .. ev1)
  };
  const tt_tree* tree = nullptr;
  tt_tree* chain = nullptr;
  int32_t chunk = 2048, order = 0, max_path = 0;
  std::vector<Seg> segs;
  std::vector<int32_t> events;
  std::vector<Round> rounds;
  int64_t fwd_calls = 0, bwd_calls = 0, pad_rows = 0, pad_pairs = 0;
  ~tt_path();
};
