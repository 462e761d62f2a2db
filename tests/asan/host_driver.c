/* Drives the library's host-only entry points (trie build, export, plan
 * image, path plan, RL weights) over random and edge-case inputs; built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_asan.py.
 * Prints "ok" and exits 0 when every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tt.h"

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)rng;
}

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c, tt_last_error()); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int one_case(int n_seqs, int max_len, int vocab, int bq, int bk) {
  int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_seqs + 1));
  off[0] = 0;
  for (int s = 0; s < n_seqs; ++s) off[s + 1] = off[s] + (int64_t)(next_u32() % (uint32_t)(max_len + 1));
  const int64_t total = off[n_seqs];
  int32_t* tok = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
  for (int64_t i = 0; i < total; ++i) tok[i] = (int32_t)(next_u32() % (uint32_t)vocab);
  /* some sequences copy a prefix of the previous one, so prefixes are shared */
  for (int s = 1; s < n_seqs; ++s) {
    const int64_t la = off[s] - off[s - 1], lb = off[s + 1] - off[s];
    const int64_t k = la < lb ? la : lb;
    if (next_u32() % 2) memcpy(tok + off[s], tok + off[s - 1], sizeof(int32_t) * (size_t)(k / 2));
  }
  tt_tree* t = NULL;
  CHECK(tree_build(tok, off, n_seqs, bq, bk, &t) == TT_OK);
  tt_tree_info inf;
  CHECK(tree_info(t, &inf) == TT_OK);
  const int64_t N = inf.n_nodes, T = inf.n_targets;
  tt_tree_arrays a;
  memset(&a, 0, sizeof(a));
  a.token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  a.depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  a.end = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  a.parent = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  a.n_pass = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 1));
  a.weight = (float*)malloc(sizeof(float) * (size_t)(N + 1));
  a.seq_pos_to_dfs = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total + 1));
  a.tgt_row_ptr = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N + 2));
  a.tgt_dfs = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 1));
  a.tgt_token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 1));
  a.tgt_w = (float*)malloc(sizeof(float) * (size_t)(T + 1));
  CHECK(tree_export(t, &a) == TT_OK);
  for (int64_t i = 0; i < N; ++i) CHECK(a.end[i] > i && a.end[i] <= N);
  size_t pb = 0;
  CHECK(tree_plan_bytes(t, &pb) == TT_OK && pb > 0);
  void* plan = malloc(pb);
  CHECK(tree_plan_copy(t, plan, pb) == TT_OK);
  CHECK(tree_plan_copy(t, plan, pb - 1) == TT_EWORKSPACE);
  float* sc = (float*)malloc(sizeof(float) * (size_t)(n_seqs + 1));
  uint8_t* mk = (uint8_t*)malloc((size_t)(total + 1));
  for (int s = 0; s < n_seqs; ++s) sc[s] = (float)((int)(next_u32() % 200) - 100) / 37.f;
  for (int64_t i = 0; i < total; ++i) mk[i] = (uint8_t)(next_u32() % 3 != 0);
  float* w = (float*)malloc(sizeof(float) * (size_t)(T + 1));
  CHECK(tree_target_weights(t, sc, mk, w) == TT_OK);
  CHECK(tree_target_weights(t, NULL, NULL, w) == TT_OK);
  for (int64_t i = 0; i < T; ++i) CHECK(w[i] == a.tgt_w[i]);
  const int chunks[3] = {64, 128, 2048};
  for (int c = 0; c < 3; ++c)
    for (int order = 0; order < 2; ++order) {
      tt_path* p = NULL;
      CHECK(tree_path_build(t, chunks[c], order, &p) == TT_OK);
      tt_path_info pi;
      CHECK(tree_path_info(p, &pi) == TT_OK);
      CHECK(pi.max_path == (N ? inf.max_depth + 1 : 0));
      const int S = pi.n_segments;
      int32_t* r0 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
      int32_t* ln = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
      int32_t* d0 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
      int32_t* pa = (int32_t*)malloc(sizeof(int32_t) * (size_t)(S + 1));
      int32_t* ev = (int32_t*)malloc(sizeof(int32_t) * (size_t)(2 * S + 1));
      CHECK(tree_path_segments(p, r0, ln, d0, pa, ev) == TT_OK);
      int64_t rows = 0;
      for (int s = 0; s < S; ++s) rows += ln[s];
      CHECK(rows == N);
      free(r0); free(ln); free(d0); free(pa); free(ev);
      tree_path_free(p);
    }
  free(w); free(sc); free(mk); free(plan);
  free(a.token); free(a.depth); free(a.end); free(a.parent); free(a.n_pass); free(a.weight);
  free(a.seq_pos_to_dfs); free(a.tgt_row_ptr); free(a.tgt_dfs); free(a.tgt_token); free(a.tgt_w);
  tree_free(t);
  free(tok); free(off);
  return 0;
}

int main(void) {
  /* error paths: nothing is built, nothing leaks */
  tt_tree* t = NULL;
  int64_t off[3] = {0, 2, 1};
  int32_t tok[2] = {1, -1};
  CHECK(tree_build(tok, off, 2, 0, 0, &t) == TT_EINVAL && t == NULL);
  off[2] = 2;
  CHECK(tree_build(tok, off, 2, 0, 0, &t) == TT_EINVAL);  /* negative token */
  CHECK(tree_build(NULL, off, 2, 0, 0, &t) == TT_EINVAL);
  CHECK(tree_build(tok, off, 1, 48, 0, &t) == TT_EINVAL); /* block not a power of two */
  tree_free(NULL);
  tree_path_free(NULL);
  const int sizes[][5] = {{0, 1, 3, 0, 0}, {1, 0, 3, 0, 0}, {1, 300, 5, 64, 64}, {7, 90, 4, 16, 32},
                          {20, 200, 3, 64, 128}, {40, 70, 2, 256, 16}, {3, 1000, 7, 128, 64}};
  for (size_t i = 0; i < sizeof(sizes) / sizeof(sizes[0]); ++i)
    for (int rep = 0; rep < 4; ++rep)
      if (one_case(sizes[i][0], sizes[i][1], sizes[i][2], sizes[i][3], sizes[i][4])) return 1;
  printf("ok\n");
  return 0;
}
