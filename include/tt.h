/*
 * tt.h -- C ABI of libtreeattn: prefix-tree attention and the branch-weighted
 * loss on one AMD MI355X (gfx950).
 *
 * What it computes.  Rollout sequences that share prefixes form a tree; the
 * tree is serialized in DFS order so that every unique token is one row and is
 * computed once (Tree Training, arXiv 2511.00413, Abstract; AReaL-DTA, arXiv
 * 2602.00482, summary page, What This Paper Is About).  Row i attends to row j
 * iff j is i or an ancestor of i -- in DFS order exactly  j <= i < end[j] --
 * with rotary position equal to the depth, which reproduces per-branch causal
 * attention row for row (Tree Training, Abstract: per-branch log-probabilities
 * must be matched exactly).  The loss is the per-token weighted NLL whose
 * weight is the fraction of branches through the token, which equals the loss
 * averaged over branches (Tree Training, Abstract).
 *
 * Conventions used by every call (the pages leave them open):
 *   - a branch is an input sequence, counted with multiplicity; B = n_seqs;
 *   - sibling order is ascending token id (lexicographic DFS; AReaL-DTA
 *     summary, Key Contributions 3);
 *   - RoPE: theta_k = base^(-2k/d), k < d/2, coordinate k paired with k + d/2
 *     ("rotate half"), position = depth;
 *   - softmax scale 1/sqrt(d) unless given; query head h uses key/value head
 *     h / (h_q / h_kv); LSE is natural-log;
 *   - every non-root row t is a loss target predicted from its parent's row.
 *
 * Ownership and errors.  Every function returns TT_OK (0) or a negative
 * tt_status and never throws or aborts.  tt_last_error() returns text for the
 * last failure on the calling thread.  All preconditions the host can check
 * are checked before anything is launched; on failure nothing is launched and
 * no output is touched.  The caller allocates every device buffer (outputs,
 * plan, workspace) and passes the stream; the library never allocates device
 * memory and never synchronises.  Launch errors are reported as TT_EDEVICE;
 * faults during execution surface at the caller's next synchronisation.  The
 * tree_* host functions (all but tree_plan_upload) make no HIP call and work
 * with no GPU present.  A built tree is immutable: concurrent calls on
 * different streams may share it.
 *
 * Layouts.  Row-major, contiguous, no padding.  Device pointers must be
 * 16-byte aligned.  "dtype" tensors are float32 (TT_F32) or bfloat16 (TT_BF16).
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TT_OK = 0,
  TT_EINVAL = -1,        /* bad argument (NULL, range, shape, alignment, layout) */
  TT_ENOMEM = -2,        /* host allocation failed */
  TT_EWORKSPACE = -3,    /* workspace or plan buffer too small */
  TT_EUNSUPPORTED = -4,  /* valid but not implemented (head dim, dtype, block size) */
  TT_EDEVICE = -5,       /* a HIP call or kernel launch failed */
  TT_EOVERFLOW = -6      /* sizes exceed the library's index ranges */
} tt_status;

typedef enum { TT_F32 = 0, TT_BF16 = 1 } tt_dtype;

/* hipStream_t, passed as an opaque pointer (NULL = the null stream). */
typedef void* tt_stream;

/* Flags of tt_attn_args (and tt_path_args). */
#define TT_ALLOW_GENERIC 1u /* bf16 shapes the matrix-core kernels do not take (head dim other than
                               128, schedule blocks other than 64) run on the vector kernels, many
                               times slower, instead of failing with TT_EUNSUPPORTED */

/* Flags of tree_attn_bwd. */
#define TT_ACCUMULATE_DKDV 1u /* d_k, d_v are float32 and the call ADDS into them */
#define TT_BWD_REUSE_ROTATED 2u /* the workspace still holds the rotated q and k that
                                   tree_attn_fwd wrote for the same arguments: skip
                                   rotating them again */

typedef struct tt_tree tt_tree; /* opaque, host memory owned by the library */

typedef struct {
  int64_t n_nodes;      /* N: unique tokens = rows of the DFS order */
  int64_t n_seqs;       /* B: input sequences (branches), with multiplicity */
  int64_t n_roots;      /* rows with no parent (first tokens of the forest) */
  int64_t n_leaves;     /* rows with no child */
  int64_t max_depth;    /* -1 if N == 0 */
  int64_t seq_tokens;   /* sum of |s| over the input */
  int64_t leaf_tokens;  /* sum over leaves of (depth+1): tokens of distinct maximal sequences */
  int64_t n_targets;    /* N - n_roots */
  int64_t pairs;        /* visible (query, key) pairs per head = sum_i (depth_i + 1) */
  int64_t dense_pairs;  /* causal pairs of the branches computed apart = sum_s |s|(|s|+1)/2 */
  int64_t block_q;      /* schedule tile sizes */
  int64_t block_k;
  int64_t n_tiles;      /* non-empty (q-block, k-block) tiles */
  int64_t n_full_tiles; /* tiles in which every pair is visible */
} tt_tree_info;

/* Caller-owned HOST arrays for tree_export; NULL members are skipped. */
typedef struct {
  int32_t* token;          /* [N] token id of each row */
  int32_t* depth;          /* [N] */
  int32_t* end;            /* [N] exclusive end of the row's subtree */
  int32_t* parent;         /* [N] -1 at a root */
  int32_t* n_pass;         /* [N] input sequences (with multiplicity) through the row */
  float* weight;           /* [N] n_pass / B rounded once to float32 */
  int32_t* seq_pos_to_dfs; /* [seq_tokens] row of each input token, input order */
  int32_t* tgt_row_ptr;    /* [N+1] CSR: targets predicted from row r are its children */
  int32_t* tgt_dfs;        /* [n_targets] child rows, ascending */
  int32_t* tgt_token;      /* [n_targets] their token ids (vocabulary index) */
  float* tgt_w;            /* [n_targets] their weights */
} tt_tree_arrays;

/*
 * tree_build -- prefix tree of the input sequences in lexicographic DFS order.
 * (Tree Training, Abstract: DFS serialization, each token once, branch-fraction
 * weights; AReaL-DTA summary, Key Contributions 3 and Methodology: rollouts
 * sorted into one prefix tree in lexicographic DFS order.)
 *   tokens       host [seq_offsets[n_seqs]] int32, each >= 0
 *   seq_offsets  host [n_seqs+1] int64, seq_offsets[0] == 0, non-decreasing
 *                (empty sequences are allowed and count towards B)
 *   n_seqs       0 <= n_seqs < 2^24 (so n_pass/B is exact to one rounding)
 *   block_q/k    schedule tile sizes, 0 = 64; powers of two in [16, 256]
 *   out          receives the tree; free with tree_free
 * Errors: TT_EINVAL (NULL, offsets, negative token, block size),
 * TT_EOVERFLOW (n_seqs >= 2^24 or more than 2^31-1 tokens), TT_ENOMEM.
 */
int tree_build(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
               int32_t block_q, int32_t block_k, tt_tree** out);

/* Frees a tree (NULL is a no-op). Do not free before a plan upload from it has completed. */
void tree_free(tt_tree* tree);

/* Sizes and statistics (AReaL-DTA summary, Main Findings 1: compression is
 * seq_tokens / n_nodes; leaves-only compression is leaf_tokens / n_nodes). */
int tree_info(const tt_tree* tree, tt_tree_info* out);

/* Copies the DFS arrays into caller-owned host arrays (NULL members skipped). */
int tree_export(const tt_tree* tree, const tt_tree_arrays* dst);

/*
 * tree_target_weights -- loss weights of the targets for RL post-training:
 * per-sequence scalars (e.g. advantages) and per-token loss masks (e.g. 0 on
 * prompt tokens).  (AReaL-DTA, arXiv 2602.00482, summary page, Main Findings
 * and Why This Matters: the trees come from RL rollouts trained with GRPO.)
 * Token k >= 1 of sequence s is predicted from position k-1 and enters the
 * branch-averaged loss with factor a_s * mask[s,k] / B, so the tree weight of
 * target row t is  w_t = (1/B) * sum of a_s over the sequences s through t
 * whose token at depth(t) is unmasked  -- summed in double over sequences in
 * input order, divided once, rounded once to float32.  Weights may be
 * negative.  With seq_scale == NULL (all 1) and token_mask == NULL (all kept)
 * this is n_pass / B, bit for bit tree_export's tgt_w.
 *   seq_scale   host [n_seqs] float32 (finite), or NULL
 *   token_mask  host [seq_tokens] uint8 in input order (nonzero = in the
 *               loss), or NULL; entries at k = 0 of a sequence are ignored
 *   tgt_w       host [n_targets] float32 output, in tree_export's tgt_dfs order
 * Errors: TT_EINVAL (NULL tree or output, non-finite scale).  Host only.
 */
int tree_target_weights(const tt_tree* tree, const float* seq_scale, const uint8_t* token_mask, float* tgt_w);

/*
 * Device plan: depth[], end[] and the tile schedule (per q-block list of
 * non-empty k-blocks tagged FULL or PARTIAL; per k-block the contiguous range
 * of query rows that see it; launch orders: q-blocks from the last row up,
 * groups of 256 keys by the end of the rows that see them, latest first, so
 * that workgroups running together share tiles).
 * tree_plan_bytes gives its size; tree_plan_upload copies it (hipMemcpyAsync on
 * `stream`) into the caller's device buffer of at least that many bytes.
 * Errors: TT_EINVAL, TT_EWORKSPACE (buffer too small), TT_EDEVICE.
 * The image's header carries its row count and an identity word (a hash of
 * the image, which holds structure only, not token ids: trees of one shape
 * have interchangeable plans).  The library records, per device address, the
 * identity of the image last uploaded there; an attention call whose plan
 * address holds no upload, or the upload of a tree of another shape, fails
 * with TT_EINVAL before anything is launched.  As a backstop for device
 * memory the host cannot see (a plan buffer overwritten by other work), every
 * kernel that reads the plan first compares the header with the tree of the
 * call and returns without writing when they differ, so a wrong plan is
 * never read out of bounds.
 */
int tree_plan_bytes(const tt_tree* tree, size_t* bytes);
int tree_plan_upload(const tt_tree* tree, void* dev_plan, size_t bytes, tt_stream stream);

/* Copies the same plan image into caller-owned HOST memory (for inspection;
 * int32 words: header, then the sections).  No HIP call. */
int tree_plan_copy(const tt_tree* tree, void* host_dst, size_t bytes);

/*
 * Attention geometry and buffers.  Query rows are the DFS rows
 * [q_off, q_off + n_q); key rows are [0, n_k).  Tree mode: q_off = 0,
 * n_q = n_k = N.  Path/chunk mode (AReaL-DTA summary, Key Contributions 2 and
 * Methodology: a long suffix split into fixed chunks run right to left against
 * the cached prefix state): queries are one chunk, keys the prefix plus the
 * chunk.  Requires 0 <= q_off, q_off % block_q == 0, q_off + n_q <= n_k <= N.
 */
typedef struct {
  const tt_tree* tree;     /* host tree the plan was built from */
  const void* plan;        /* device plan from tree_plan_upload */
  int32_t q_off, n_q, n_k;
  int32_t h_q, h_kv, d;    /* h_q % h_kv == 0; d = 128 (bf16) or d in {16..256, %16} (f32) */
  tt_dtype dtype;
  float scale;             /* 0 = 1/sqrt(d) */
  float rope_base;         /* 0 = no rotation */
  const void* q;           /* device [n_q, h_q, d] dtype */
  const void* k;           /* device [n_k, h_kv, d] dtype */
  const void* v;           /* device [n_k, h_kv, d] dtype */
  void* o;                 /* device [n_q, h_q, d] dtype: output of fwd, input of bwd */
  float* lse;              /* device [n_q, h_q] float32: output of fwd, input of bwd */
  void* workspace;         /* device scratch, >= tree_attn_workspace_bytes: the query operand,
                              rotated k and a (cos, sin) table of the tree's depths (with
                              RoPE) first, at the same offsets for both calls; for the
                              backward also D and fp32 dQ.  The library keeps nothing there between calls; a
                              caller that passes the forward's workspace, unmodified, to the
                              backward may set TT_BWD_REUSE_ROTATED */
  size_t workspace_bytes;
  uint32_t flags;          /* 0 or TT_ALLOW_GENERIC; other bits: TT_EINVAL */
} tt_attn_args;

/* Kernels.  bf16 with head dim 128 (and the default 64-row schedule blocks)
 * runs on the hand-written matrix-core kernels for any GQA group size and any
 * tensor size; other bf16 shapes fail with TT_EUNSUPPORTED unless
 * TT_ALLOW_GENERIC is set.  float32 runs on the vector kernels. */

/* Workspace size for tree_attn_fwd (for_bwd = 0) or tree_attn_bwd (for_bwd = 1). */
int tree_attn_workspace_bytes(const tt_attn_args* args, int for_bwd, size_t* bytes);

/*
 * tree_attn_fwd -- O[i,h] = sum over visible j of softmax_j(scale q'_i.k'_j) v_j and
 * LSE[i,h], where ' is the rotation at the row's depth (Tree Training,
 * Abstract; AReaL-DTA summary, Key Contributions 1: shared prefix segments
 * computed once).  Overwrites o and lse.
 */
int tree_attn_fwd(const tt_attn_args* args, tt_stream stream);

/*
 * tree_attn_bwd -- gradients of sum(dO * O) with respect to q, k, v, recomputing
 * the probabilities from LSE.  A shared prefix row receives the sum of the
 * gradients of all its descendants' queries (AReaL-DTA summary, Key
 * Contributions 1 and Methodology: gradients from all descendant leaves
 * accumulated into the shared prefix).
 *   a.o, a.lse  the forward's outputs for the same arguments
 *   d_o         device [n_q, h_q, d] dtype
 *   d_q         device [n_q, h_q, d] dtype, overwritten
 *   d_k, d_v    device [n_k, h_kv, d]: dtype and overwritten, or float32 and
 *               added into with TT_ACCUMULATE_DKDV (chunked path mode: the
 *               prefix keys collect every chunk's contribution)
 *   flags       TT_ACCUMULATE_DKDV, TT_BWD_REUSE_ROTATED (the caller vouches
 *               that the workspace holds what tree_attn_fwd wrote there for
 *               these q, k, tree, q_off, rope_base; results are then those of a
 *               call without the flag).  Other bits: TT_EINVAL.
 */
typedef struct {
  tt_attn_args a;
  const void* d_o;
  void* d_q;
  void* d_k;
  void* d_v;
  uint32_t flags;
} tt_attn_bwd_args;

int tree_attn_bwd(const tt_attn_bwd_args* args, tt_stream stream);

/*
 * Weighted tree NLL (Tree Training, Abstract: branch-averaged loss == per-token
 * weighted loss).  For every row r with targets t (token x_t, weight w_t):
 *   loss   += sum_t w_t (lse(z_r) - z_r[x_t])
 *   logp_t  = z_r[x_t] - lse(z_r)
 *   dZ_r    = (sum_t w_t) softmax(z_r) - sum_t w_t e_{x_t}
 * Two modes, exactly one per call:
 *   logits mode: z = logits [n_rows, vocab] (dtype logits_dtype); d_logits
 *                (same dtype and shape, may alias logits) receives dZ.
 *   fused mode:  z = hidden [n_rows, d_model] @ w_vocab [d_model, vocab], both
 *                bf16, d_model and vocab multiples of 8; z and dZ live in the
 *                workspace as bf16; d_hidden [n_rows, d_model] bf16 receives
 *                dZ w_vocab^T and d_w_vocab [d_model, vocab] (dtype dw_dtype)
 *                receives hidden^T dZ.
 * vocab <= 262144 (TT_EUNSUPPORTED beyond).
 * Targets are a device CSR: tgt_row_ptr [n_rows+1], tgt_id [n_tgt] (0 <= id <
 * vocab), tgt_w [n_tgt].  loss is a device float32 scalar (overwritten); logp
 * [n_tgt] float32 or NULL; each gradient pointer may be NULL to skip it.
 */
typedef struct {
  int32_t n_rows, d_model, vocab, n_tgt;
  const void* hidden;
  const void* w_vocab;
  const void* logits;
  tt_dtype logits_dtype;
  const int32_t* tgt_row_ptr;
  const int32_t* tgt_id;
  const float* tgt_w;
  float* loss;
  float* logp;
  void* d_hidden;
  void* d_w_vocab;
  tt_dtype dw_dtype;
  void* d_logits;
  void* workspace;
  size_t workspace_bytes;
} tt_nll_args;

int tree_nll_workspace_bytes(const tt_nll_args* args, size_t* bytes);
int tree_weighted_nll(const tt_nll_args* args, tt_stream stream);

/*
 * tree_weighted_nll_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): tree_weighted_nll in logits mode with its per-row partial
 * losses in a static device array of TT_NOALLOC_MAX_ROWS float32 (4 MiB) per
 * GPU, held until the process ends, instead of the workspace (workspace and
 * workspace_bytes are ignored).  It calls no allocating routine; the first
 * call on a device looks the array up once (hipGetSymbolAddress).  The
 * stream's device must be the current device.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Every row's entry is
 * written before it is summed, so nothing needs clearing between calls.
 * Results equal tree_weighted_nll's bit for bit.
 * Errors: those of tree_weighted_nll; TT_EUNSUPPORTED in fused mode;
 * TT_EWORKSPACE when n_rows > TT_NOALLOC_MAX_ROWS; TT_EDEVICE if the array
 * cannot be reached.
 */
#define TT_NOALLOC_MAX_ROWS (1 << 20)
int tree_weighted_nll_noalloc(const tt_nll_args* args, tt_stream stream);

/*
 * Path mode: one attention layer over the tree, walked depth-first with a
 * stack that holds only the current root-to-node path (AReaL-DTA, arXiv
 * 2602.00482, summary page, Methodology in Plain English: forward only the new
 * segment on entering a branch against the cached ancestors, backpropagate a
 * segment when it is left for good, live state proportional to the longest
 * path; Key Contributions 2: long suffixes backpropagated in fixed-length
 * chunks, right to left).
 *
 * A segment is a maximal run of DFS rows in which every row but the last has
 * exactly one child; the segments form a tree.  Entering a segment pushes its
 * Q, K (rotated at their depths) and V onto the stack at positions = depths;
 * leaving it (after all descendants) pops it.  Consecutive enters form a
 * forward round and consecutive leaves a backward round: the round's
 * segments lie one on the next on the stack, so a round is one chunked pass
 * over its positions -- one forward and one backward round per leaf
 * (AReaL-DTA, Key Contributions 2: push-pop execution, about one regular
 * forward/backward round per leaf).  A forward round is one call over its
 * positions against the stack below them; a backward round runs in chunks
 * (boundaries at multiples of the chunk length) from the right, adding dK, dV
 * into float32 stack accumulators, then writes each popped segment's dK, dV
 * rows out and clears their stack slots.  On the matrix cores with groups of
 * a multiple of 4 query heads (or of 2 over an even number of kv heads),
 * consecutive chunk calls share one launch
 * (three for chunks of up to 2048 rows, two above; each with its own dO
 * copy, dQ block and pair of accumulators, summed when the segment is
 * popped), so that one chunk's workgroups fill the CUs another leaves idle.  Each call starts at the 64-aligned
 * position at or below its first query; the ancestor rows below it are
 * recomputed (with a zero upstream gradient in the backward: "pad rows",
 * counted in tt_path_info), so results equal tree mode (tree_attn_fwd/bwd)
 * up to the order of floating-point sums.
 *
 * tree_path_build
 *   tree    built tree; must outlive the path object
 *   chunk   queries per backward call, a positive multiple of 64 (Key
 *           Contributions 2 gives 2048 as the default and 4096 as the
 *           faster setting)
 *   order   child visiting order: 0 = DFS (ascending token id); 1 = greedy:
 *           a node's last child is the one whose chain of last descendants
 *           is shortest (children by descending chain length, ties in DFS
 *           order), so short segments extend their parent's backward round
 *           instead of forming short rounds of their own (AReaL-DTA, Key
 *           Contributions 2 names a greedy DFS ordering that avoids short
 *           backward steps without defining it; this is that reading)
 *   out     receives the path object; free with tree_path_free
 * Errors: TT_EINVAL (NULL, chunk, order), TT_ENOMEM.  Host only.
 */
typedef struct tt_path tt_path;

typedef struct {
  int32_t n_segments;
  int32_t max_path;      /* longest root-to-leaf path in rows (max depth + 1): the stack size */
  int32_t chunk, order;
  int64_t fwd_calls;     /* attention calls of the forward rounds (one per round) */
  int64_t bwd_calls;     /* attention calls of the backward rounds */
  int64_t pad_rows;      /* ancestor query rows recomputed by all calls (64-alignment of a round's first call) */
  int64_t query_rows;    /* query rows all calls compute: 2 N + pad_rows */
  int64_t pad_pairs;     /* visible (query, key) pairs per head of the pad rows: recompute cost */
} tt_path_info;

int tree_path_build(const tt_tree* tree, int32_t chunk, int32_t order, tt_path** out);
void tree_path_free(tt_path* path);
int tree_path_info(const tt_path* path, tt_path_info* out);

/* Copies the segment table and the walk into caller-owned HOST arrays (NULL
 * members skipped): row0, len, depth0, parent (-1 at a root) [n_segments];
 * events [2 n_segments], e >= 0 entering segment e, e < 0 leaving -1 - e. */
int tree_path_segments(const tt_path* path, int32_t* row0, int32_t* len, int32_t* depth0, int32_t* parent,
                       int32_t* events);

/*
 * tree_attn_path -- forward (d_o == NULL) or forward then backward of one
 * layer, walked as above.  In the combined call each segment's backward runs
 * when the walk leaves it, as in the pages' push-pop execution.
 *   path          from tree_path_build
 *   h_q, h_kv, d, dtype, scale, rope_base   as in tt_attn_args
 *   q, k, v       [N,h_q,d], [N,h_kv,d], [N,h_kv,d] tree rows (DFS order)
 *   o, lse        [N,h_q,d], [N,h_q] outputs, written for every row
 *   d_o           [N,h_q,d] upstream gradient, or NULL for forward only
 *   d_q, d_k, d_v [N,h_q,d], [N,h_kv,d], [N,h_kv,d] outputs in dtype,
 *                 overwritten (ignored when d_o is NULL)
 *   plan          from tree_path_plan_upload for this path
 *   workspace     tree_path_workspace_bytes bytes, 256-byte aligned: the
 *                 stack (Q, K, V, O, LSE and, with d_o, float32 dK, dV: two
 *                 sets where chunk calls share a launch) of max_path
 *                 positions (bf16 head dim 128: also each position's tree
 *                 row and a (cos, sin) table) plus per-call buffers of
 *                 chunk + 64 rows; proportional to the longest path, not N
 * Errors: TT_EINVAL, TT_EUNSUPPORTED, TT_EWORKSPACE, TT_EOVERFLOW, TT_EDEVICE.
 */
typedef struct {
  const tt_path* path;
  const void* plan;        /* device plan of the walk, filled once by tree_path_plan_upload */
  int32_t h_q, h_kv, d;
  tt_dtype dtype;
  float scale;
  float rope_base;
  const void *q, *k, *v;
  void* o;
  float* lse;
  const void* d_o;
  void *d_q, *d_k, *d_v;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;          /* 0 or TT_ALLOW_GENERIC */
} tt_path_args;

/* The walk's device plan: the schedule of one chain of max_path rows, which
 * serves every attention call of the walk (stack position = depth).  Upload it
 * once per path object (hipMemcpyAsync on `stream`, like tree_plan_upload);
 * tree_attn_path then copies nothing from the host.
 * Errors: TT_EINVAL, TT_EWORKSPACE (buffer too small), TT_EDEVICE. */
int tree_path_plan_bytes(const tt_path* path, size_t* bytes);
int tree_path_plan_upload(const tt_path* path, void* dev_plan, size_t bytes, tt_stream stream);

int tree_path_workspace_bytes(const tt_path_args* args, size_t* bytes);
int tree_attn_path(const tt_path_args* args, tt_stream stream);

/*
 * Kernel timing (diagnostics).  While enabled on the calling thread, every
 * kernel this library launches from that thread is bracketed by two HIP
 * events recorded on the launch stream.  tt_timing_collect waits for the
 * recorded events, returns per kernel name the launch count, total and
 * maximum duration, and clears the record.  Events are created on first use
 * and reused; no device memory is allocated.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
  double max_ms;
} tt_kernel_time;

int tt_timing_enable(int on);
int tt_timing_collect(tt_kernel_time* out, int capacity, int* count);

/*
 * Matrix-core throughput probe (measurement).  Launches n_blocks workgroups
 * of 512 threads on `stream`; every wave issues iters * 32 dense
 * 32x32x16 bf16 MFMAs on register operands.  `out` is a caller-owned device
 * buffer of n_blocks * 512 floats (overwritten with per-thread sums); *flops
 * receives the launch's FLOP count, so flops / elapsed time is the sustained
 * bf16 MFMA rate, clock throttling included.  n_blocks in [1, 65536], iters
 * in [1, 2^20]; TT_EINVAL otherwise (nothing launched), TT_EDEVICE if the
 * launch fails.
 */
int tt_probe_mfma(int32_t n_blocks, int32_t iters, float* out, tt_stream stream, double* flops);

/* Text of the last error on this thread ("" if none). Valid until the next call. */
const char* tt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TT_H */
