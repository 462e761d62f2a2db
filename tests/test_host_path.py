"""Host side of path mode (tree_path_build), CPU only.

The walk plan is checked against the tree's own parent/child structure taken
from the oracle's DFS arrays:
* segments partition the rows in DFS order, each is a chain (every row but
  the last has exactly one child, which is the next row), and no two adjacent
  segments could be merged (maximality);
* a segment's parent is the segment holding its first row's parent;
* the events are a depth-first walk: each segment entered once, left once,
  children entered while their parent is on the stack, stack depth in rows
  never above max_path = max depth + 1;
* order 0 visits children by ascending first row; order 1 by descending
  length of the chain of last descendants (recomputed here from the walk
  itself), ties by first row;
* rounds are the maximal runs of enters and of leaves, each covering the
  stack positions of its segments; a forward round is one call, a backward
  round one call per chunk (boundaries at multiples of the chunk); each call
  starts at the 64-aligned position at or below its first query, which sets
  the pad-row counts.
"""
import numpy as np
import pytest

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle.tree import dfs_arrays


def _expected_segments(o):
    N = o["N"]
    nchild = np.bincount(o["parent"][o["parent"] >= 0], minlength=N) if N else np.zeros(0, np.int64)
    starts = [i for i in range(N) if not (i > 0 and o["parent"][i] == i - 1 and nchild[i - 1] == 1)]
    return starts, nchild


def _check(seqs, chunk, order):
    t = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    p = tt.Path(t, chunk, order)
    s = p.segments()
    inf = p.info
    N = o["N"]
    S = inf["n_segments"]
    starts, nchild = _expected_segments(o)
    assert S == len(starts)
    np.testing.assert_array_equal(s["row0"], starts)
    ends = list(starts[1:]) + [N]
    np.testing.assert_array_equal(s["len"], np.diff(starts + [N]) if N else [])
    seg_of = np.zeros(N, dtype=np.int64)
    for k, (a, b) in enumerate(zip(starts, ends)):
        seg_of[a:b] = k
        for r in range(a + 1, b):  # a chain: r's parent is r-1, whose only child is r
            assert o["parent"][r] == r - 1 and nchild[r - 1] == 1
        assert s["depth0"][k] == o["depth"][a]
        np.testing.assert_array_equal(o["depth"][a:b], o["depth"][a] + np.arange(b - a))
        par = o["parent"][a]
        assert s["parent"][k] == (-1 if par < 0 else seg_of[par])
        if par >= 0:
            assert par == ends[s["parent"][k]] - 1  # attaches at its parent segment's last row
    assert inf["max_path"] == (o["max_depth"] + 1 if N else 0)
    # the walk
    ev = s["events"]
    assert len(ev) == 2 * S
    entered, left, stack, rows_on_stack = set(), set(), [], 0
    kids_seen = {}
    for e in ev:
        if e >= 0:
            assert e not in entered
            par = s["parent"][e]
            assert (par < 0 and not stack) or (stack and stack[-1] == par)
            kids_seen.setdefault(par, []).append(e)
            entered.add(e)
            stack.append(e)
            rows_on_stack += s["len"][e]
            assert rows_on_stack == s["depth0"][e] + s["len"][e] <= inf["max_path"]
        else:
            k = -1 - e
            assert stack and stack[-1] == k and k not in left
            left.add(k)
            stack.pop()
            rows_on_stack -= s["len"][k]
    assert not stack and len(entered) == len(left) == S
    chain = {}

    def chain_len(k):  # own length plus the chain of its last child in the walk
        if k not in chain:
            kids = kids_seen.get(k, [])
            chain[k] = s["len"][k] + (chain_len(kids[-1]) if kids else 0)
        return chain[k]

    for par, kids in kids_seen.items():
        want = sorted(kids, key=lambda k: s["row0"][k])
        if order == 1:
            want = sorted(want, key=lambda k: -chain_len(k))  # stable: ties stay in row order
        assert kids == want
    # rounds and chunk accounting
    calls = {False: 0, True: 0}
    pad = pad_pairs = 0
    i = 0
    while i < len(ev):
        bwd = ev[i] < 0
        j = i
        while j < len(ev) and (ev[j] < 0) == bwd:
            j += 1
        segs = [(-1 - e if bwd else e) for e in ev[i:j]]
        lo = min(s["depth0"][k] for k in segs)
        hi = max(s["depth0"][k] + s["len"][k] for k in segs)
        assert hi - lo == sum(s["len"][k] for k in segs)   # stacked one on the next
        c0 = lo
        while c0 < hi:  # a forward round is one call, a backward round one call per chunk
            calls[bwd] += 1
            pad += c0 % 64
            pad_pairs += sum(r + 1 for r in range(c0 - c0 % 64, c0))  # a pad row at position r sees r + 1 keys
            c0 = min(hi, (c0 // chunk + 1) * chunk) if bwd else hi
        i = j
    leaves = sum(1 for k in range(S) if k not in kids_seen)
    assert inf["fwd_calls"] == calls[False] and inf["bwd_calls"] == calls[True]
    assert calls[False] == leaves and calls[True] >= leaves
    assert inf["pad_rows"] == pad and inf["query_rows"] == 2 * N + pad
    assert inf["pad_pairs"] == pad_pairs
    return p


@pytest.mark.parametrize("case", range(12))
def test_path_plan_random(case):
    rng = np.random.default_rng(100 + case)
    seqs = ts.trees.random_small_tree(seed=100 + case, n_seqs=int(rng.integers(1, 12)), max_len=90, vocab=5,
                                      p_dup=0.2, p_prefix=0.3).seqs
    for chunk in (64, 128):
        for order in (0, 1):
            _check(seqs, chunk, order)


def test_path_plan_workloads_and_edges():
    _check(ts.trees.tiny_tree().seqs, 64, 0)
    _check(ts.trees.tiny_tree().seqs, 2048, 1)
    _check([list(range(300))], 128, 0)       # one chain: one segment, ceil chunks
    _check([[1], [2], [3]], 64, 0)           # three one-row roots
    _check([[5, 6], [5, 6], [5]], 64, 1)     # duplicates and a contained prefix
    _check([], 64, 0)                        # empty tree
    _check([[]], 64, 0)                      # one empty sequence


def test_path_plan_c2_shape():
    """The 8B-shape agentic tree: the walk's stack never exceeds the longest path."""
    tree = ts.trees.agentic_beam_tree(seed=0)
    p = _check(tree.seqs, 2048, 0)
    assert p.info["max_path"] == max(len(s) for s in tree.seqs)


def test_path_build_errors():
    lib = tt.lib()
    t = tt.Tree([[1, 2, 3]])
    import ctypes
    h = ctypes.c_void_p()
    for chunk, order in ((0, 0), (100, 0), (-64, 0), (64, 2), (64, -1)):
        assert lib.tree_path_build(t.handle, chunk, order, ctypes.byref(h)) == tt.TT_EINVAL
        assert tt.last_error()
    assert lib.tree_path_build(None, 64, 0, ctypes.byref(h)) == tt.TT_EINVAL
    assert lib.tree_path_build(t.handle, 64, 0, None) == tt.TT_EINVAL
    assert lib.tree_path_info(None, None) == tt.TT_EINVAL
    assert lib.tree_path_segments(None, None, None, None, None, None) == tt.TT_EINVAL
    p = tt.Path(t, 64, 0)
    args = tt.PathArgs(path=p.handle, h_q=2, h_kv=1, d=128, dtype=tt.TT_BF16)
    n = ctypes.c_size_t()
    assert lib.tree_path_workspace_bytes(ctypes.byref(args), ctypes.byref(n)) == tt.TT_OK and n.value > 0
    # the device entry point validates before touching the device
    bad = [dict(h_q=3, h_kv=2), dict(d=100), dict(d=0), dict(dtype=7), dict(scale=-1.0),
           dict(rope_base=float("inf"))]
    for kw in bad:
        a = tt.PathArgs(path=p.handle, h_q=2, h_kv=1, d=128, dtype=tt.TT_BF16)
        for key, val in kw.items():
            setattr(a, key, val)
        assert lib.tree_attn_path(ctypes.byref(a), None) < 0, kw
    a = tt.PathArgs(path=p.handle, h_q=2, h_kv=1, d=128, dtype=tt.TT_BF16)  # q, k, v, o, lse missing
    assert lib.tree_attn_path(ctypes.byref(a), None) == tt.TT_EINVAL
    assert lib.tree_attn_path(None, None) == tt.TT_EINVAL
    # every buffer given, but no plan / a plan the library never filled / bf16 head dim 64
    F = 0x100000
    full = dict(path=p.handle, h_q=2, h_kv=1, d=128, dtype=tt.TT_BF16, q=F, k=F, v=F, o=F, lse=F, workspace=F,
                workspace_bytes=1 << 40)
    a = tt.PathArgs(**full)
    assert lib.tree_attn_path(ctypes.byref(a), None) == tt.TT_EINVAL and "plan is NULL" in tt.last_error()
    a = tt.PathArgs(plan=F, **full)
    assert lib.tree_attn_path(ctypes.byref(a), None) == tt.TT_EINVAL and "upload" in tt.last_error()
    a = tt.PathArgs(plan=F, **dict(full, d=64))
    assert lib.tree_attn_path(ctypes.byref(a), None) == tt.TT_EUNSUPPORTED
    a = tt.PathArgs(plan=F, flags=tt.TT_ALLOW_GENERIC, **dict(full, d=64))
    assert lib.tree_attn_path(ctypes.byref(a), None) == tt.TT_EINVAL and "upload" in tt.last_error()
    # the walk's plan is the chain of the longest path (host copy size)
    assert p.plan_bytes() > 0 and p.plan_bytes() % 256 == 0


def _path_ws_expected(L, chunk, hq, hk, d, es, bwd, slots, mfma):
    """The walk's workspace as tree_attn_path documents it: the stack of L
    positions (Q, K, V, O in the data type, LSE fp32; on the matrix cores also
    an int32 tree row and the (cos, sin) table entry per position) and, with a
    backward, `slots` sets of fp32 dK/dV accumulators, dO copies, D and (matrix
    cores) bf16 dQ blocks of chunk + 64 rows, and one fp32 dQ block; every
    buffer 256-byte aligned."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    C = chunk + 64
    n = al(L * hq * d * es) + 2 * al(L * hk * d * es) + al(L * hq * d * es) + al(L * hq * 4)
    if mfma:
        n += al(L * 4) + al(L * (d // 2) * 8)
    if bwd:
        n += 2 * slots * al(L * hk * d * 4) + slots * al(C * hq * d * es) + slots * al(C * hq * 4)
        n += al(C * hq * d * 4)
        if mfma:
            n += slots * al(C * hq * d * 2)
    return n


@pytest.mark.parametrize("hq,hk,d,dtype,chunk,slots", [(8, 2, 128, "bf16", 128, 3), (32, 8, 128, "bf16", 2048, 3),
                                                       (32, 8, 128, "bf16", 4096, 2), (4, 2, 128, "bf16", 128, 3),
                                                       (16, 8, 128, "bf16", 4096, 2), (2, 1, 128, "bf16", 128, 1),
                                                       (6, 2, 128, "bf16", 128, 1), (2, 2, 128, "bf16", 128, 1),
                                                       (8, 2, 64, "bf16", 128, 1), (8, 2, 64, "f32", 128, 1)])
def test_path_workspace_slots(hq, hk, d, dtype, chunk, slots):
    """Matrix-core walks whose backward runs as one launch (groups of a
    multiple of 4 heads, or of 2 over an even number of kv heads) hold several
    sets of per-call buffers and accumulators (three chunks per backward
    launch up to chunks of 2048 rows, two above); other shapes one."""
    import ctypes
    case = ts.random_small_tree(3, n_seqs=6, max_len=300, vocab=3)
    t = tt.Tree(case.seqs)
    p = tt.Path(t, chunk, 0)
    L = p.info["max_path"]
    dt = tt.TT_BF16 if dtype == "bf16" else tt.TT_F32
    es = 2 if dtype == "bf16" else 4
    for bwd in (False, True):
        args = tt.PathArgs(path=p.handle, h_q=hq, h_kv=hk, d=d, dtype=dt, d_o=0x100000 if bwd else None)
        n = ctypes.c_size_t()
        assert tt.lib().tree_path_workspace_bytes(ctypes.byref(args), ctypes.byref(n)) == tt.TT_OK
        mfma = dtype == "bf16" and d == 128
        assert n.value == _path_ws_expected(L, chunk, hq, hk, d, es, bwd, slots, mfma), (bwd, n.value)
