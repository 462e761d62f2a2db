"""Pins for oracle/tree.py, oracle/metrics.py and oracle/schedule.py (CPU only).

Each check is independent of the oracle's own code path: brute force over
explicit prefix tuples, closed forms of the tiny tree, invariants, and the
pages' printed compression arithmetic.
"""
import json
import os

import numpy as np
import pytest

import treesynth as ts
from oracle.tree import dfs_arrays, branch_rows
from oracle.metrics import metrics
from oracle.schedule import tiles

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force(seqs):
    """DFS arrays straight from the definition: set of prefix tuples, sorted."""
    pref = set()
    for s in seqs:
        t = tuple(int(x) for x in s)
        for k in range(1, len(t) + 1):
            pref.add(t[:k])
    order = sorted(pref)
    idx = {p: i for i, p in enumerate(order)}
    N = len(order)
    B = len(seqs)
    token = np.array([p[-1] for p in order], dtype=np.int64)
    depth = np.array([len(p) - 1 for p in order], dtype=np.int64)
    parent = np.array([idx[p[:-1]] if len(p) > 1 else -1 for p in order], dtype=np.int64)
    end = np.array([i + sum(1 for q in order if q[:len(p)] == p) for i, p in enumerate(order)],
                   dtype=np.int64)
    n_pass = np.array([sum(1 for s in seqs if tuple(int(x) for x in s[:len(p)]) == p)
                       for p in order], dtype=np.int64)
    seq_pos = np.array([idx[tuple(int(x) for x in s[:k + 1])] for s in seqs for k in range(len(s))],
                       dtype=np.int64)
    return dict(N=N, B=B, token=token, depth=depth, parent=parent, end=end, n_pass=n_pass,
                seq_pos_to_dfs=seq_pos)


CASES = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=v, p_empty=pe)
         for s, (n, L, v, pe) in enumerate(
             [(1, 1, 3, 0.0), (1, 30, 5, 0.0), (5, 20, 3, 0.0), (8, 40, 4, 0.1),
              (12, 25, 2, 0.2), (3, 60, 50, 0.0), (20, 12, 3, 0.1), (6, 33, 6, 0.0)] * 4)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c.seed}")
def test_dfs_matches_prefix_sort_bruteforce(case):
    seqs = case.seqs
    a = dfs_arrays(seqs)
    b = brute_force(seqs)
    assert a["N"] == b["N"]
    for key in ("token", "depth", "parent", "end", "n_pass", "seq_pos_to_dfs"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    # weight = n_pass / B rounded once to float32 (both rows of integers are exact)
    if b["B"]:
        w = np.array([np.float32(n / b["B"]) for n in b["n_pass"]], dtype=np.float32)
        np.testing.assert_array_equal(a["weight"], w)


@pytest.mark.parametrize("case", CASES[:16], ids=lambda c: f"seed{c.seed}")
def test_dfs_invariants(case):
    a = dfs_arrays(case.seqs)
    N = a["N"]
    idx = np.arange(N)
    assert np.all(idx < a["end"]) and np.all(a["end"] <= N)
    # subtree ranges nest: a child's range lies inside its parent's
    for i in range(N):
        p = a["parent"][i]
        if p >= 0:
            assert p < i and a["end"][i] <= a["end"][p]
            assert a["depth"][i] == a["depth"][p] + 1
    roots = a["parent"] < 0
    nonempty = sum(1 for s in case.seqs if len(s))
    assert int(a["n_pass"][roots].sum()) == nonempty
    # targets CSR: the children of row r, ascending
    for r in range(N):
        kids = a["tgt_dfs"][a["tgt_row_ptr"][r]:a["tgt_row_ptr"][r + 1]]
        assert list(kids) == [i for i in range(N) if a["parent"][i] == r]
    # leaves-only branches still cover every row
    cover = np.zeros(N, dtype=int)
    for rows in branch_rows(a, "leaves"):
        cover[rows] += 1
    assert N == 0 or cover.min() >= 1


def test_tiny_tree_closed_forms():
    """Closed forms of the tiny tree: 64-token root, four 32-token children,
    child 0 split into two 16-token leaves; B = 5 leaf sequences."""
    t = ts.tiny_tree(0)
    a = dfs_arrays(t.seqs)
    assert a["N"] == 64 + 4 * 32 + 2 * 16 == 224
    assert a["B"] == 5 and a["n_leaves"] == 5 and a["n_roots"] == 1
    assert a["max_depth"] == 64 + 32 + 16 - 1
    vals, counts = np.unique(a["weight"], return_counts=True)
    got = {round(float(v), 6): int(c) for v, c in zip(vals, counts)}
    # root: all 5 sequences; child 0's 32 tokens: 2 of 5; everything else: 1 of 5
    assert got == {1.0: 64, 0.4: 32, 0.2: 128}
    # sum of target weights = sum over sequences of (|s| - 1) / B
    w_targets = float(np.sum(a["n_pass"][a["parent"] >= 0])) / 5
    assert abs(w_targets - (2 * 111 + 3 * 95) / 5) < 1e-12 and abs(w_targets - 101.4) < 1e-12
    m = metrics(t.seqs, a)
    assert m["seq_tokens"] == 2 * 112 + 3 * 96 == 512
    # visible pairs per head: each row sees depth+1 keys
    root = 64 * 65 // 2
    child = sum(64 + k for k in range(1, 33))       # a 32-token child at depths 64..95
    leaf = sum(96 + k for k in range(1, 17))        # a 16-token leaf at depths 96..111
    assert m["pairs"] == root + 4 * child + 2 * leaf == 15728
    assert m["dense_pairs"] == 2 * (112 * 113 // 2) + 3 * (96 * 97 // 2) == 26624


def test_pages_compression_arithmetic():
    """The page's printed sharing percentages follow from the printed
    compression rates through sharing = 1 - 1/compression."""
    g = json.load(open(os.path.join(GOLDEN, "pages_compression.json")))
    for c in g["cases"]:
        assert round(100.0 * (1.0 - 1.0 / c["compression"]), 1) == c["sharing_percent"]
    # and the oracle's metric uses exactly that relation
    t = ts.tiny_tree(0)
    m = metrics(t.seqs, dfs_arrays(t.seqs))
    assert abs(m["sharing"] - (1.0 - 1.0 / m["compression"])) < 1e-15


def test_metrics_bruteforce():
    for case in CASES[:10]:
        a = dfs_arrays(case.seqs)
        m = metrics(case.seqs, a)
        distinct = {tuple(int(x) for x in s) for s in case.seqs if len(s)}
        maximal = [s for s in distinct if not any(o != s and o[:len(s)] == s for o in distinct)]
        assert m["leaf_tokens"] == sum(len(s) for s in maximal)
        assert m["pairs"] == sum(len(p) for p in
                                 {tuple(int(x) for x in s[:k]) for s in case.seqs
                                  for k in range(1, len(s) + 1)})


def test_schedule_special_cases():
    # one chain: block lower triangle, strictly-below-diagonal blocks FULL
    chain = dfs_arrays([np.arange(20) % 7])
    t = tiles(chain["parent"], 4, 4)
    assert set(t) == {(qb, kb) for qb in range(5) for kb in range(qb + 1)}
    assert all(t[(qb, kb)] == (kb < qb) for (qb, kb) in t)
    # single-token sequences: every row sees only itself -> diagonal, never FULL
    star = dfs_arrays([np.array([i]) for i in range(10)])
    t = tiles(star["parent"], 4, 4)
    assert set(t) == {(0, 0), (1, 1), (2, 2)} and not any(t.values())
    # ragged key block at the end is never FULL
    chain = dfs_arrays([np.arange(18) % 5])
    t = tiles(chain["parent"], 4, 4)
    assert t[(4, 3)] is True and t[(4, 4)] is False
