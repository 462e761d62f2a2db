"""Non-empty tiles of the tree attention, by enumerating every (query, key) pair.

Visibility (the only rule that reproduces per-branch attention, Tree Training,
Abstract): key row j is seen by query row i iff j is i or an ancestor of i.
Here that is decided by walking parent pointers, not from subtree ends.

A tile (qb, kb) covers query rows [qb*bq, qb*bq+bq) and key rows
[kb*bk, kb*bk+bk), both cut at N.  It is listed if any pair in it is
visible, and flagged FULL if every pair of real rows in it is visible and the
key block is complete (no key row past N).
"""
import numpy as np


def visible_matrix(parent):
    N = len(parent)
    vis = np.zeros((N, N), dtype=bool)
    for i in range(N):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = int(parent[j])
    return vis


def tiles(parent, bq, bk):
    """Dict {(qb, kb): full_flag} of non-empty tiles."""
    N = len(parent)
    vis = visible_matrix(parent)
    out = {}
    nqb = (N + bq - 1) // bq
    nkb = (N + bk - 1) // bk
    for qb in range(nqb):
        i0, i1 = qb * bq, min(N, qb * bq + bq)
        for kb in range(nkb):
            j0, j1 = kb * bk, min(N, kb * bk + bk)
            sub = vis[i0:i1, j0:j1]
            if sub.any():
                out[(qb, kb)] = bool(sub.all()) and (j1 - j0 == bk)
    return out
