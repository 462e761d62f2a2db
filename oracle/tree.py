"""DFS serialization of the prefix tree of a set of token sequences (fp64/int oracle).

Definition followed (Tree Training, Abstract; AReaL-DTA summary, Key
Contributions 3 and Methodology):

* the tree's tokens are the distinct non-empty prefixes p of the input
  sequences -- a shared opening appears once, branches split where sequences
  diverge;
* the DFS index of p is its rank in lexicographic order of those prefixes
  (a proper prefix sorts before its extensions), i.e. preorder with children
  in ascending token id;
* depth(p) = |p| - 1, parent(p) = index of p[:-1] (or -1 for |p| = 1),
  end(p) = index(p) + number of prefixes extending p (p included),
  n_pass(p) = number of input sequences, with multiplicity, that start with p,
  weight(p) = float32(n_pass(p) / B) with B the number of input sequences.

How the order is produced: sort the sequences lexicographically; walking them
in that order, sequence s_i contributes exactly its prefixes longer than its
longest common prefix with s_{i-1}, shortest first.  Every such prefix is
larger than all prefixes contributed before it (they share s_i's first
lcp tokens and then either end or are smaller at position lcp), so the
emission order is the lexicographic order.  Plain Python; no trie.
"""
import numpy as np


def _lcp(a, b):
    n = min(len(a), len(b))
    i = 0
    while i < n and a[i] == b[i]:
        i += 1
    return i


def dfs_arrays(seqs):
    """Return a dict with the DFS arrays of the prefix tree of `seqs`.

    Keys: N, B, token, depth, parent, end, n_pass (int64 arrays), weight
    (float32), seq_pos_to_dfs (int64 [sum |s|], input order), tgt_row_ptr
    (int64 [N+1]), tgt_dfs (children of each row, ascending), n_roots,
    n_leaves, max_depth.
    """
    B = len(seqs)
    tups = [tuple(int(t) for t in s) for s in seqs]
    order = sorted(range(B), key=lambda b: tups[b])
    token, depth, parent = [], [], []
    nodes_of = [None] * B
    prev, prev_nodes = None, []
    for b in order:
        s = tups[b]
        l = _lcp(prev, s) if prev is not None else 0
        nodes = list(prev_nodes[:l])
        for k in range(l, len(s)):
            idx = len(token)
            token.append(s[k])
            depth.append(k)
            parent.append(nodes[k - 1] if k > 0 else -1)
            nodes.append(idx)
        nodes_of[b] = nodes
        prev, prev_nodes = s, nodes
    N = len(token)
    token = np.array(token, dtype=np.int64)
    depth = np.array(depth, dtype=np.int64)
    parent = np.array(parent, dtype=np.int64)

    # subtree sizes and pass counts, accumulated child -> parent in reverse DFS order
    size = np.ones(N, dtype=np.int64)
    n_pass = np.zeros(N, dtype=np.int64)
    for b in range(B):
        if len(nodes_of[b]):
            n_pass[nodes_of[b][-1]] += 1
    for i in range(N - 1, -1, -1):
        p = parent[i]
        if p >= 0:
            size[p] += size[i]
            n_pass[p] += n_pass[i]
    idx = np.arange(N, dtype=np.int64)
    end = idx + size
    weight = (n_pass.astype(np.float64) / float(B)).astype(np.float32) if B else np.zeros(0, np.float32)

    seq_pos = np.array([n for b in range(B) for n in nodes_of[b]], dtype=np.int64)

    children = [[] for _ in range(N)]
    for i in range(N):
        if parent[i] >= 0:
            children[parent[i]].append(i)
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    for i in range(N):
        row_ptr[i + 1] = row_ptr[i] + len(children[i])
    tgt = np.array([c for i in range(N) for c in children[i]], dtype=np.int64)

    n_roots = int(np.sum(parent < 0))
    n_leaves = int(np.sum(end == idx + 1))
    return dict(N=N, B=B, token=token, depth=depth, parent=parent, end=end,
                n_pass=n_pass, weight=weight, seq_pos_to_dfs=seq_pos,
                nodes_of=nodes_of, tgt_row_ptr=row_ptr, tgt_dfs=tgt,
                n_roots=n_roots, n_leaves=n_leaves,
                max_depth=int(depth.max()) if N else -1)


def branch_rows(tree, which="all"):
    """Row lists of the branches the per-branch computations run over.

    which="all": every input sequence, with multiplicity (empty ones skipped).
    which="leaves": one sequence per leaf of the tree (the distinct maximal
    sequences); together they still cover every row.
    """
    nodes_of = tree["nodes_of"]
    if which == "all":
        return [np.array(n, dtype=np.int64) for n in nodes_of if len(n)]
    seen = set()
    out = []
    end = tree["end"]
    for n in nodes_of:
        if not len(n):
            continue
        t = n[-1]
        if end[t] == t + 1 and t not in seen:
            seen.add(t)
            out.append(np.array(n, dtype=np.int64))
    return out
