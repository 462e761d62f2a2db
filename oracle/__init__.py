"""Plain fp64 CPU oracle for prefix-tree attention and the weighted tree loss.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this package.  It never imports
the HIP library, torch, or anything from the product package, and the product
never imports it.

What it computes, and where the pages define it:

* tree.py      -- the unique prefixes of the input sequences in lexicographic
                  DFS order, with depth, subtree end, parent, pass counts and
                  branch-fraction weights (Tree Training, Abstract: DFS
                  serialization visits each token once, and each token's loss
                  weight is the fraction of branches through it; AReaL-DTA
                  summary, Key Contributions 3: lexicographic DFS order).
* attention.py -- attention computed per branch: every input sequence is
                  linearised and run through textbook causal attention on its
                  own (Tree Training, Abstract: tree log-probabilities must
                  equal independent per-branch computation).  The tree result
                  of a row is its value in any branch through it; the tree
                  gradient of a row is the sum over its copies.
* nll.py       -- the loss averaged over branches, and the equal per-token
                  weighted loss (Tree Training, Abstract), plus the lm-head
                  product and its gradients.
* schedule.py  -- the set of non-empty (query-block, key-block) tiles by
                  enumeration of every visible pair.
* metrics.py   -- compression and pair counts (AReaL-DTA summary, Main
                  Findings 1).

Every function is pinned by tests that do not reuse its code (brute force on
tiny inputs, closed forms, identities the pages state, finite differences);
none of it is "parity unpinned".
"""
