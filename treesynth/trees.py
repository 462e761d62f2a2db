"""Synthetic rollout trees.

Each generator grows its own tree of token *segments*: a segment is a run of
tokens hanging under a parent segment, sibling segments start with distinct
token ids, and every sequence is the concatenation of the segments on a
root-to-node chain.  The construction therefore knows its own unique-token
count (the total length of the segments in use); it never derives it from the
sequences.  Token ids are uniform over the vocabulary.

The shapes follow the workloads of the pages: multi-turn agent rollouts whose
calls contain one another (AReaL-DTA, Main Findings on compression: about
9.4x total and 5.6x leaves-only), 16K-context agentic trees at the 8B scale
(AReaL-DTA, Methodology: 16K context), one long root-to-leaf path processed in
fixed chunks (AReaL-DTA, Key Contributions 2), and a tiny tree for exact
checks.
"""
from dataclasses import dataclass, field
from typing import List, Dict, Any

import numpy as np

from .tensors import rng_for


@dataclass
class SynthTree:
    name: str
    seqs: List[np.ndarray]            # int32 token ids, one array per input sequence
    vocab: int
    n_unique: int                     # unique tokens known from the construction
    seed: int
    params: Dict[str, Any] = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return len(self.seqs)

    @property
    def seq_tokens(self) -> int:
        return int(sum(len(s) for s in self.seqs))

    def flat(self):
        """(tokens int32 [sum |s|], offsets int64 [B+1]) in input order."""
        offs = np.zeros(len(self.seqs) + 1, dtype=np.int64)
        for i, s in enumerate(self.seqs):
            offs[i + 1] = offs[i] + len(s)
        toks = (np.concatenate([np.asarray(s, dtype=np.int32) for s in self.seqs])
                if self.seqs else np.zeros(0, dtype=np.int32))
        return toks.astype(np.int32), offs


class _SegTree:
    """Book-keeping of the generator's own segments."""

    def __init__(self):
        self.parent: List[int] = []
        self.toks: List[np.ndarray] = []
        self.alive: List[bool] = []

    def add(self, parent: int, toks: np.ndarray) -> int:
        assert len(toks) >= 1
        self.parent.append(parent)
        self.toks.append(np.asarray(toks, dtype=np.int32))
        self.alive.append(True)
        return len(self.toks) - 1

    def chain(self, seg: int) -> List[int]:
        out = []
        while seg >= 0:
            out.append(seg)
            seg = self.parent[seg]
        return out[::-1]

    def seq(self, seg: int) -> np.ndarray:
        return np.concatenate([self.toks[s] for s in self.chain(seg)])

    def used_length(self, segs) -> int:
        return int(sum(len(self.toks[s]) for s in segs))


def _tokens(rng, n, vocab, first=None):
    t = rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)
    if first is not None and n > 0:
        t[0] = first
    return t


def _distinct_firsts(rng, k, vocab):
    return rng.choice(vocab, size=k, replace=False).astype(np.int32)


# ---------------------------------------------------------------- tiny tree
def tiny_tree(seed: int = 0) -> SynthTree:
    """Root segment of 64 tokens, four 32-token children, the first of which
    splits into two 16-token leaves: five leaves, 224 unique tokens, vocab 1000.

    Draw order: root tokens; the 4 distinct child first tokens; the 31 tail
    tokens of each child in order; the 2 distinct leaf first tokens; the 15
    tail tokens of each leaf.
    """
    V = 1000
    rng = rng_for(seed)
    st = _SegTree()
    root = st.add(-1, _tokens(rng, 64, V))
    firsts = _distinct_firsts(rng, 4, V)
    kids = [st.add(root, np.concatenate([[firsts[c]], _tokens(rng, 31, V)]).astype(np.int32))
            for c in range(4)]
    lf = _distinct_firsts(rng, 2, V)
    leaves = [st.add(kids[0], np.concatenate([[lf[c]], _tokens(rng, 15, V)]).astype(np.int32))
              for c in range(2)]
    ends = [leaves[0], leaves[1], kids[1], kids[2], kids[3]]
    seqs = [st.seq(e) for e in ends]
    return SynthTree("tiny", seqs, V, 64 + 4 * 32 + 2 * 16, seed,
                     dict(root=64, children=4, child_len=32, split_leaves=2, leaf_len=16))


# ---------------------------------------------------------------- RL forest
def rl_forest(seed: int, n_trees: int = 2, prompt: int = 2048, rollouts: int = 8,
              turns: int = 4, turn_len=(256, 1024), vocab: int = 151936) -> SynthTree:
    """Forest of multi-turn RL rollout trees.

    Each tree: a shared prompt, then `turns` turns.  At every turn each group
    of rollouts that still share their whole history splits into consecutive
    sub-groups of size U{1..8} (the last one capped); every sub-group gets one
    new segment of length U[turn_len].  The training sequences are the
    per-turn prefixes (prompt + turns 1..k) of every rollout, so a rollout's
    earlier calls are contained in its later ones and rollouts that share a
    turn contribute duplicate sequences.
    """
    rng = rng_for(seed)
    st = _SegTree()
    prompt_firsts = _distinct_firsts(rng, n_trees, vocab)
    seqs = []
    used = []
    for t in range(n_trees):
        root = st.add(-1, _tokens(rng, prompt, vocab, first=prompt_firsts[t]))
        used.append(root)
        groups = [(list(range(rollouts)), root)]
        seg_of = {}  # (rollout, turn) -> segment id
        for k in range(turns):
            new_groups = []
            for members, parent in groups:
                sizes = []
                left = len(members)
                while left > 0:
                    s = int(rng.integers(1, 9))
                    s = min(s, left)
                    sizes.append(s)
                    left -= s
                firsts = _distinct_firsts(rng, len(sizes), vocab)
                pos = 0
                for g, s in enumerate(sizes):
                    L = int(rng.integers(turn_len[0], turn_len[1] + 1))
                    seg = st.add(parent, _tokens(rng, L, vocab, first=firsts[g]))
                    used.append(seg)
                    sub = members[pos:pos + s]
                    pos += s
                    for r in sub:
                        seg_of[(r, k)] = seg
                    new_groups.append((sub, seg))
            groups = new_groups
        for r in range(rollouts):
            for k in range(turns):
                seqs.append(st.seq(seg_of[(r, k)]))
    return SynthTree("rl_forest", seqs, vocab, st.used_length(used), seed,
                     dict(n_trees=n_trees, prompt=prompt, rollouts=rollouts, turns=turns,
                          turn_len=list(turn_len)))


def rl_forest_accepted(start_seed: int = 0, target_comp=(9.0, 9.8),
                       target_n=(21600, 26400), max_tries: int = 10000) -> SynthTree:
    """First seed >= start_seed whose forest has compression (total sequence
    tokens / unique tokens) in target_comp and unique-token count in target_n."""
    for s in range(start_seed, start_seed + max_tries):
        t = rl_forest(s)
        comp = t.seq_tokens / t.n_unique
        if target_comp[0] <= comp <= target_comp[1] and target_n[0] <= t.n_unique <= target_n[1]:
            t.params["accepted_after"] = s - start_seed
            t.params["compression"] = comp
            return t
    raise RuntimeError("no accepted seed")


# ---------------------------------------------------------------- beam trees
def _beam(rng, st, root, vocab, turns, branch, width, seg_len):
    leaves = [root]
    for _ in range(turns):
        new = []
        for p in leaves:
            firsts = _distinct_firsts(rng, branch, vocab)
            for b in range(branch):
                L = int(rng.integers(seg_len[0], seg_len[1] + 1))
                new.append(st.add(p, _tokens(rng, L, vocab, first=firsts[b])))
        if len(new) > width:
            keep = np.sort(rng.choice(len(new), size=width, replace=False))
            keep_set = set(keep.tolist())
            for i in range(len(new)):
                if i not in keep_set:
                    st.alive[new[i]] = False
            new = [new[i] for i in keep]
        leaves = new
    return leaves


def _live_segments(st, leaves):
    segs = set()
    for lf in leaves:
        segs.update(st.chain(lf))
    return segs


def agentic_beam_tree(seed: int, root_len: int = 4096, turns: int = 10, branch: int = 2,
                      width: int = 16, seg_len=(512, 2048), n_max: int = 67200,
                      vocab: int = 151936) -> SynthTree:
    """Agentic tree: a root segment, then `turns` turns in which every live
    leaf branches into `branch` children (segments of length U[seg_len]) and
    a random subset of `width` leaves is kept.  Afterwards random leaves are
    dropped (with the segments only they used) until the unique-token count
    is at most n_max.  Sequences are the surviving root-to-leaf paths."""
    rng = rng_for(seed)
    st = _SegTree()
    root = st.add(-1, _tokens(rng, root_len, vocab))
    leaves = _beam(rng, st, root, vocab, turns, branch, width, seg_len)
    n_literal = st.used_length(_live_segments(st, leaves))
    while st.used_length(_live_segments(st, leaves)) > n_max and len(leaves) > 1:
        drop = int(rng.integers(0, len(leaves)))
        leaves = leaves[:drop] + leaves[drop + 1:]
    segs = _live_segments(st, leaves)
    seqs = [st.seq(lf) for lf in leaves]
    return SynthTree("agentic_beam", seqs, vocab, st.used_length(segs), seed,
                     dict(root_len=root_len, turns=turns, branch=branch, width=width,
                          seg_len=list(seg_len), n_max=n_max, n_before_drop=n_literal,
                          leaves=len(leaves)))


def long_chain(seed: int, length: int = 49152, vocab: int = 151936) -> SynthTree:
    """One root-to-leaf path of `length` tokens."""
    rng = rng_for(seed)
    return SynthTree("chain", [_tokens(rng, length, vocab)], vocab, length, seed,
                     dict(length=length))


def lmhead_tree(seed: int, leaves: int = 32, depth: int = 10, seg_len=(512, 2048),
                n_total: int = 16384, compression: float = 5.5,
                vocab: int = 151936) -> SynthTree:
    """A `leaves`-leaf beam tree (branch 2, width `leaves`, `depth` turns) whose
    segment lengths are then rescaled by one common factor s, and whose root
    length R is chosen, so that the unique-token count is exactly n_total and
    total sequence tokens / unique tokens is about `compression`.

    With E the sum of non-root segment lengths and A the sum over leaves of
    their path's non-root length: leaves*R + s*A = compression*n_total and
    R + s*E = n_total.  Rescaled lengths are rounded (at least 1) and the
    rounding remainder goes to the root."""
    rng = rng_for(seed)
    st = _SegTree()
    root = st.add(-1, np.zeros(1, dtype=np.int32))  # length fixed below
    lv = _beam(rng, st, root, vocab, depth, 2, leaves, seg_len)
    segs = sorted(_live_segments(st, lv) - {root})
    E = sum(len(st.toks[s]) for s in segs)
    A = sum(sum(len(st.toks[s]) for s in st.chain(lf) if s != root) for lf in lv)
    s = (compression * n_total - leaves * n_total) / (A - leaves * E)
    new_len = {g: max(1, int(round(s * len(st.toks[g])))) for g in segs}
    R = n_total - sum(new_len.values())
    assert R >= 1
    for g in segs:
        first = st.toks[g][0]
        st.toks[g] = _tokens(rng, new_len[g], vocab, first=first)
    st.toks[root] = _tokens(rng, R, vocab)
    seqs = [st.seq(lf) for lf in lv]
    return SynthTree("lmhead_tree", seqs, vocab, n_total, seed,
                     dict(leaves=leaves, depth=depth, seg_len=list(seg_len), scale=s,
                          root_len=R, target_compression=compression))


# ---------------------------------------------------------------- small random sets
def random_small_tree(seed: int, n_seqs: int = 6, max_len: int = 40, vocab: int = 7,
                      p_dup: float = 0.15, p_prefix: float = 0.2, p_empty: float = 0.0,
                      min_len: int = 1) -> SynthTree:
    """Small random sequence sets with heavy accidental sharing (tiny vocab),
    exact duplicates, sequences contained in others and, optionally, empty
    sequences.  The unique-token count is not known by construction here
    (n_unique = -1); such sets exercise the tree builder itself."""
    rng = rng_for(seed)
    seqs: List[np.ndarray] = []
    for _ in range(n_seqs):
        u = rng.random()
        if p_empty > 0 and rng.random() < p_empty:
            seqs.append(np.zeros(0, dtype=np.int32))
        elif seqs and u < p_dup:
            seqs.append(seqs[int(rng.integers(0, len(seqs)))].copy())
        elif seqs and u < p_dup + p_prefix:
            base = seqs[int(rng.integers(0, len(seqs)))]
            cut = int(rng.integers(0, len(base) + 1))
            seqs.append(base[:cut].copy() if cut >= min_len else base.copy())
        else:
            if seqs and rng.random() < 0.7:
                base = seqs[int(rng.integers(0, len(seqs)))]
                cut = int(rng.integers(0, len(base) + 1))
                ext = int(rng.integers(max(0, min_len - cut), max_len - cut + 1)) if max_len > cut else 0
                s = np.concatenate([base[:cut], _tokens(rng, ext, vocab)]).astype(np.int32)
            else:
                L = int(rng.integers(min_len, max_len + 1))
                s = _tokens(rng, L, vocab)
            seqs.append(s)
    return SynthTree("random_small", seqs, vocab, -1, seed,
                     dict(n_seqs=n_seqs, max_len=max_len, vocab=vocab))


# ---------------------------------------------------------------- nested shape
def nested_tree(seed: int, spec, vocab: int = 151936, name: str = "nested") -> SynthTree:
    """A tree of segments with given lengths: spec = (length, [child specs]).
    Every root-to-leaf chain of segments is one input sequence (leaves in the
    spec's order); sibling segments start with distinct token ids.

    Draw order: depth first through the spec -- a segment's tokens, then the
    distinct first tokens of its children, then each child in turn."""
    rng = rng_for(seed)
    st = _SegTree()
    ends = []

    def grow(parent, sp, first):
        length, kids = sp
        seg = st.add(parent, _tokens(rng, length, vocab, first=first))
        if not kids:
            ends.append(seg)
            return
        firsts = _distinct_firsts(rng, len(kids), vocab)
        for c, kid in enumerate(kids):
            grow(seg, kid, int(firsts[c]))

    grow(-1, spec, None)
    seqs = [st.seq(e) for e in ends]
    return SynthTree(name, seqs, vocab, st.used_length(range(len(st.toks))), seed, dict(spec=repr(spec)))
