"""Compression and attention-pair counts.

AReaL-DTA summary, Main Findings 1: compression is total sequence tokens over
unique tree tokens; the leaves-only figure counts each distinct maximal
sequence once (rollouts contained in others collapsed); sharing = 1 - 1/compression.
"""


def metrics(seqs, tree):
    depth = tree["depth"]
    end = tree["end"]
    N = tree["N"]
    seq_tokens = sum(len(s) for s in seqs)
    leaf_tokens = int(sum(int(depth[i]) + 1 for i in range(N) if end[i] == i + 1))
    pairs = int(sum(int(d) + 1 for d in depth))                       # visible (query, key) per head
    dense_pairs = int(sum(len(s) * (len(s) + 1) // 2 for s in seqs))  # causal pairs, every branch alone
    return dict(
        N=N, seq_tokens=seq_tokens, leaf_tokens=leaf_tokens,
        compression=seq_tokens / N if N else 0.0,
        leaf_compression=leaf_tokens / N if N else 0.0,
        sharing=1.0 - N / seq_tokens if seq_tokens else 0.0,
        pairs=pairs, dense_pairs=dense_pairs,
    )
