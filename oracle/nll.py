"""Weighted log-softmax NLL over the tree, and the same loss averaged over branches (fp64).

Tree Training, Abstract: the loss averaged over all branches, each branch
trained on its own, is the same number as a per-token weighted loss whose
weight is the fraction of branches passing through the token.

Readings (the pages are silent):
  * a branch is an input sequence, counted with multiplicity, B = #sequences;
  * a branch's loss is the SUM of its next-token NLLs, and the branch-averaged
    loss is (1/B) * sum over branches -- the only reading under which the
    identity is exact;
  * every non-root row t is a target, predicted from its parent's logits row:
    its token id x_t indexes the parent's vocabulary row, its weight is
    w_t = n_pass(t)/B.
"""
import numpy as np


def _lse(z):
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


def tree_loss(parent, token, weight, logits):
    """Per-token weighted loss over the tree's rows.

    parent/token: int arrays [N]; weight: [N] (w_t for target t); logits: [N,V].
    Returns (loss, logp [N] with nan at roots, dZ [N,V])."""
    z = np.asarray(logits, dtype=np.float64)
    lse = _lse(z)
    soft = np.exp(z - lse[:, None])
    N = len(parent)
    loss = 0.0
    logp = np.full(N, np.nan)
    dz = np.zeros_like(z)
    for t in range(N):
        r = int(parent[t])
        if r < 0:
            continue
        x = int(token[t])
        w = float(weight[t])
        lp = z[r, x] - lse[r]
        logp[t] = lp
        loss += -w * lp
        dz[r] += w * soft[r]
        dz[r, x] -= w
    return loss, logp, dz


def branch_loss(nodes_of, token, logits):
    """Loss averaged over branches: (1/B) * sum_s sum_{k>=1} -log softmax(z[node(s,k-1)])[x_{s,k}].

    nodes_of: per input sequence, its row at each position.  Returns
    (loss, per-copy logp list, dZ [N,V] accumulated over copies)."""
    z = np.asarray(logits, dtype=np.float64)
    lse = _lse(z)
    soft = np.exp(z - lse[:, None])
    B = len(nodes_of)
    loss = 0.0
    dz = np.zeros_like(z)
    copies = []
    for nodes in nodes_of:
        lps = []
        for k in range(1, len(nodes)):
            r = nodes[k - 1]
            x = int(token[nodes[k]])
            lp = z[r, x] - lse[r]
            lps.append((nodes[k], lp))
            loss += -lp / B
            dz[r] += soft[r] / B
            dz[r, x] -= 1.0 / B
        copies.append(lps)
    return loss, copies, dz


def lmhead(hidden, w_vocab, parent, token, weight):
    """Fused lm-head: z = H W, tree loss, dZ, dH = dZ W^T, dW = H^T dZ (fp64)."""
    H = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(w_vocab, dtype=np.float64)
    z = H @ W
    loss, logp, dz = tree_loss(parent, token, weight, z)
    return loss, logp, dz, dz @ W.T, H.T @ dz


def lmhead_rows(hidden_rows, w_vocab, targets):
    """Row-local part of the fused lm-head for selected rows.

    targets: per selected row, a list of (token id, weight).  Returns per row
    (lse, [logp of each target], dZ row, dH row)."""
    W = np.asarray(w_vocab, dtype=np.float64)
    out = []
    for h, tg in zip(hidden_rows, targets):
        z = np.asarray(h, dtype=np.float64) @ W
        m = z.max()
        lse = m + np.log(np.exp(z - m).sum())
        soft = np.exp(z - lse)
        wsum = sum(w for _, w in tg)
        dz = wsum * soft
        lps = []
        for x, w in tg:
            lps.append(z[x] - lse)
            dz[x] -= w
        out.append((lse, lps, dz, dz @ W.T))
    return out


def lmhead_lse(hidden, w_vocab, row_block=256):
    """Log-sum-exp of every row of z = H W (fp64), z formed one block of rows
    at a time so that the whole [rows, vocab] matrix is never held at once
    (the fused lm-head at full vocabulary size)."""
    H = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(w_vocab, dtype=np.float64)
    out = np.empty(H.shape[0])
    for r0 in range(0, H.shape[0], row_block):
        out[r0:r0 + row_block] = _lse(H[r0:r0 + row_block] @ W)
    return out


def lmhead_target_logp(hidden, w_vocab, lse, parent, token, weight):
    """Loss and per-target log-probabilities from per-row LSE (fp64).

    Target t is predicted from row parent[t]: logp_t = z[parent t][x_t] -
    lse[parent t] with z[r][x] = H_r . W[:, x]; loss = -sum_t w_t logp_t.
    Returns (loss, logp [N] with nan at roots)."""
    H = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(w_vocab, dtype=np.float64)
    parent = np.asarray(parent)
    t = np.nonzero(parent >= 0)[0]
    r = parent[t]
    x = np.asarray(token)[t]
    z = np.einsum("td,dt->t", H[r], W[:, x])
    logp = np.full(len(parent), np.nan)
    logp[t] = z - np.asarray(lse)[r]
    loss = -float(np.sum(np.asarray(weight, dtype=np.float64)[t] * logp[t]))
    return loss, logp


def lmhead_dw_columns(hidden, w_vocab, lse, parent, token, weight, cols):
    """Columns `cols` of dW = H^T dZ (fp64), where row r of dZ is
    (sum of its targets' weights) softmax(z_r) - sum over its targets t of
    w_t e_{x_t}; only the selected columns of z and dZ are formed."""
    H = np.asarray(hidden, dtype=np.float64)
    W = np.asarray(w_vocab, dtype=np.float64)
    cols = np.asarray(cols)
    parent = np.asarray(parent)
    weight = np.asarray(weight, dtype=np.float64)
    wsum = np.zeros(H.shape[0])
    for t in np.nonzero(parent >= 0)[0]:
        wsum[parent[t]] += weight[t]
    dz = wsum[:, None] * np.exp(H @ W[:, cols] - np.asarray(lse)[:, None])
    where = {int(c): n for n, c in enumerate(cols)}
    for t in np.nonzero(parent >= 0)[0]:
        n = where.get(int(token[t]))
        if n is not None:
            dz[parent[t], n] -= weight[t]
    return H.T @ dz


def rl_weights(seq_pos_to_dfs, seq_lens, N, seq_scale=None, token_mask=None):
    """Per-row target weights for per-sequence scalars and per-token masks (fp64).

    AReaL-DTA (arXiv 2602.00482), summary page, Main Findings and Why This
    Matters: the method is used for RL post-training (GRPO), where each rollout
    carries its own scalar (its advantage) and prompt tokens carry no loss.
    Reading: token k >= 1 of sequence s, predicted from position k-1, enters
    the branch loss with factor a_s * mask[s,k]; the tree weight of row t is
    w_t = (1/B) * sum over sequences s through t with mask[s, depth t] = 1 of
    a_s.  Sums run over sequences in input order.  Returns w [N] (0 at roots)."""
    B = len(seq_lens)
    w = np.zeros(N, dtype=np.float64)
    off = 0
    for s, L in enumerate(seq_lens):
        a = 1.0 if seq_scale is None else float(seq_scale[s])
        for k in range(1, L):
            if token_mask is None or token_mask[off + k]:
                w[seq_pos_to_dfs[off + k]] += a
        off += L
    return w / B if B else w


def branch_loss_rl(nodes_of, token, logits, seq_scale=None, token_mask=None):
    """(1/B) * sum_s a_s * sum_{k>=1, mask[s,k]} -log softmax(z[node(s,k-1)])[x_{s,k}] and its dZ (fp64)."""
    z = np.asarray(logits, dtype=np.float64)
    lse = _lse(z)
    soft = np.exp(z - lse[:, None])
    B = len(nodes_of)
    loss = 0.0
    dz = np.zeros_like(z)
    off = 0
    for s, nodes in enumerate(nodes_of):
        a = 1.0 if seq_scale is None else float(seq_scale[s])
        for k in range(1, len(nodes)):
            if token_mask is not None and not token_mask[off + k]:
                continue
            r = nodes[k - 1]
            x = int(token[nodes[k]])
            loss += -a * (z[r, x] - lse[r]) / B
            dz[r] += a * soft[r] / B
            dz[r, x] -= a / B
        off += len(nodes)
    return loss, dz
