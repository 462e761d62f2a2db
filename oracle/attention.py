"""Tree attention computed branch by branch, in fp64.

The pages fix what the tree computation must equal (Tree Training, Abstract:
log-probabilities identical to computing every branch on its own; AReaL-DTA
summary, What This Paper Is About: each unique prefix computed once with
correct gradients).  So the oracle does exactly that: it linearises each
branch (an input sequence), applies RoPE at positions 0..L-1, and runs plain
causal softmax attention on it.

Conventions (the pages are silent; readings stated here and used by both sides):
  * scale = 1/sqrt(d) unless given;
  * GQA: query head h reads key/value head h // (Hq/Hkv);
  * LSE is the natural-log log-sum-exp of the scaled scores;
  * the tree's row i takes the value of any copy of i (all copies agree; the
    tests check that), and a gradient with respect to row i is the sum over
    the copies of i, where the copies share the upstream gradient dO_i in any
    split that sums to dO_i (the per-branch graph is linear in dO).
"""
import numpy as np

from .rope import rotate
from .tree import branch_rows


def _gqa(hq, hkv):
    assert hq % hkv == 0
    return hq // hkv


def causal_forward(q, k, v, scale):
    """Textbook causal attention on one linear sequence.

    q: [L, Hq, d]; k, v: [L, Hkv, d] (already rotated). Returns O [L,Hq,d],
    LSE [L,Hq] and the probabilities P [Hq, L, L]."""
    L, hq, d = q.shape
    g = _gqa(hq, k.shape[1])
    O = np.zeros((L, hq, d))
    LSE = np.zeros((L, hq))
    P = np.zeros((hq, L, L))
    tri = np.tril(np.ones((L, L), dtype=bool))
    for h in range(hq):
        S = scale * (q[:, h, :] @ k[:, h // g, :].T)
        S = np.where(tri, S, -np.inf)
        m = S.max(axis=1)
        E = np.exp(S - m[:, None])
        l = E.sum(axis=1)
        P[h] = E / l[:, None]
        LSE[:, h] = m + np.log(l)
        O[:, h, :] = P[h] @ v[:, h // g, :]
    return O, LSE, P


def causal_backward(q, k, v, O, P, dO, scale):
    """Gradients of sum(dO * O) for one linear sequence (rotated inputs)."""
    L, hq, d = q.shape
    g = _gqa(hq, k.shape[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        kv = h // g
        dv[:, kv, :] += P[h].T @ dO[:, h, :]
        dP = dO[:, h, :] @ v[:, kv, :].T
        D = np.sum(dO[:, h, :] * O[:, h, :], axis=1)
        dS = P[h] * (dP - D[:, None])
        dq[:, h, :] = scale * (dS @ k[:, kv, :])
        dk[:, kv, :] += scale * (dS.T @ q[:, h, :])
    return dq, dk, dv


def _scale(d, scale):
    return 1.0 / np.sqrt(d) if not scale else float(scale)


def forward(tree, q, k, v, scale=None, rope_base=10000.0, which="all"):
    """Per-branch forward over the whole tree.

    q [N,Hq,d], k/v [N,Hkv,d] as fp64 (exact widenings of the inputs).
    Returns O [N,Hq,d], LSE [N,Hq] and the largest disagreement between two
    copies of the same row (max |O| and max |LSE| difference)."""
    N, hq, d = q.shape
    sc = _scale(d, scale)
    O = np.full((N, hq, d), np.nan)
    LSE = np.full((N, hq), np.nan)
    dis_o = 0.0
    dis_l = 0.0
    for rows in branch_rows(tree, which):
        pos = np.arange(len(rows))
        qr = rotate(q[rows], pos, rope_base)
        kr = rotate(k[rows], pos, rope_base)
        o, lse, _ = causal_forward(qr, kr, v[rows], sc)
        seen = ~np.isnan(LSE[rows, 0])
        if np.any(seen):
            dis_o = max(dis_o, float(np.max(np.abs(O[rows][seen] - o[seen]))))
            dis_l = max(dis_l, float(np.max(np.abs(LSE[rows][seen] - lse[seen]))))
        O[rows] = o
        LSE[rows] = lse
    return O, LSE, (dis_o, dis_l)


def backward(tree, q, k, v, dO, scale=None, rope_base=10000.0, which="all"):
    """Per-branch backward over the whole tree: dQ [N,Hq,d], dK/dV [N,Hkv,d].

    Each copy of row i receives dO_i / (number of chosen branches through i);
    the tree gradient of a row is the sum over its copies."""
    N, hq, d = q.shape
    sc = _scale(d, scale)
    branches = branch_rows(tree, which)
    cnt = np.zeros(N)
    for rows in branches:
        cnt[rows] += 1.0
    dQ = np.zeros_like(q, dtype=np.float64)
    dK = np.zeros_like(k, dtype=np.float64)
    dV = np.zeros_like(v, dtype=np.float64)
    for rows in branches:
        pos = np.arange(len(rows))
        qr = rotate(q[rows], pos, rope_base)
        kr = rotate(k[rows], pos, rope_base)
        o, _, P = causal_forward(qr, kr, v[rows], sc)
        up = dO[rows] / cnt[rows][:, None, None]
        dqr, dkr, dv = causal_backward(qr, kr, v[rows], o, P, up, sc)
        dQ[rows] += rotate(dqr, pos, rope_base, inverse=True)
        dK[rows] += rotate(dkr, pos, rope_base, inverse=True)
        dV[rows] += dv
    return dQ, dK, dV


# ------------------------------------------------------------------ sampled rows
def ancestors(tree, i):
    """Rows of the branch ending at row i, root first (walks parent pointers)."""
    out = []
    parent = tree["parent"]
    while i >= 0:
        out.append(int(i))
        i = int(parent[i])
    return np.array(out[::-1], dtype=np.int64)


def forward_rows(tree, q, k, v, rows, scale=None, rope_base=10000.0, get=None):
    """O and LSE of selected rows, each from the branch ending at that row.

    `get(name, idx)` may supply fp64 rows of q/k/v lazily (for inputs too
    large to widen whole); otherwise q, k, v are fp64 arrays."""
    if get is None:
        get = lambda name, idx: {"q": q, "k": k, "v": v}[name][idx]  # noqa: E731
    out_o, out_l = [], []
    for i in rows:
        br = ancestors(tree, i)
        pos = np.arange(len(br))
        qi = rotate(get("q", br[-1:]), pos[-1:], rope_base)[0]        # [Hq,d]
        kr = rotate(get("k", br), pos, rope_base)                      # [L,Hkv,d]
        vr = get("v", br)
        hq, d = qi.shape
        g = _gqa(hq, kr.shape[1])
        sc = _scale(d, scale)
        o = np.zeros((hq, d))
        lse = np.zeros(hq)
        for h in range(hq):
            s = sc * (kr[:, h // g, :] @ qi[h])
            m = s.max()
            e = np.exp(s - m)
            lse[h] = m + np.log(e.sum())
            o[h] = (e / e.sum()) @ vr[:, h // g, :]
        out_o.append(o)
        out_l.append(lse)
    return np.array(out_o), np.array(out_l)


def dq_rows(tree, q, k, v, dO, rows, scale=None, rope_base=10000.0, get=None):
    """dQ of selected rows.  Row i's query appears only in branches through i,
    and in each it sees exactly i's ancestors, so dQ_i is the single-copy
    gradient with the full dO_i."""
    if get is None:
        get = lambda name, idx: {"q": q, "k": k, "v": v, "do": dO}[name][idx]  # noqa: E731
    out = []
    for i in rows:
        br = ancestors(tree, i)
        pos = np.arange(len(br))
        qi = rotate(get("q", br[-1:]), pos[-1:], rope_base)[0]
        kr = rotate(get("k", br), pos, rope_base)
        vr = get("v", br)
        doi = get("do", np.array([i]))[0]
        hq, d = qi.shape
        g = _gqa(hq, kr.shape[1])
        sc = _scale(d, scale)
        dq = np.zeros((hq, d))
        for h in range(hq):
            s = sc * (kr[:, h // g, :] @ qi[h])
            p = np.exp(s - s.max())
            p /= p.sum()
            o = p @ vr[:, h // g, :]
            dp = vr[:, h // g, :] @ doi[h]
            ds = p * (dp - doi[h] @ o)
            dq[h] = sc * (ds @ kr[:, h // g, :])
        out.append(rotate(dq[None], pos[-1:], rope_base, inverse=True)[0])
    return np.array(out)


def dkdv_keys(tree, q, k, v, dO, keys, scale=None, rope_base=10000.0, get=None,
              q_lo=0, q_hi=None):
    """dK and dV of selected key rows.

    Key j is seen by the queries of its subtree (rows j..end[j]-1); each of
    those queries i contributes through the branch ending at i.  Queries
    outside [q_lo, q_hi) carry dO = 0 (chunked suffix mode)."""
    if get is None:
        get = lambda name, idx: {"q": q, "k": k, "v": v, "do": dO}[name][idx]  # noqa: E731
    end = tree["end"]
    depth = tree["depth"]
    outk, outv = [], []
    for j in keys:
        j = int(j)
        hi = int(end[j]) if q_hi is None else min(int(end[j]), q_hi)
        qs = range(max(j, q_lo), hi)
        kj = get("k", np.array([j]))
        hkv, d = kj.shape[1], kj.shape[2]
        dk = np.zeros((hkv, d))
        dv = np.zeros((hkv, d))
        for i in qs:
            br = ancestors(tree, i)
            pos = np.arange(len(br))
            qi = rotate(get("q", br[-1:]), pos[-1:], rope_base)[0]
            kr = rotate(get("k", br), pos, rope_base)
            vr = get("v", br)
            doi = get("do", np.array([i]))[0]
            hq = qi.shape[0]
            g = _gqa(hq, hkv)
            sc = _scale(d, scale)
            jpos = int(depth[j])
            for h in range(hq):
                s = sc * (kr[:, h // g, :] @ qi[h])
                p = np.exp(s - s.max())
                p /= p.sum()
                o = p @ vr[:, h // g, :]
                dp = vr[:, h // g, :] @ doi[h]
                ds = p * (dp - doi[h] @ o)
                dv[h // g] += p[jpos] * doi[h]
                dk[h // g] += sc * ds[jpos] * qi[h]
        outk.append(rotate(dk[None], np.array([depth[j]]), rope_base, inverse=True)[0])
        outv.append(dv)
    return np.array(outk), np.array(outv)
