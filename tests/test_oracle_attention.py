"""Pins for oracle/attention.py and oracle/rope.py (CPU only).

* the pages' identity: every copy of a row gets the same output in every branch;
* brute force on the DFS array with a mask built by walking parent pointers;
* closed form with K = 0: LSE = ln(depth+1), O = mean of ancestor V rows;
* B = 1 reduces to torch's causal scaled_dot_product_attention (fp64, CPU),
  and its autograd gradients;
* central finite differences of the oracle's forward for its backward;
* RoPE closed forms.
"""
import numpy as np
import pytest
import torch

import treesynth as ts
from oracle import attention as A
from oracle.rope import rotate
from oracle.tree import dfs_arrays


def _inputs(seed, N, hq, hkv, d, std=1.0):
    rng = ts.rng_for(seed)
    q = ts.normal_f32(rng, (N, hq, d), std).astype(np.float64)
    k = ts.normal_f32(rng, (N, hkv, d), std).astype(np.float64)
    v = ts.normal_f32(rng, (N, hkv, d), std).astype(np.float64)
    do = ts.normal_f32(rng, (N, hq, d)).astype(np.float64)
    return q, k, v, do


TREES = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=voc)
         for s, (n, L, voc) in enumerate([(6, 20, 3), (4, 30, 2), (9, 15, 4), (1, 25, 5), (5, 12, 50)])]


@pytest.mark.parametrize("case", TREES, ids=lambda c: f"seed{c.seed}")
@pytest.mark.parametrize("heads", [(1, 1), (4, 2)])
def test_copies_agree_and_bruteforce(case, heads):
    tree = dfs_arrays(case.seqs)
    N = tree["N"]
    hq, hkv = heads
    d = 8
    q, k, v, _ = _inputs(7, N, hq, hkv, d)
    O, LSE, (dis_o, dis_l) = A.forward(tree, q, k, v, rope_base=100.0, which="all")
    assert dis_o < 1e-12 and dis_l < 1e-12          # identical per-branch results per copy
    O2, LSE2, _ = A.forward(tree, q, k, v, rope_base=100.0, which="leaves")
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(LSE2, LSE, atol=1e-12)

    # brute force on the DFS array: rotate every row at its depth, mask = ancestors by parent walk
    parent = tree["parent"]
    depth = tree["depth"]
    vis = np.zeros((N, N), dtype=bool)
    for i in range(N):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = parent[j]
    qr = rotate(q, depth, 100.0)
    kr = rotate(k, depth, 100.0)
    g = hq // hkv
    for h in range(hq):
        S = (qr[:, h] @ kr[:, h // g].T) / np.sqrt(d)
        S[~vis] = -np.inf
        lse = np.log(np.exp(S - S.max(1, keepdims=True)).sum(1)) + S.max(1)
        P = np.exp(S - lse[:, None])
        np.testing.assert_allclose(LSE[:, h], lse, rtol=0, atol=1e-12)
        np.testing.assert_allclose(O[:, h], P @ v[:, h // g], rtol=0, atol=1e-12)


def test_zero_keys_closed_form():
    case = ts.tiny_tree(0)
    tree = dfs_arrays(case.seqs)
    N = tree["N"]
    q, _, v, _ = _inputs(3, N, 2, 1, 16)
    k = np.zeros((N, 1, 16))
    O, LSE, _ = A.forward(tree, q, k, v)
    np.testing.assert_allclose(LSE, np.log(tree["depth"] + 1.0)[:, None].repeat(2, 1), atol=1e-13)
    # O = mean of V over the row and its ancestors (walked here by parent pointers)
    for i in range(N):
        anc = []
        j = i
        while j >= 0:
            anc.append(j)
            j = tree["parent"][j]
        np.testing.assert_allclose(O[i, 0], v[anc, 0].mean(0), atol=1e-13)
        np.testing.assert_allclose(O[i, 1], v[anc, 0].mean(0), atol=1e-13)


def _torch_causal(q, k, v, hq, hkv):
    """torch CPU fp64 causal SDPA, GQA by repeating kv heads; inputs [L,H,d]."""
    g = hq // hkv
    qt = q.permute(1, 0, 2)[None]
    kt = k.repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    vt = v.repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2)


def test_single_branch_is_torch_causal_attention():
    L, hq, hkv, d = 37, 4, 2, 16
    tree = dfs_arrays([np.arange(L)])
    q, k, v, do = _inputs(11, L, hq, hkv, d)
    O, _, _ = A.forward(tree, q, k, v, rope_base=0)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ot = _torch_causal(qt, kt, vt, hq, hkv)
    np.testing.assert_allclose(O, ot.detach().numpy(), atol=1e-12)
    (ot * torch.tensor(do)).sum().backward()
    dQ, dK, dV = A.backward(tree, q, k, v, do, rope_base=0)
    np.testing.assert_allclose(dQ, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dK, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dV, vt.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("which", ["all", "leaves"])
def test_backward_finite_differences(which):
    case = ts.random_small_tree(4, n_seqs=5, max_len=9, vocab=3)
    tree = dfs_arrays(case.seqs)
    N = tree["N"]
    hq, hkv, d = 2, 1, 4
    q, k, v, do = _inputs(5, N, hq, hkv, d)
    dQ, dK, dV = A.backward(tree, q, k, v, do, rope_base=50.0, which=which)

    def f(qq, kk, vv):
        O, _, _ = A.forward(tree, qq, kk, vv, rope_base=50.0)
        return float(np.sum(O * do))

    rng = np.random.default_rng(0)
    h = 1e-6
    for name, grad in (("q", dQ), ("k", dK), ("v", dV)):
        for _ in range(3):
            base = {"q": q, "k": k, "v": v}
            u = rng.standard_normal(base[name].shape)
            plus = dict(base)
            minus = dict(base)
            plus[name] = base[name] + h * u
            minus[name] = base[name] - h * u
            fd = (f(plus["q"], plus["k"], plus["v"]) - f(minus["q"], minus["k"], minus["v"])) / (2 * h)
            assert abs(fd - float(np.sum(grad * u))) < 1e-7 * max(1.0, abs(fd)), name


def test_dv_sums_to_do():
    """Rows of P sum to one, so summing dV over all keys gives the sum of dO
    over the query heads of each kv group."""
    case = ts.random_small_tree(9, n_seqs=7, max_len=20, vocab=3)
    tree = dfs_arrays(case.seqs)
    q, k, v, do = _inputs(2, tree["N"], 4, 2, 8)
    _, _, dV = A.backward(tree, q, k, v, do)
    np.testing.assert_allclose(dV.sum(0), do.reshape(tree["N"], 2, 2, 8).sum((0, 2)), atol=1e-11)


def test_sampled_rows_match_full():
    case = ts.random_small_tree(12, n_seqs=6, max_len=25, vocab=3)
    tree = dfs_arrays(case.seqs)
    N = tree["N"]
    q, k, v, do = _inputs(8, N, 4, 2, 8)
    O, LSE, _ = A.forward(tree, q, k, v)
    dQ, dK, dV = A.backward(tree, q, k, v, do)
    rows = np.arange(0, N, 3)
    o, lse = A.forward_rows(tree, q, k, v, rows)
    np.testing.assert_allclose(o, O[rows], atol=1e-12)
    np.testing.assert_allclose(lse, LSE[rows], atol=1e-12)
    np.testing.assert_allclose(A.dq_rows(tree, q, k, v, do, rows), dQ[rows], atol=1e-11)
    dk, dv = A.dkdv_keys(tree, q, k, v, do, rows)
    np.testing.assert_allclose(dk, dK[rows], atol=1e-11)
    np.testing.assert_allclose(dv, dV[rows], atol=1e-11)


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 3, 8))
    pos = np.arange(9) * 5
    # identity at position 0
    np.testing.assert_allclose(rotate(x[:1], [0], 10000.0), x[:1], atol=0)
    # norm preserved per (row, head)
    y = rotate(x, pos, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # inverse undoes it
    np.testing.assert_allclose(rotate(y, pos, 10000.0, inverse=True), x, atol=1e-13)
    # scores depend on the position difference only
    qv, kv = rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8))
    s1 = np.sum(rotate(qv, [7], 10000.0) * rotate(kv, [3], 10000.0))
    s2 = np.sum(rotate(qv, [107], 10000.0) * rotate(kv, [103], 10000.0))
    assert abs(s1 - s2) < 1e-12
    # d = 2: theta_0 = 1, a plain plane rotation by the position (in radians)
    p = 0.75
    xy = np.array([[[2.0, -1.0]]])
    want = np.array([2.0 * np.cos(p) + 1.0 * np.sin(p), -1.0 * np.cos(p) + 2.0 * np.sin(p)])
    np.testing.assert_allclose(rotate(xy, [p], 10000.0)[0, 0], want, atol=1e-15)
    # d = 4, base 100: second pair turns at 100^(-1/2) = 0.1 rad per position
    e = np.zeros((1, 1, 4))
    e[0, 0, 1] = 1.0
    r = rotate(e, [3.0], 100.0)[0, 0]
    np.testing.assert_allclose(r, [0, np.cos(0.3), 0, np.sin(0.3)], atol=1e-15)


@pytest.mark.parametrize("q_lo,q_hi", [(0, None), (7, None), (5, 19), (12, 13), (30, 30)])
def test_dkdv_keys_query_range_is_backward_with_do_zeroed(q_lo, q_hi):
    """dkdv_keys restricted to the queries [q_lo, q_hi) (the reference of the
    chunked suffix mode) equals the full per-branch backward whose upstream
    gradient is zero outside that range: attention is linear in dO, so the
    queries outside it contribute nothing."""
    case = ts.random_small_tree(21, n_seqs=6, max_len=24, vocab=3)
    tree = dfs_arrays(case.seqs)
    N = tree["N"]
    q, k, v, do = _inputs(17, N, 4, 2, 8)
    hi = N if q_hi is None else q_hi
    masked = do.copy()
    masked[:q_lo] = 0.0
    masked[hi:] = 0.0
    _, dK, dV = A.backward(tree, q, k, v, masked, rope_base=100.0)
    keys = np.arange(N)
    dk, dv = A.dkdv_keys(tree, q, k, v, do, keys, rope_base=100.0, q_lo=q_lo, q_hi=q_hi)
    np.testing.assert_allclose(dk, dK, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, dV, rtol=0, atol=1e-11)


def test_dkdv_keys_chain_suffix():
    """The chunked path configuration in small: one chain, queries restricted
    to its suffix; equal to the backward with dO = 0 on the prefix."""
    L, prefix = 40, 26
    tree = dfs_arrays([np.arange(L)])
    q, k, v, do = _inputs(23, L, 2, 1, 8)
    masked = do.copy()
    masked[:prefix] = 0.0
    _, dK, dV = A.backward(tree, q, k, v, masked)
    keys = np.array([0, 5, prefix - 1, prefix, L - 2, L - 1])
    dk, dv = A.dkdv_keys(tree, q, k, v, do, keys, q_lo=prefix)
    np.testing.assert_allclose(dk, dK[keys], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, dV[keys], rtol=0, atol=1e-11)
