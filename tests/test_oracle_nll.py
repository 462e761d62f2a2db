"""Pins for oracle/nll.py (CPU only).

* the pages' identity: the loss averaged over branches equals the per-token
  weighted tree loss (Tree Training, Abstract), with equal gradients;
* closed form with zero logits: loss = (sum_s (|s|-1) / B) ln V;
* B = 1 is torch's summed cross entropy (fp64, CPU);
* finite differences for dZ, dH, dW;
* row-weight invariant: sum of a row's target weights = w_row - (#sequences ending at row)/B;
* the row-blocked full-vocabulary helpers (per-row LSE, target logp, selected dW
  columns) equal the whole-matrix lm-head on small sizes, with blocks that split the rows.
"""
import numpy as np
import pytest
import torch

import treesynth as ts
from oracle.nll import (tree_loss, branch_loss, lmhead, lmhead_rows, lmhead_lse, lmhead_target_logp,
                        lmhead_dw_columns)
from oracle.tree import dfs_arrays

CASES = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=6)
         for s, (n, L) in enumerate([(7, 15), (3, 30), (12, 10), (1, 20), (9, 25)])]


def _exact_w(tree):
    return tree["n_pass"].astype(np.float64) / tree["B"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c.seed}")
def test_branch_average_equals_weighted_tree_loss(case):
    tree = dfs_arrays(case.seqs)
    V = 6
    z = np.random.default_rng(case.seed).standard_normal((tree["N"], V)) * 2.0
    lt, logp, dzt = tree_loss(tree["parent"], tree["token"], _exact_w(tree), z)
    lb, copies, dzb = branch_loss(tree["nodes_of"], tree["token"], z)
    assert abs(lt - lb) <= 1e-12 * abs(lb)
    np.testing.assert_allclose(dzt, dzb, atol=1e-13)
    for lps in copies:                      # every copy's logp equals the tree row's
        for node, lp in lps:
            assert abs(logp[node] - lp) < 1e-13


def test_zero_logits_closed_form():
    case = ts.tiny_tree(0)
    tree = dfs_arrays(case.seqs)
    V = 1000
    loss, logp, _ = tree_loss(tree["parent"], tree["token"], _exact_w(tree), np.zeros((tree["N"], V)))
    want = (sum(len(s) - 1 for s in case.seqs) / len(case.seqs)) * np.log(V)
    assert abs(want - 101.4 * np.log(1000.0)) < 1e-12
    assert abs(loss - want) < 1e-10
    assert abs(round(loss, 3) - 700.446) < 1e-9


def test_single_branch_is_torch_cross_entropy():
    rng = np.random.default_rng(3)
    seq = rng.integers(0, 9, size=23)
    tree = dfs_arrays([seq])
    z = rng.standard_normal((tree["N"], 9))
    loss, _, dz = tree_loss(tree["parent"], tree["token"], _exact_w(tree), z)
    zt = torch.tensor(z[:-1], requires_grad=True)
    ce = torch.nn.functional.cross_entropy(zt, torch.tensor(seq[1:]), reduction="sum")
    ce.backward()
    assert abs(loss - ce.item()) < 1e-12
    np.testing.assert_allclose(dz[:-1], zt.grad.numpy(), atol=1e-13)
    assert np.all(dz[-1] == 0)


def test_row_weight_invariant():
    for case in CASES:
        tree = dfs_arrays(case.seqs)
        w = _exact_w(tree)
        ends = np.zeros(tree["N"])
        for n in tree["nodes_of"]:
            if len(n):
                ends[n[-1]] += 1
        for r in range(tree["N"]):
            kids = tree["tgt_dfs"][tree["tgt_row_ptr"][r]:tree["tgt_row_ptr"][r + 1]]
            assert abs(w[kids].sum() - (w[r] - ends[r] / tree["B"])) < 1e-12


def test_lmhead_finite_differences():
    case = ts.random_small_tree(21, n_seqs=4, max_len=8, vocab=5)
    tree = dfs_arrays(case.seqs)
    N, dm, V = tree["N"], 6, 5
    rng = np.random.default_rng(4)
    H = rng.standard_normal((N, dm))
    W = rng.standard_normal((dm, V)) * 0.5
    w = _exact_w(tree)
    loss, _, dz, dH, dW = lmhead(H, W, tree["parent"], tree["token"], w)
    h = 1e-6
    for name, grad in (("H", dH), ("W", dW)):
        for _ in range(3):
            u = rng.standard_normal(grad.shape)
            if name == "H":
                fp = lmhead(H + h * u, W, tree["parent"], tree["token"], w)[0]
                fm = lmhead(H - h * u, W, tree["parent"], tree["token"], w)[0]
            else:
                fp = lmhead(H, W + h * u, tree["parent"], tree["token"], w)[0]
                fm = lmhead(H, W - h * u, tree["parent"], tree["token"], w)[0]
            assert abs((fp - fm) / (2 * h) - np.sum(grad * u)) < 1e-7
    z = H @ W
    u = rng.standard_normal(z.shape)
    fp = tree_loss(tree["parent"], tree["token"], w, z + h * u)[0]
    fm = tree_loss(tree["parent"], tree["token"], w, z - h * u)[0]
    assert abs((fp - fm) / (2 * h) - np.sum(dz * u)) < 1e-7
    # dZ rows sum to zero, hence so do dW's rows
    np.testing.assert_allclose(dz.sum(1), 0, atol=1e-13)
    np.testing.assert_allclose(dW.sum(1), 0, atol=1e-12)
    # row-local form agrees
    rows = [r for r in range(N) if tree["tgt_row_ptr"][r + 1] > tree["tgt_row_ptr"][r]]
    tg = [[(int(tree["token"][t]), w[t]) for t in tree["tgt_dfs"][tree["tgt_row_ptr"][r]:tree["tgt_row_ptr"][r + 1]]]
          for r in rows]
    for r, (lse, lps, dzr, dhr) in zip(rows, lmhead_rows(H[rows], W, tg)):
        np.testing.assert_allclose(dzr, dz[r], atol=1e-13)
        np.testing.assert_allclose(dhr, dH[r], atol=1e-12)


@pytest.mark.parametrize("row_block", [1, 7, 1000])
def test_lmhead_row_blocked_helpers(row_block):
    """lmhead_lse / lmhead_target_logp / lmhead_dw_columns (used at the full
    vocabulary size, where z cannot be held whole) against lmhead, which forms
    z = H W at once and whose loss and gradients are pinned above."""
    case = ts.random_small_tree(31, n_seqs=8, max_len=18, vocab=40)
    tree = dfs_arrays(case.seqs)
    N, dm, V = tree["N"], 12, 40
    rng = np.random.default_rng(5)
    H = rng.standard_normal((N, dm))
    W = rng.standard_normal((dm, V)) * 0.3
    w = _exact_w(tree)
    loss, logp, dz, dH, dW = lmhead(H, W, tree["parent"], tree["token"], w)
    lse = lmhead_lse(H, W, row_block=row_block)
    l2, lp2 = lmhead_target_logp(H, W, lse, tree["parent"], tree["token"], w)
    assert abs(l2 - loss) <= 1e-12 * abs(loss)
    t = tree["parent"] >= 0
    np.testing.assert_allclose(lp2[t], logp[t], rtol=0, atol=1e-12)
    assert np.all(np.isnan(lp2[~t]))
    cols = np.array([0, 3, int(tree["token"][1]), V - 1, 17])
    np.testing.assert_allclose(lmhead_dw_columns(H, W, lse, tree["parent"], tree["token"], w, cols), dW[:, cols],
                               rtol=0, atol=1e-12)
