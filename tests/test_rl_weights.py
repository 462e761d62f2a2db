"""RL target weights: per-sequence scalars a_s and per-token loss masks (CPU only).

Oracle pins (oracle/nll.py rl_weights, branch_loss_rl):
* the pages' identity extended to scaled, masked branches: the tree loss with
  w_t = (1/B) sum_{s through t, unmasked} a_s equals (1/B) sum_s a_s sum_k
  mask[s,k] NLL_{s,k}, with equal dZ -- for negative scalars too;
* a_s = 1 and no mask give n_pass / B;
* zero logits: loss = (1/B) sum_s a_s #{k >= 1 unmasked} ln V;
* a fully masked sequence contributes nothing.
Library (tree_target_weights) against the oracle: bit-exact float32.
"""
import ctypes

import numpy as np
import pytest

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle.nll import branch_loss_rl, rl_weights, tree_loss
from oracle.tree import dfs_arrays

CASES = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=4, p_dup=0.2, p_prefix=0.3)
         for s, (n, L) in enumerate([(7, 15), (3, 30), (12, 10), (1, 20), (9, 25), (6, 12)])]


def _rl_inputs(case, seed):
    rng = np.random.default_rng(seed)
    B = len(case.seqs)
    a = rng.standard_normal(B).astype(np.float32)          # advantages, either sign
    total = sum(len(s) for s in case.seqs)
    mask = (rng.random(total) < 0.7).astype(np.uint8)      # ~30% masked (prompt-like)
    return a, mask


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"seed{c.seed}")
def test_identity_scaled_masked_branches(case):
    o = dfs_arrays(case.seqs)
    a, mask = _rl_inputs(case, case.seed)
    w = rl_weights(o["seq_pos_to_dfs"], [len(s) for s in case.seqs], o["N"], a, mask)
    z = np.random.default_rng(case.seed + 7).standard_normal((o["N"], 5)) * 2.0
    lt, _, dzt = tree_loss(o["parent"], o["token"], w, z)
    lb, dzb = branch_loss_rl(o["nodes_of"], o["token"], z, a, mask)
    assert abs(lt - lb) <= 1e-12 * max(1.0, abs(lb))
    np.testing.assert_allclose(dzt, dzb, atol=1e-13)


def test_reduces_to_branch_fraction_and_closed_forms():
    case = ts.tiny_tree(0)
    o = dfs_arrays(case.seqs)
    lens = [len(s) for s in case.seqs]
    w = rl_weights(o["seq_pos_to_dfs"], lens, o["N"])
    nonroot = o["parent"] >= 0
    np.testing.assert_array_equal(w[nonroot], o["n_pass"][nonroot] / len(case.seqs))
    # zero logits, prompt mask on the first 64 tokens of every sequence, scalars 1..5
    V = 1000
    a = np.arange(1, 6, dtype=np.float32)
    mask = np.concatenate([(np.arange(L) >= 64).astype(np.uint8) for L in lens])
    w = rl_weights(o["seq_pos_to_dfs"], lens, o["N"], a, mask)
    loss, _, _ = tree_loss(o["parent"], o["token"], w, np.zeros((o["N"], V)))
    want = sum(float(a[s]) * max(0, L - 64) for s, L in enumerate(lens)) / len(lens) * np.log(V)
    assert abs(loss - want) < 1e-10 * want
    # a fully masked sequence changes nothing
    m2 = mask.copy()
    m2[: lens[0]] = 0
    w2 = rl_weights(o["seq_pos_to_dfs"], lens, o["N"], a, m2)
    w3 = rl_weights(o["seq_pos_to_dfs"][lens[0]:], lens[1:], o["N"], a[1:], mask[lens[0]:]) * (len(lens) - 1) / len(lens)
    np.testing.assert_allclose(w2, w3, rtol=0, atol=1e-15)


@pytest.mark.parametrize("case", CASES + [ts.tiny_tree(0), ts.rl_forest_accepted(0)], ids=lambda c: f"seed{c.seed}")
def test_library_bit_exact(case):
    t = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    ex = t.export()
    lens = [len(s) for s in case.seqs]
    a, mask = _rl_inputs(case, 99)
    for sc, mk in ((None, None), (a, None), (None, mask), (a, mask)):
        got = t.target_weights(sc, mk)
        want = rl_weights(o["seq_pos_to_dfs"], lens, o["N"], sc, mk)[o["tgt_dfs"]].astype(np.float32)
        assert got.tobytes() == want.tobytes()
    assert t.target_weights().tobytes() == ex["tgt_w"].tobytes()   # no scalars, no mask: n_pass / B


def test_library_errors():
    t = tt.Tree([[1, 2, 3], [1, 2]])
    lib = tt.lib()
    out = np.zeros(2, dtype=np.float32)
    fp = out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.tree_target_weights(None, None, None, fp) == tt.TT_EINVAL
    assert lib.tree_target_weights(t.handle, None, None, None) == tt.TT_EINVAL
    bad = np.array([1.0, np.nan], dtype=np.float32)
    assert lib.tree_target_weights(t.handle, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), None,
                                   fp) == tt.TT_EINVAL
    with pytest.raises(ValueError):
        t.target_weights(seq_scale=np.ones(3))
    with pytest.raises(ValueError):
        t.target_weights(token_mask=np.ones(4))
