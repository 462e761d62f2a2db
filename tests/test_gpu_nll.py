"""GPU parity of the weighted tree NLL (logits mode) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle.nll import tree_loss, branch_loss, branch_loss_rl
from oracle.tree import dfs_arrays
from tests.gpu_util import rel_err, f32_input, bf16_input

pytestmark = pytest.mark.gpu


def _targets(tree):
    a = tree.export()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    return a, dev(a["tgt_row_ptr"]), dev(a["tgt_token"]), dev(a["tgt_w"])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_tree_logits_mode(dtype):
    case = ts.tiny_tree(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    a, rp, tid, tw = _targets(tree)
    rng = ts.rng_for(1)
    z, zn = (f32_input if dtype == torch.float32 else bf16_input)(rng, (tree.N, 1000))
    out = tt.tree_weighted_nll(rp, tid, tw, logits=z)
    loss, logp, dz = tree_loss(o["parent"], o["token"], o["weight"].astype(np.float64), zn)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert abs(out["loss"].item() - loss) / abs(loss) < tol
    assert rel_err(out["logp"], logp[a["tgt_dfs"]]) < tol
    assert rel_err(out["d_logits"], dz) < tol
    # the pages' identity holds for the GPU loss too (exact weights on the oracle side)
    lb, _, _ = branch_loss(o["nodes_of"], o["token"], zn)
    assert abs(out["loss"].item() - lb) / abs(lb) < tol


def test_in_place_and_duplicates_fp32():
    """d_logits may alias logits; a row whose target list repeats a token id
    gets the summed weight at that position."""
    rng = ts.rng_for(4)
    n, V = 5, 37
    z, zn = f32_input(rng, (n, V))
    rp = torch.tensor([0, 3, 3, 4, 6, 6], dtype=torch.int32, device="cuda")
    ids = torch.tensor([5, 5, 36, 0, 1, 2], dtype=torch.int32, device="cuda")
    w = torch.tensor([0.25, 0.5, 1.0, 0.75, 0.1, 0.2], dtype=torch.float32, device="cuda")
    parent = np.array([-1, 0, 0, 0, 2, 3, 3])  # a small tree carrying the same targets
    want = np.zeros((n, V))
    loss = 0.0
    ids_n, w_n, rp_n = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64), rp.cpu().numpy()
    for r in range(n):
        zr = zn[r]
        lse = np.log(np.exp(zr - zr.max()).sum()) + zr.max()
        W = w_n[rp_n[r]:rp_n[r + 1]].sum()
        want[r] = W * np.exp(zr - lse)
        for t in range(rp_n[r], rp_n[r + 1]):
            want[r, ids_n[t]] -= w_n[t]
            loss += w_n[t] * (lse - zr[ids_n[t]])
    del parent
    zc = z.clone()
    out = tt.tree_weighted_nll(rp, ids, w, logits=zc, d_logits=zc)
    assert abs(out["loss"].item() - loss) / abs(loss) < 1e-5
    assert rel_err(zc, want) < 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rl_weights_logits_mode(dtype):
    """Per-sequence advantages (either sign) and prompt masks through tree_target_weights
    and the NLL kernel equal the scaled, masked per-branch loss of the oracle."""
    case = ts.rl_forest(5, n_trees=2, prompt=40, rollouts=4, turns=2, turn_len=(10, 30), vocab=512)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    a = tree.export()
    rng = np.random.default_rng(11)
    adv = rng.standard_normal(len(case.seqs)).astype(np.float32)
    mask = np.concatenate([(np.arange(len(s)) >= 40).astype(np.uint8) for s in case.seqs])  # prompt masked
    tw = torch.from_numpy(tree.target_weights(adv, mask)).cuda()
    rp = torch.from_numpy(a["tgt_row_ptr"]).cuda()
    tid = torch.from_numpy(a["tgt_token"]).cuda()
    V = 512
    z, zn = (f32_input if dtype == torch.float32 else bf16_input)(ts.rng_for(12), (tree.N, V))
    print(f"N={tree.N} targets={len(a['tgt_dfs'])} dtype={dtype}", flush=True)
    out = tt.tree_weighted_nll(rp, tid, tw, logits=z)
    lb, dzb = branch_loss_rl(o["nodes_of"], o["token"], zn, adv, mask)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert abs(out["loss"].item() - lb) / abs(lb) < tol, (out["loss"].item(), lb)
    assert rel_err(out["d_logits"], dzb) < tol
