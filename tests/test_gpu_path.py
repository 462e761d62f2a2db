"""GPU parity of path mode (tree_attn_path) against the fp64 oracle and tree mode.

Path mode walks the tree depth-first with a stack of the current path and
must give the tree-mode results: O and LSE of every row, and dQ, dK, dV equal
to the per-branch gradients summed over copies.  bf16 (MFMA path, d = 128)
within 2e-2 of the oracle like the tree-mode kernels; fp32 (generic path,
d = 64) within 1e-5 (measured: at most 5e-7).  Chunks of 64 and 128 rows make calls start off 64-row
boundaries (pad rows) and split segments; both child orders are covered.
"""
import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle import attention as OA
from oracle.tree import dfs_arrays
from tests.gpu_util import inputs, rel_err

pytestmark = pytest.mark.gpu

TREES = {
    "beam_small": lambda: ts.agentic_beam_tree(5, root_len=300, turns=4, width=4, seg_len=(40, 160), n_max=10**9),
    "random": lambda: ts.random_small_tree(7, n_seqs=10, max_len=400, vocab=3),
    "forest": lambda: ts.rl_forest(3, n_trees=3, prompt=100, rollouts=4, turns=3, turn_len=(30, 90)),
    "chain": lambda: ts.long_chain(2, length=777),
}


def _run(name, dtype, d, hq, hkv, chunk, order, seed, backward=True):
    case = TREES[name]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    path = tt.Path(tree, chunk, order)
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(dtype, seed, tree.N, tree.N, hq, hkv, d, d ** -0.5)
    print(f"{name}: N={tree.N} dtype={dtype} hq={hq} hkv={hkv} chunk={chunk} order={order} "
          f"segments={path.info['n_segments']} pad_rows={path.info['pad_rows']}", flush=True)
    out = tt.tree_attn_path(path, q, k, v, d_o=do if backward else None)
    return tree, o, (q, k, v, do), (qn, kn, vn, don), out


@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("chunk,order", [(64, 0), (128, 1)])
def test_path_bf16_vs_oracle_and_tree_mode(name, chunk, order):
    tree, o, (q, k, v, do), (qn, kn, vn, don), (O, L, dq, dk, dv) = _run(name, torch.bfloat16, 128, 8, 2, chunk,
                                                                         order, 51)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        assert rel_err(g_, r_) < 2e-2, (n, rel_err(g_, r_))
    # tree mode on the same inputs (same kernels, other summation order)
    plan = tree.upload_plan()
    Ot, Lt = tt.tree_attn_fwd(tree, plan, q, k, v)
    dqt, dkt, dvt = tt.tree_attn_bwd(tree, plan, q, k, v, Ot, Lt, do)
    for n, g_, t_ in (("o", O, Ot), ("lse", L, Lt), ("dq", dq, dqt), ("dk", dk, dkt), ("dv", dv, dvt)):
        r = t_.double().cpu().numpy()
        assert rel_err(g_, r) < 1e-2, (n, rel_err(g_, r))


@pytest.mark.parametrize("hq,hkv", [(8, 1), (12, 1)])
def test_path_bf16_wide_groups_vs_oracle(hq, hkv):
    """Groups of 8 and 12 query heads: the shared backward launches split each
    group over several four-head dQ workgroups (and 12 is not a power of
    two)."""
    _, o, _, (qn, kn, vn, don), (O, L, dq, dk, dv) = _run("beam_small", torch.bfloat16, 128, hq, hkv, 64, 0, 55)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        print(f"  {n}: {rel_err(g_, r_):.2e}", flush=True)
        assert rel_err(g_, r_) < 2e-2, (n, rel_err(g_, r_))


@pytest.mark.parametrize("name", ["beam_small", "chain"])
@pytest.mark.parametrize("hq,hkv", [(4, 2), (2, 1)])
def test_path_bf16_gqa2_vs_oracle(name, hq, hkv):
    """Groups of two query heads.  Over an even number of kv heads the dQ
    workgroups take two kv heads' pairs, so consecutive chunks share a
    backward launch as groups of four do; over one kv head each chunk is its
    own call (dQ and dK/dV as separate launches, one accumulator)."""
    _, o, _, (qn, kn, vn, don), (O, L, dq, dk, dv) = _run(name, torch.bfloat16, 128, hq, hkv, 64, 0, 54)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        print(f"  {n}: {rel_err(g_, r_):.2e}", flush=True)
        assert rel_err(g_, r_) < 2e-2, (n, rel_err(g_, r_))


@pytest.mark.parametrize("name", ["beam_small", "random"])
def test_path_f32_vs_oracle(name):
    _, o, _, (qn, kn, vn, don), (O, L, dq, dk, dv) = _run(name, torch.float32, 64, 4, 2, 64, 0, 52)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        print(f"  {n}: {rel_err(g_, r_):.2e}", flush=True)
        assert rel_err(g_, r_) < 1e-5, (n, rel_err(g_, r_))


def test_path_bf16_no_rope_custom_scale_vs_oracle():
    """rope_base = 0 on the matrix-core walk: the push only scales the query
    operand (no table), and no gradient is rotated back."""
    case = TREES["beam_small"]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    path = tt.Path(tree, 128, 0)
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.bfloat16, 57, tree.N, tree.N, 8, 2, 128, 128 ** -0.5)
    O, L, dq, dk, dv = tt.tree_attn_path(path, q, k, v, d_o=do, scale=0.05, rope_base=0.0)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, scale=0.05, rope_base=0, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, scale=0.05, rope_base=0, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        assert rel_err(g_, r_) < 2e-2, (n, rel_err(g_, r_))


def test_path_forward_only_and_orders_agree():
    """Forward-only walk gives the combined walk's O and LSE; the child order
    changes no result (every call is deterministic per row)."""
    _, _, (q, k, v, do), _, (O0, L0) = _run("forest", torch.bfloat16, 128, 4, 1, 128, 0, 53, backward=False)
    tree = tt.Tree(TREES["forest"]().seqs)
    O1, L1, dq1, dk1, dv1 = tt.tree_attn_path(tt.Path(tree, 128, 1), q, k, v, d_o=do)
    O2, L2, dq2, dk2, dv2 = tt.tree_attn_path(tt.Path(tree, 128, 0), q, k, v, d_o=do)
    assert torch.equal(O0, O1) and torch.equal(L0, L1) and torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.equal(dq1, dq2)
    for a, b in ((dk1, dk2), (dv1, dv2)):
        assert rel_err(a, b.double().cpu().numpy()) < 1e-2


def test_path_chain_equals_chunked_chain():
    """A single chain in path mode: one segment, ceil(L / chunk) calls, right to left."""
    tree, o, _, (qn, kn, vn, don), (O, L, dq, dk, dv) = _run("chain", torch.bfloat16, 128, 4, 2, 192, 0, 54)
    Or, Lr, _ = OA.forward(o, qn, kn, vn)
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don)
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        assert rel_err(g_, r_) < 2e-2, (n, rel_err(g_, r_))


def _gpu_rel(a, b):
    """max |a - b| / max |b| over whole tensors, computed on the GPU in fp32."""
    a, b = a.float(), b.float()
    return ((a - b).abs().max() / b.abs().max().clamp_min(1e-30)).item()


def test_path_agentic_8b_shape_vs_tree_mode_and_sampled_oracle():
    """The 8B-shape agentic tree at full size, walked at the bench's chunk
    (2048): every output equals tree mode's; sampled rows and keys equal the
    oracle's per-branch values."""
    case = ts.agentic_beam_tree(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    N = tree.N
    rng = ts.rng_for(2100)
    qb = ts.normal_bf16(rng, (N, 32, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    ob = ts.normal_bf16(rng, (N, 32, 128), 1.0)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(ob)
    path = tt.Path(tree, 2048, 0)
    print(f"N={N} segments={path.info['n_segments']} calls={path.info['fwd_calls']}", flush=True)
    O, L, dq, dk, dv = tt.tree_attn_path(path, q, k, v, d_o=do)
    plan = tree.upload_plan()
    Ot, Lt = tt.tree_attn_fwd(tree, plan, q, k, v)
    dqt, dkt, dvt = tt.tree_attn_bwd(tree, plan, q, k, v, Ot, Lt, do)
    for n, a, b in (("o", O, Ot), ("lse", L, Lt), ("dq", dq, dqt), ("dk", dk, dkt), ("dv", dv, dvt)):
        assert _gpu_rel(a, b) < 1e-2, (n, _gpu_rel(a, b))

    def get(name, idx):
        return ts.bf16_bits_to_f64({"q": qb, "k": kb, "v": vb, "do": ob}[name][idx])

    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 10).astype(int), [0, N - 1]]))
    ri = torch.as_tensor(rows, device="cuda")
    Or, Lr = OA.forward_rows(o, None, None, None, rows, get=get)
    assert rel_err(O[ri], Or) < 2e-2 and rel_err(L[ri], Lr) < 2e-2
    assert rel_err(dq[ri], OA.dq_rows(o, None, None, None, None, rows, get=get)) < 2e-2
    small = np.nonzero(o["end"] - np.arange(N) <= 40)[0]
    keys = small[np.linspace(0, len(small) - 1, 5).astype(int)]
    rk, rv = OA.dkdv_keys(o, None, None, None, None, keys, get=get)
    ki = torch.as_tensor(keys, device="cuda")
    assert rel_err(dk[ki], rk) < 2e-2 and rel_err(dv[ki], rv) < 2e-2
