"""HIP graph capture of the library's calls.

Every entry point launches on the caller's stream only, never allocates device
memory and never synchronises, and clears buffers with a fill kernel rather
than a memset, so a whole step can be captured once and replayed: tree-mode
forward + backward (bf16, the matrix-core kernels, the backward reusing the
forward's rotated Q and K), the path-mode walk, and the fp32 tiny tree's
forward + backward + weighted NLL.  Every kernel is deterministic (no atomics,
fixed reduction order), so each replay, with unrelated eager work between
replays, must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from tests.gpu_util import inputs

pytestmark = pytest.mark.gpu


def _capture(fn):
    """fn() captured into a graph after two eager warm-up calls on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _replays(g, outs, ref, disturb, n=3):
    for i in range(n):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, r), t in zip(ref.items(), outs):
            assert torch.equal(t, r), (i, name)
        print(f"replay {i}: equal to the eager result", flush=True)


def test_graph_tree_mode_step():
    case = ts.agentic_beam_tree(5, root_len=300, turns=4, width=4, seg_len=(40, 160), n_max=10**9)
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    (q, _), (k, _), (v, _), (do, _) = inputs(torch.bfloat16, 61, tree.N, tree.N, 8, 2, 128, 128 ** -0.5)
    o, lse = torch.empty_like(q), torch.empty(tree.N, 8, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = max(tt.attn_workspace_bytes(tree, plan, q, k, v, True), tt.attn_workspace_bytes(tree, plan, q, k, v, False))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def step():
        tt.tree_attn_fwd(tree, plan, q, k, v, o=o, lse=lse, workspace=ws)
        tt.tree_attn_bwd(tree, plan, q, k, v, o, lse, do, d_q=dq, d_k=dk, d_v=dv, workspace=ws, reuse_rotated=True)

    step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    print(f"N={tree.N}", flush=True)
    g, _ = _capture(step)
    q2 = q.flip(0).contiguous()

    def disturb():  # eager calls on other inputs between replays (same workspace)
        tt.tree_attn_fwd(tree, plan, q2, k, v, workspace=ws)

    _replays(g, [o, lse, dq, dk, dv], ref, disturb)


def test_graph_path_walk():
    case = ts.random_small_tree(7, n_seqs=10, max_len=400, vocab=3)
    tree = tt.Tree(case.seqs)
    path = tt.Path(tree, 128, 0)
    (q, _), (k, _), (v, _), (do, _) = inputs(torch.bfloat16, 62, tree.N, tree.N, 8, 2, 128, 128 ** -0.5)
    o, lse = torch.empty_like(q), torch.empty(tree.N, 8, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = tt.path_workspace_bytes(path, q, k, v, True)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def walk():
        tt.tree_attn_path(path, q, k, v, d_o=do, o=o, lse=lse, d_q=dq, d_k=dk, d_v=dv, workspace=ws)

    walk()  # uploads the walk's plan once (not inside the capture)
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv))}
    print(f"N={tree.N} segments={path.info['n_segments']}", flush=True)
    g, _ = _capture(walk)
    do2 = (do * 2).contiguous()

    def disturb():
        tt.tree_attn_path(path, q, k, v, d_o=do2, o=o, lse=lse, d_q=dq, d_k=dk, d_v=dv, workspace=ws)

    _replays(g, [o, lse, dq, dk, dv], ref, disturb)


def test_graph_tiny_tree_fp32_with_nll():
    case = ts.tiny_tree(0)
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    rng = ts.rng_for(63)
    q, k, v, do = (torch.from_numpy(ts.normal_f32(rng, (tree.N, 1, 64), 1.0)).cuda() for _ in range(4))
    z = torch.from_numpy(ts.normal_f32(rng, (tree.N, 1000), 1.0)).cuda()
    a = tree.export()
    rp, tid, tw = (torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in ("tgt_row_ptr", "tgt_token", "tgt_w"))
    o, lse = torch.empty_like(q), torch.empty(tree.N, 1, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dz = torch.empty_like(z)

    def step():
        tt.tree_attn_fwd(tree, plan, q, k, v, o=o, lse=lse)
        tt.tree_attn_bwd(tree, plan, q, k, v, o, lse, do, d_q=dq, d_k=dk, d_v=dv)
        return tt.tree_weighted_nll(rp, tid, tw, logits=z, d_logits=dz)

    eager = step()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("dz", dz),
                                     ("loss", eager["loss"]), ("logp", eager["logp"]))}
    g, out = _capture(step)
    z2 = (z + 1).contiguous()

    def disturb():
        tt.tree_weighted_nll(rp, tid, tw, logits=z2)

    _replays(g, [o, lse, dq, dk, dv, dz, out["loss"], out["logp"]], ref, disturb)
