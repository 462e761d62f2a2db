"""GPU parity of tree attention (through the C ABI) against the fp64 oracle.

Tolerance: max |gpu - oracle| / max |oracle| per tensor, 1e-5 for float32
inputs and 2e-2 for bf16 inputs.  Every input comes from treesynth with a
fixed seed; both sides get the same values.
"""
import ctypes

import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle import attention as OA
from oracle.tree import dfs_arrays
from tests.gpu_util import inputs, rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def _run_tree(seqs, dtype, hq, hkv, d, seed, std=1.0, rope=10000.0, which="leaves", check_bwd=True,
              allow_generic=False):
    tree = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    N = tree.N
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(dtype, seed, N, N, hq, hkv, d, std)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v, rope_base=rope, allow_generic=allow_generic)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, rope_base=rope, which=which)
    tol = TOL[dtype]
    print(f"N={N} hq={hq} hkv={hkv} d={d} {dtype}", flush=True)
    assert rel_err(O, Or) < tol, rel_err(O, Or)
    assert rel_err(L, Lr) < tol, rel_err(L, Lr)
    if not check_bwd:
        return
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do, rope_base=rope, allow_generic=allow_generic)
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, rope_base=rope, which=which)
    assert rel_err(dq, dQr) < tol, ("dq", rel_err(dq, dQr))
    assert rel_err(dk, dKr) < tol, ("dk", rel_err(dk, dKr))
    assert rel_err(dv, dVr) < tol, ("dv", rel_err(dv, dVr))


def test_tiny_tree_fp32():
    """Tiny tree: 64-token root, four 32-token children, one split into two 16-token leaves."""
    _run_tree(ts.tiny_tree(0).seqs, torch.float32, 1, 1, 64, seed=0, which="all")


RANDOM = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=v)
          for s, (n, L, v) in enumerate([(6, 90, 3), (12, 150, 4), (3, 300, 50), (20, 40, 2), (1, 200, 9)])]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: f"seed{c.seed}")
@pytest.mark.parametrize("geom", [(1, 1, 64), (4, 2, 16), (8, 2, 128), (2, 2, 256)])
def test_random_trees_fp32(case, geom):
    hq, hkv, d = geom
    _run_tree(case.seqs, torch.float32, hq, hkv, d, seed=case.seed + 100)


@pytest.mark.parametrize("case", RANDOM[:3], ids=lambda c: f"seed{c.seed}")
def test_random_trees_bf16_generic(case):
    # head dim 64 in bf16 runs the vector kernels, when asked for
    _run_tree(case.seqs, torch.bfloat16, 4, 1, 64, seed=case.seed + 200, allow_generic=True)
    tree = tt.Tree(case.seqs)
    (q, _), (k, _), (v, _), _ = inputs(torch.bfloat16, 1, tree.N, tree.N, 4, 1, 64, 1.0)
    with pytest.raises(tt.TTError, match="TT_ALLOW_GENERIC"):
        tt.tree_attn_fwd(tree, tree.upload_plan(), q, k, v)


def test_no_rope_and_custom_scale_fp32():
    case = RANDOM[0]
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.float32, 5, tree.N, tree.N, 2, 1, 32, 1.0)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v, scale=0.3, rope_base=0.0)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, scale=0.3, rope_base=0, which="leaves")
    assert rel_err(O, Or) < 1e-5 and rel_err(L, Lr) < 1e-5


def test_forward_deterministic():
    case = RANDOM[1]
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    (q, _), (k, _), (v, _), _ = inputs(torch.float32, 9, tree.N, tree.N, 4, 2, 64, 1.0)
    O1, L1 = tt.tree_attn_fwd(tree, plan, q, k, v)
    O2, L2 = tt.tree_attn_fwd(tree, plan, q, k, v)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


@pytest.mark.parametrize("dtype", [torch.float32])
def test_chunked_path_mode(dtype):
    """One root-to-leaf path: a cached prefix, then a suffix processed in fixed
    chunks from right to left (the ragged chunk first), each chunk's forward and
    backward against all keys up to its end, dK/dV added into fp32 buffers.
    The sum over chunks must equal the backward of the whole suffix at once
    (dO = 0 on the prefix rows)."""
    L, prefix, chunk = 700, 256, 128
    seqs = ts.long_chain(3, length=L).seqs
    tree = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    plan = tree.upload_plan()
    hq, hkv, d = 4, 2, 64
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(dtype, 21, L, L, hq, hkv, d, 1.0)
    don[:prefix] = 0.0
    Or, Lr, _ = OA.forward(o, qn, kn, vn)
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don)
    dk = torch.zeros(L, hkv, d, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    starts = list(range(prefix, L, chunk))
    for s in reversed(starts):
        e = min(L, s + chunk)
        Oc, Lc = tt.tree_attn_fwd(tree, plan, q[s:e], k[:e], v[:e], q_off=s)
        assert rel_err(Oc, Or[s:e]) < 1e-5 and rel_err(Lc, Lr[s:e]) < 1e-5
        dqc, _, _ = tt.tree_attn_bwd(tree, plan, q[s:e], k[:e], v[:e], Oc, Lc, do[s:e], q_off=s,
                                     d_k=dk[:e], d_v=dv[:e], accumulate=True)
        assert rel_err(dqc, dQr[s:e]) < 1e-5
    assert rel_err(dk, dKr) < 1e-5 and rel_err(dv, dVr) < 1e-5


def test_empty_and_single():
    tree = tt.Tree([np.array([7])])
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.float32, 1, 1, 1, 2, 1, 16, 1.0)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    # a single row sees only itself: O = v, LSE = scale * q.k
    np.testing.assert_allclose(O.cpu().numpy()[0], np.repeat(vn[0], 2, axis=0), rtol=1e-6)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)
    assert float(dq.abs().max()) < 1e-5 and float(dk.abs().max()) < 1e-5
    np.testing.assert_allclose(dv.cpu().numpy()[0], don[0].sum(0, keepdims=True), rtol=1e-6)


def test_probe_mfma_rate_plausible():
    """The sustained bf16 MFMA rate lies between a quarter of the published
    2.5 PFLOP/s peak and the peak itself (it cannot exceed the hardware)."""
    rate = tt.probe_mfma(n_blocks=512, iters=500, reps=2)
    print(f"sustained bf16 MFMA: {rate:.1f} TFLOP/s", flush=True)
    assert 625.0 < rate < 2520.0, rate


def test_plan_of_another_tree():
    """A plan address the library filled for a tree of another shape is
    rejected on the host (TT_EINVAL, nothing launched, outputs untouched).  A
    buffer whose device contents were overwritten behind the library's back
    (here by a plain device copy of another tree's image) passes the host
    check; the kernels' header check then returns without writing, so the
    outputs keep their previous contents and nothing is read out of bounds
    (the buffer is sized for the tree of the call)."""
    small = tt.Tree([[1, 2, 3, 4], [1, 2, 5]])
    big_case = ts.random_small_tree(11, n_seqs=8, max_len=300, vocab=3)
    big = tt.Tree(big_case.seqs)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.zeros(big.plan_bytes(), dtype=torch.uint8, device="cuda")
    assert tt.lib().tree_plan_upload(small.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel(), st) == tt.TT_OK
    torch.cuda.synchronize()
    for dtype, hq, hkv, d in ((torch.float32, 4, 2, 64), (torch.bfloat16, 8, 2, 128)):
        (q, _), (k, _), (v, _), (do, _) = inputs(dtype, 5, big.N, big.N, hq, hkv, d, d ** -0.5)
        o = torch.full_like(q, 7.0)
        lse = torch.full((big.N, hq), 7.0, dtype=torch.float32, device="cuda")
        with pytest.raises(tt.TTError, match="another shape"):
            tt.tree_attn_fwd(big, buf, q, k, v, o=o, lse=lse)
        with pytest.raises(tt.TTError, match="another shape"):
            tt.tree_attn_bwd(big, buf, q, k, v, o, lse, do)
        assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all())
    # the host records the big tree's upload; then the bytes are replaced on the device
    good = big.upload_plan()
    assert tt.lib().tree_plan_upload(big.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel(), st) == tt.TT_OK
    other = torch.zeros_like(buf)
    assert tt.lib().tree_plan_upload(small.handle, ctypes.c_void_p(other.data_ptr()), other.numel(), st) == tt.TT_OK
    buf.copy_(other)
    torch.cuda.synchronize()
    for dtype, hq, hkv, d in ((torch.float32, 4, 2, 64), (torch.bfloat16, 8, 2, 128)):
        print(f"stale plan bytes: N={big.N} dtype={dtype} d={d}", flush=True)
        (q, _), (k, _), (v, _), (do, _) = inputs(dtype, 5, big.N, big.N, hq, hkv, d, d ** -0.5)
        o = torch.full_like(q, 7.0)
        lse = torch.full((big.N, hq), 7.0, dtype=torch.float32, device="cuda")
        tt.tree_attn_fwd(big, buf, q, k, v, o=o, lse=lse)
        dq = torch.full_like(q, 7.0)
        dk, dv = torch.full_like(k, 7.0), torch.full_like(v, 7.0)
        tt.tree_attn_bwd(big, buf, q, k, v, o, lse, do, d_q=dq, d_k=dk, d_v=dv)
        torch.cuda.synchronize()
        for t_ in (o, lse, dq, dk, dv):
            assert bool((t_.float() == 7.0).all())
    # the right plan works
    (q, qn), (k, kn), (v, vn), _ = inputs(torch.float32, 5, big.N, big.N, 4, 2, 64, 64 ** -0.5)
    O, L = tt.tree_attn_fwd(big, good, q, k, v)
    Or, Lr, _ = OA.forward(dfs_arrays(big_case.seqs), qn, kn, vn, which="leaves")
    assert rel_err(O, Or) < 1e-4 and rel_err(L, Lr) < 1e-4
