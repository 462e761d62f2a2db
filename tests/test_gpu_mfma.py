"""GPU parity of the bf16 MFMA tree-attention kernels (head dim 128) against the fp64 oracle.

Tolerance 2e-2 (max |gpu - oracle| / max |oracle| per tensor; where printed,
also per row: each row judged against its own maximum).  Trees span several
64-row tiles and end in a ragged tile; GQA groups 1, 2, 3, 4 and 8; scores
both mild (std 1/sqrt(128)) and peaky (std 1), and scores built to move the
forward's running max along the walk; long query walks over a shared
4096-token root; the full 8B tree against the same kernels run branch by
branch; tensors past 4 GiB.
"""
import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle import attention as OA
from oracle.tree import dfs_arrays
from tests.gpu_util import inputs, rel_err, row_rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-2

TREES = {
    "beam_small": lambda: ts.agentic_beam_tree(5, root_len=300, turns=4, width=4, seg_len=(40, 160), n_max=10**9),
    "random": lambda: ts.random_small_tree(7, n_seqs=10, max_len=400, vocab=3),
    "forest": lambda: ts.rl_forest(3, n_trees=3, prompt=100, rollouts=4, turns=3, turn_len=(30, 90)),
    "chain": lambda: ts.long_chain(2, length=777),
}


def _fwd_case(name, hq, hkv, std, seed):
    case = TREES[name]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), _ = inputs(torch.bfloat16, seed, tree.N, tree.N, hq, hkv, 128, std)
    print(f"{name}: N={tree.N} hq={hq} hkv={hkv} std={std}", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    return O, L, Or, Lr


@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("heads", [(8, 2), (4, 2), (2, 2), (16, 2), (6, 2)])
def test_mfma_forward(name, heads):
    O, L, Or, Lr = _fwd_case(name, heads[0], heads[1], 128 ** -0.5, 31)
    assert rel_err(O, Or) < TOL, rel_err(O, Or)
    assert rel_err(L, Lr) < TOL, rel_err(L, Lr)


@pytest.mark.parametrize("name", ["beam_small", "chain"])
def test_mfma_forward_peaky(name):
    O, L, Or, Lr = _fwd_case(name, 4, 1, 1.0, 32)
    assert rel_err(O, Or) < TOL, rel_err(O, Or)
    assert rel_err(L, Lr) < TOL, rel_err(L, Lr)


def _moving_max_inputs(N, hq, hkv, prof, seed):
    """bf16 q, k, v (device, and exact fp64 copies) whose score of query head
    h against key row j is, in log2 units, about (1 + h/8) (s_j + noise_j):
    q rows are one unit direction u, k row j is u times its target score."""
    rng = np.random.default_rng(seed)
    j = np.arange(N, dtype=np.float64)
    if prof == "rising":        # every 32-key half climbs 16 log2 units
        s = 0.5 * j
    elif prof == "sawtooth":    # climbs and falls: some tiles move the max, some do not
        s = 12.0 * np.sin(j / 37.0) + 0.02 * j
    else:                       # flat, then +20 from a key in the second half of a tile
        s = np.where(j >= (N // 128) * 64 + 45, 20.0, 0.0)
    u = rng.normal(size=128)
    u /= np.linalg.norm(u)
    kn = (s[:, None] + rng.normal(0.0, 1.0, (N, hkv)))[..., None] * u * (128 ** 0.5 / np.log2(np.e))
    qn = (1.0 + np.arange(hq) / 8.0)[None, :, None] * u + rng.normal(0.0, 1e-3, (N, hq, 128))
    vn = rng.normal(size=(N, hkv, 128))
    out = []
    for x in (qn, kn, vn):
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).cuda()
        out.append((t, t.float().cpu().double().numpy()))
    return out


@pytest.mark.parametrize("prof", ["rising", "sawtooth", "step"])
@pytest.mark.parametrize("name,heads", [("beam_small", (8, 2)), ("chain", (4, 2)), ("forest", (8, 2))])
def test_mfma_forward_moving_max(prof, name, heads):
    """Scores that move the running max along the walk.  The forward takes its
    exponentials against the running max and redoes a tile when a row's
    partial sum over a 32-key half passes the bound or the row meets its
    first visible key: here whole walks of tiles do that (rising), some tiles
    do and others not (sawtooth), or one jump lands in a tile's second half
    after a quiet first half (step).  No RoPE, so each score is the one
    constructed."""
    case = TREES[name]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn) = _moving_max_inputs(tree.N, heads[0], heads[1], prof, 41)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v, rope_base=0.0)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, rope_base=0.0, which="leaves")
    e_o, e_row, e_l = rel_err(O, Or), row_rel_err(O, Or), rel_err(L, Lr)
    print(f"{name} {prof} N={tree.N}: O {e_o:.2e} (per row {e_row:.2e}), LSE {e_l:.2e}", flush=True)
    assert np.isfinite(O.float().cpu().numpy()).all() and np.isfinite(L.cpu().numpy()).all()
    assert e_o < TOL and e_row < TOL and e_l < TOL


def test_mfma_forward_deterministic():
    case = TREES["forest"]()
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    (q, _), (k, _), (v, _), _ = inputs(torch.bfloat16, 3, tree.N, tree.N, 8, 2, 128, 1.0)
    O1, L1 = tt.tree_attn_fwd(tree, plan, q, k, v)
    O2, L2 = tt.tree_attn_fwd(tree, plan, q, k, v)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_mfma_forward_chunks():
    """Path mode: chunks of the suffix against all keys up to their end."""
    L, prefix, chunk = 1000, 448, 192
    seqs = ts.long_chain(4, length=L).seqs
    tree = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), _ = inputs(torch.bfloat16, 8, L, L, 8, 2, 128, 128 ** -0.5)
    Or, Lr, _ = OA.forward(o, qn, kn, vn)
    for s in reversed(range(prefix, L, chunk)):
        e = min(L, s + chunk)
        Oc, Lc = tt.tree_attn_fwd(tree, plan, q[s:e], k[:e], v[:e], q_off=s)
        assert rel_err(Oc, Or[s:e]) < TOL and rel_err(Lc, Lr[s:e]) < TOL


def _lazy_rows(bits_q, bits_k, bits_v):
    def get(name, idx):
        src = {"q": bits_q, "k": bits_k, "v": bits_v}[name]
        return ts.bf16_bits_to_f64(src[idx])
    return get


def test_mfma_forward_agentic_8b_shape_sampled():
    """The 8B-shape agentic tree at full size (32 query heads, 8 kv heads):
    sampled rows against the oracle's per-row branch computation."""
    case = ts.agentic_beam_tree(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    N = tree.N
    rng = ts.rng_for(1000)
    qb = ts.normal_bf16(rng, (N, 32, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    plan = tree.upload_plan()
    O, L = tt.tree_attn_fwd(tree, plan, dev(qb), dev(kb), dev(vb))
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 24).astype(int), [0, 63, 64, N - 1],
                                     ts.rng_for(5).integers(0, N, 8)]))
    Or, Lr = OA.forward_rows(o, None, None, None, rows, get=_lazy_rows(qb, kb, vb))
    ri = torch.as_tensor(rows, device=O.device)
    assert rel_err(O[ri], Or) < TOL and rel_err(L[ri], Lr) < TOL


def test_mfma_forward_rl_forest_1p7b_sampled():
    """The 1.7B-shape RL forest at full size (16 query heads, 8 kv heads),
    forward only as timed: sampled rows against the oracle's per-row branch
    computation."""
    case = ts.rl_forest_accepted(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    N = tree.N
    rng = ts.rng_for(1100)
    qb = ts.normal_bf16(rng, (N, 16, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    plan = tree.upload_plan()
    print(f"rl forest seed {case.seed}: N={N}", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, dev(qb), dev(kb), dev(vb))
    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 24).astype(int), [0, 63, 64, N - 1],
                                     ts.rng_for(6).integers(0, N, 8)]))
    Or, Lr = OA.forward_rows(o, None, None, None, rows, get=_lazy_rows(qb, kb, vb))
    ri = torch.as_tensor(rows, device=O.device)
    assert rel_err(O[ri], Or) < TOL and rel_err(L[ri], Lr) < TOL


# ------------------------------------------------------------------ backward
def _bwd_case(name, hq, hkv, std, seed):
    case = TREES[name]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.bfloat16, seed, tree.N, tree.N, hq, hkv, 128, std)
    print(f"{name}: N={tree.N} hq={hq} hkv={hkv} std={std}", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    return (dq, dk, dv), (dQr, dKr, dVr)


@pytest.mark.parametrize("name", list(TREES))
@pytest.mark.parametrize("heads", [(8, 2), (4, 2), (2, 2), (16, 2), (6, 2), (16, 8), (2, 1)])
def test_mfma_backward(name, heads):
    """Groups of 4 (and multiples) and groups of 2 over an even number of kv
    heads run dQ and dK/dV in one launch (a GQA-2 dQ workgroup takes two kv
    heads: (4, 2), (16, 8)); groups of 1, 3 and groups of 2 over one kv head
    run them as two launches."""
    got, ref = _bwd_case(name, heads[0], heads[1], 128 ** -0.5, 41)
    for n, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        assert rel_err(g_, r_) < TOL, (n, rel_err(g_, r_))


@pytest.mark.parametrize("name", ["beam_small", "forest"])
def test_mfma_backward_peaky(name):
    got, ref = _bwd_case(name, 4, 1, 1.0, 42)
    for n, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        assert rel_err(g_, r_) < TOL, (n, rel_err(g_, r_))


def test_mfma_backward_no_rope_custom_scale():
    """rope_base = 0: no rotation anywhere (the dQ and dK/dV epilogues only
    scale and convert); a scale other than 1/sqrt(d)."""
    case = TREES["beam_small"]()
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.bfloat16, 43, tree.N, tree.N, 8, 2, 128, 128 ** -0.5)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v, scale=0.05, rope_base=0.0)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do, scale=0.05, rope_base=0.0)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, scale=0.05, rope_base=0, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, scale=0.05, rope_base=0, which="leaves")
    assert rel_err(O, Or) < TOL and rel_err(L, Lr) < TOL
    for n, g_, r_ in zip(("dq", "dk", "dv"), (dq, dk, dv), (dQr, dKr, dVr)):
        assert rel_err(g_, r_) < TOL, (n, rel_err(g_, r_))


@pytest.mark.parametrize("rope_base", [10000.0, 0.0])
def test_mfma_backward_reuses_forward_rotation(rope_base):
    """TT_BWD_REUSE_ROTATED with the forward's workspace gives the same bits
    as a backward that rotates q and k itself (the forward kernel makes its
    own query operand, the backward's RoPE kernel the same one); a q_off
    chunk too, and the scaled copy without rotation."""
    case = TREES["forest"]()
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    (q, _), (k, _), (v, _), (do, _) = inputs(torch.bfloat16, 44, tree.N, tree.N, 8, 2, 128, 128 ** -0.5)
    for q_off in (0, 128):
        qc, doc = q[q_off:], do[q_off:]
        nb = max(tt.attn_workspace_bytes(tree, plan, qc, k, v, fb, q_off=q_off, rope_base=rope_base)
                 for fb in (True, False))
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        O, L = tt.tree_attn_fwd(tree, plan, qc, k, v, q_off=q_off, rope_base=rope_base, workspace=ws)
        got = tt.tree_attn_bwd(tree, plan, qc, k, v, O, L, doc, q_off=q_off, rope_base=rope_base, workspace=ws,
                               reuse_rotated=True)
        ref = tt.tree_attn_bwd(tree, plan, qc, k, v, O, L, doc, q_off=q_off, rope_base=rope_base)
        for n, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g_, r_), (q_off, n)


def test_mfma_backward_chunks_accumulate():
    """Right-to-left chunks of a suffix against a cached prefix, dK/dV added
    into fp32 buffers across chunks == oracle backward with dO = 0 on the prefix."""
    L, prefix, chunk = 1000, 448, 192
    seqs = ts.long_chain(6, length=L).seqs
    tree = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.bfloat16, 9, L, L, 8, 2, 128, 128 ** -0.5)
    don[:prefix] = 0.0
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don)
    dk = torch.zeros(L, 2, 128, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    for s in reversed(range(prefix, L, chunk)):
        e = min(L, s + chunk)
        Oc, Lc = tt.tree_attn_fwd(tree, plan, q[s:e], k[:e], v[:e], q_off=s)
        dqc, _, _ = tt.tree_attn_bwd(tree, plan, q[s:e], k[:e], v[:e], Oc, Lc, do[s:e], q_off=s,
                                     d_k=dk[:e], d_v=dv[:e], accumulate=True)
        assert rel_err(dqc, dQr[s:e]) < TOL
    assert rel_err(dk, dKr) < TOL and rel_err(dv, dVr) < TOL


def test_mfma_backward_agentic_8b_shape_sampled():
    """8B-shape agentic tree at full size: dQ on sampled rows; dK/dV on keys
    with small subtrees; over all keys, sum_j dV_j = sum over the group's
    query heads of sum_i dO_i, and sum_j R(depth_j) dK_j = 0 (rows of dS sum
    to zero)."""
    case = ts.agentic_beam_tree(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    N = tree.N
    rng = ts.rng_for(2000)
    qb = ts.normal_bf16(rng, (N, 32, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    ob = ts.normal_bf16(rng, (N, 32, 128), 1.0)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    plan = tree.upload_plan()
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(ob)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)

    def get(name, idx):
        return ts.bf16_bits_to_f64({"q": qb, "k": kb, "v": vb, "do": ob}[name][idx])

    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 12).astype(int), [0, N - 1]]))
    ref = OA.dq_rows(o, None, None, None, None, rows, get=get)
    assert rel_err(dq[torch.as_tensor(rows, device="cuda")], ref) < TOL
    # keys whose subtree holds at most 40 rows (deep in a leaf segment)
    small = np.nonzero(o["end"] - np.arange(N) <= 40)[0]
    keys = small[np.linspace(0, len(small) - 1, 6).astype(int)]
    rk, rv = OA.dkdv_keys(o, None, None, None, None, keys, get=get)
    ki = torch.as_tensor(keys, device="cuda")
    assert rel_err(dk[ki], rk) < TOL and rel_err(dv[ki], rv) < TOL
    # identities over all keys
    sdv = dv.float().sum(0).cpu().double().numpy()
    sdo = do.float().reshape(N, 8, 4, 128).sum((0, 2)).cpu().double().numpy()
    assert rel_err(torch.from_numpy(sdv), sdo) < TOL
    from oracle.rope import rotate
    dkr = rotate(dk.float().cpu().double().numpy(), o["depth"], 10000.0)
    tot = np.abs(dkr.sum(0)).max()
    assert tot < 2e-2 * np.abs(dkr).sum(0).max(), tot


def test_mfma_backward_rl_forest_1p7b_sampled():
    """The 1.7B-shape RL forest at full size (16 query heads, 8 kv heads: the
    one-launch backward with dQ workgroups over kv-head pairs, 2,840 of them
    beside 712 dK/dV workgroups): dQ on sampled rows, dK/dV on sampled keys
    with subtrees of up to 40 rows and on one key whose subtree holds about 100
    rows; over all keys, sum_j dV_j = sum over the group's two
    query heads of sum_i dO_i, and sum_j R(depth_j) dK_j = 0."""
    case = ts.rl_forest_accepted(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    N = tree.N
    rng = ts.rng_for(2100)
    qb = ts.normal_bf16(rng, (N, 16, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (N, 8, 128), 128 ** -0.5)
    ob = ts.normal_bf16(rng, (N, 16, 128), 1.0)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    plan = tree.upload_plan()
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(ob)
    print(f"rl forest seed {case.seed}: N={N}", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)

    def get(name, idx):
        return ts.bf16_bits_to_f64({"q": qb, "k": kb, "v": vb, "do": ob}[name][idx])

    rows = np.unique(np.concatenate([np.linspace(0, N - 1, 12).astype(int), [0, 63, 64, N - 1]]))
    ref = OA.dq_rows(o, None, None, None, None, rows, get=get)
    assert rel_err(dq[torch.as_tensor(rows, device="cuda")], ref) < TOL
    sub = o["end"] - np.arange(N)
    small = np.nonzero(sub <= 40)[0]
    keys = small[np.linspace(0, len(small) - 1, 6).astype(int)]
    # and the last key whose subtree holds 100-300 rows (the oracle's cost per
    # key grows with subtree rows x depth: ~10 s here)
    mid = np.nonzero((sub >= 100) & (sub <= 300))[0]
    keys = np.concatenate([keys, mid[-1:]])
    print(f"keys {keys.tolist()} subtree rows {sub[keys].tolist()}", flush=True)
    rk, rv = OA.dkdv_keys(o, None, None, None, None, keys, get=get)
    ki = torch.as_tensor(keys, device="cuda")
    assert rel_err(dk[ki], rk) < TOL and rel_err(dv[ki], rv) < TOL
    sdv = dv.float().sum(0).cpu().double().numpy()
    sdo = do.float().reshape(N, 8, 2, 128).sum((0, 2)).cpu().double().numpy()
    assert rel_err(torch.from_numpy(sdv), sdo) < TOL
    from oracle.rope import rotate
    dkr = rotate(dk.float().cpu().double().numpy(), o["depth"], 10000.0)
    tot = np.abs(dkr.sum(0)).max()
    assert tot < 2e-2 * np.abs(dkr).sum(0).max(), tot


def test_mfma_chain_suffix_chunks_8b_full():
    """The 8B-shape path configuration at full size, launched as timed: a
    49,152-token chain whose last 16,384 queries run in 2048-row chunks right
    to left against all earlier keys, dK/dV added into fp32 buffers.  The
    chunks partition the queries, so the result equals one call over the whole
    suffix; sampled suffix rows (O, LSE, dQ) and the last keys (dK, dV) equal
    the oracle's; over all keys sum_j dV_j is the sum of the suffix dO over the
    group's query heads and sum_j R(depth_j) dK_j = 0."""
    L, prefix, chunk = 49152, 32768, 2048
    case = ts.long_chain(0)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    rng = ts.rng_for(2200)
    qb = ts.normal_bf16(rng, (L, 32, 128), 128 ** -0.5)
    kb = ts.normal_bf16(rng, (L, 8, 128), 128 ** -0.5)
    vb = ts.normal_bf16(rng, (L, 8, 128), 128 ** -0.5)
    ob = ts.normal_bf16(rng, (L, 32, 128), 1.0)
    ob[:prefix] = 0  # bf16 +0: no upstream gradient on the cached prefix
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(ob)
    plan = tree.upload_plan()
    dk = torch.zeros(L, 8, 128, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    O = torch.empty(L - prefix, 32, 128, dtype=torch.bfloat16, device="cuda")
    Ls = torch.empty(L - prefix, 32, dtype=torch.float32, device="cuda")
    dq = torch.empty_like(O)
    for s in reversed(range(prefix, L, chunk)):
        e = min(L, s + chunk)
        print(f"chunk [{s}, {e})", flush=True)
        Oc, Lc = tt.tree_attn_fwd(tree, plan, q[s:e], k[:e], v[:e], q_off=s)
        dqc, _, _ = tt.tree_attn_bwd(tree, plan, q[s:e], k[:e], v[:e], Oc, Lc, do[s:e], q_off=s,
                                     d_k=dk[:e], d_v=dv[:e], accumulate=True)
        O[s - prefix:e - prefix], Ls[s - prefix:e - prefix], dq[s - prefix:e - prefix] = Oc, Lc, dqc
    print("one call over the suffix", flush=True)
    Ou, Lu = tt.tree_attn_fwd(tree, plan, q[prefix:], k, v, q_off=prefix)
    dqu, dku, dvu = tt.tree_attn_bwd(tree, plan, q[prefix:], k, v, Ou, Lu, do[prefix:], q_off=prefix)
    for n, a, b in (("o", O, Ou), ("lse", Ls, Lu), ("dq", dq, dqu), ("dk", dk, dku), ("dv", dv, dvu)):
        r = ((a.float() - b.float()).abs().max() / b.float().abs().max()).item()
        assert r < 1e-2, (n, r)

    def get(name, idx):
        return ts.bf16_bits_to_f64({"q": qb, "k": kb, "v": vb, "do": ob}[name][idx])

    rows = np.array([prefix, prefix + chunk - 1, prefix + chunk, L - chunk - 1, L - chunk, L - 1])
    Or, Lr = OA.forward_rows(o, None, None, None, rows, get=get)
    ri = torch.as_tensor(rows - prefix, device="cuda")
    assert rel_err(O[ri], Or) < TOL and rel_err(Ls[ri], Lr) < TOL
    assert rel_err(dq[ri], OA.dq_rows(o, None, None, None, None, rows, get=get)) < TOL
    keys = np.array([L - 5, L - 2, L - 1])
    rk, rv = OA.dkdv_keys(o, None, None, None, None, keys, get=get, q_lo=prefix)
    ki = torch.as_tensor(keys, device="cuda")
    assert rel_err(dk[ki], rk) < TOL and rel_err(dv[ki], rv) < TOL
    sdv = dv.sum(0).cpu().double().numpy()
    sdo = do[prefix:].float().reshape(L - prefix, 8, 4, 128).sum((0, 2)).cpu().double().numpy()
    assert rel_err(torch.from_numpy(sdv), sdo) < TOL
    from oracle.rope import rotate
    dkr = rotate(dk.cpu().double().numpy(), o["depth"], 10000.0)
    tot = np.abs(dkr.sum(0)).max()
    assert tot < 2e-2 * np.abs(dkr).sum(0).max(), tot


# ------------------------------------------------------------------ long walks, full size
# a 4096-token root under four 1024-token children, the first splitting into
# two 1024-token leaves: N = 10240, so every dK/dV workgroup over the root
# walks the 160 query tiles of the whole tree (x 4 heads of its group)
MID_SPEC = (4096, [(1024, [(1024, []), (1024, [])]), (1024, []), (1024, []), (1024, [])])


def test_mfma_backward_long_walks_full_tensor():
    """Full-tensor dQ, dK, dV against the oracle where the dK/dV kernel takes
    its long paths: the shared root's keys collect the gradient of all 10,240
    queries below them (AReaL-DTA summary, Key Contributions 1: a shared
    prefix is backpropagated once with the gradients of all descendant leaves
    accumulated).  Errors per tensor are held to 2e-2, and per row too for O,
    LSE, dK and dV.  dQ's per-row error is printed only: the depth-0 query sees
    only itself, so its dQ is exactly zero (dS = P (dP - D) with P = 1 and
    D = dP), and shallow queries' dQ nearly cancels, so their own maxima are
    no scale for the rounding of D = rowsum(dO * O) from the bf16 O."""
    case = ts.nested_tree(17, MID_SPEC)
    tree = tt.Tree(case.seqs)
    o = dfs_arrays(case.seqs)
    plan = tree.upload_plan()
    (q, qn), (k, kn), (v, vn), (do, don) = inputs(torch.bfloat16, 51, tree.N, tree.N, 4, 1, 128, 128 ** -0.5)
    print(f"mid tree N={tree.N} hq=4 hkv=1", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)
    Or, Lr, _ = OA.forward(o, qn, kn, vn, which="leaves")
    dQr, dKr, dVr = OA.backward(o, qn, kn, vn, don, which="leaves")
    for n, g_, r_ in (("o", O, Or), ("lse", L, Lr), ("dq", dq, dQr), ("dk", dk, dKr), ("dv", dv, dVr)):
        e, er = rel_err(g_, r_), row_rel_err(g_, r_)
        print(f"  {n}: tensor {e:.2e}  per-row {er:.2e}", flush=True)
        assert e < TOL and (n == "dq" or er < TOL), (n, e, er)


def test_mfma_tree_sibling_order_invariant():
    """Results per input token do not depend on the sibling order of the DFS
    serialization: the same sequences with every token id mirrored (so every
    sibling list is reversed and rows move) give the same O, LSE, dQ, dK, dV
    per (sequence, position), up to bf16 rounding of differently ordered sums."""
    case = ts.nested_tree(18, MID_SPEC, vocab=1000)
    a = tt.Tree(case.seqs)
    b = tt.Tree([999 - np.asarray(s_) for s_ in case.seqs])
    ea, eb = a.export(), b.export()
    perm = np.empty(a.N, dtype=np.int64)              # row of tree a -> row of tree b
    perm[ea["seq_pos_to_dfs"]] = eb["seq_pos_to_dfs"]
    assert not np.array_equal(perm, np.arange(a.N))   # the rows really moved
    pa, pb = a.upload_plan(), b.upload_plan()
    (q, _), (k, _), (v, _), (do, _) = inputs(torch.bfloat16, 52, a.N, a.N, 8, 2, 128, 128 ** -0.5)
    pt = torch.as_tensor(perm, device="cuda")
    qb_, kb_, vb_, dob = (torch.empty_like(x) for x in (q, k, v, do))
    for src, dst in ((q, qb_), (k, kb_), (v, vb_), (do, dob)):
        dst[pt] = src
    Oa, La = tt.tree_attn_fwd(a, pa, q, k, v)
    ga = tt.tree_attn_bwd(a, pa, q, k, v, Oa, La, do)
    Ob, Lb = tt.tree_attn_fwd(b, pb, qb_, kb_, vb_)
    gb = tt.tree_attn_bwd(b, pb, qb_, kb_, vb_, Ob, Lb, dob)
    for n, x, y in (("o", Oa, Ob), ("lse", La, Lb), ("dq", ga[0], gb[0]), ("dk", ga[1], gb[1]), ("dv", ga[2], gb[2])):
        ref = y[pt].float().cpu().double().numpy()
        e = rel_err(x, ref)
        print(f"  {n}: {e:.2e}", flush=True)
        assert e < 1e-2, (n, e)


def test_mfma_8b_tree_equals_branches_summed():
    """The 8B-shape agentic tree at full size against the same kernels run on
    every root-to-leaf branch as its own chain: tree-mode dK, dV of every key
    (the 4,096-token root included, whose workgroups walk 1,032 query tiles
    per head) equal the sum over the key's copies in the branches, and dQ,
    O, LSE equal the branch values.  Each tree row's upstream gradient goes
    whole to the first branch through it and zero to the others (the
    gradients are linear in dO, so the copies still sum to the tree's).
    Held to 2e-2 per tensor, and per row for all but dQ (whose shallow rows
    cancel; printed)."""
    case = ts.agentic_beam_tree(0)
    tree = tt.Tree(case.seqs)
    ex = tree.export()
    N = tree.N
    g = torch.Generator(device="cuda").manual_seed(77)
    mk = lambda *sh, std=128 ** -0.5: (torch.randn(*sh, device="cuda", generator=g) * std).to(torch.bfloat16)  # noqa
    q, k, v, do = mk(N, 32, 128), mk(N, 8, 128), mk(N, 8, 128), mk(N, 32, 128, std=1.0)
    plan = tree.upload_plan()
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)
    sdq = torch.zeros(N, 32, 128, device="cuda")
    sdk = torch.zeros(N, 8, 128, device="cuda")
    sdv = torch.zeros_like(sdk)
    bo = torch.zeros(N, 32, 128, device="cuda")
    bl = torch.zeros(N, 32, device="cuda")
    owned = torch.zeros(N, dtype=torch.bool, device="cuda")
    off = 0
    for b, s_ in enumerate(case.seqs):
        rows = torch.as_tensor(ex["seq_pos_to_dfs"][off:off + len(s_)].astype(np.int64), device="cuda")
        off += len(s_)
        mine = ~owned[rows]
        owned[rows] = True
        bt = tt.Tree([s_])
        bp = bt.upload_plan()
        qb_, kb_, vb_ = q[rows].contiguous(), k[rows].contiguous(), v[rows].contiguous()
        dob = (do[rows] * mine[:, None, None]).contiguous()
        print(f"branch {b}: {len(s_)} rows, {int(mine.sum())} owned", flush=True)
        Ob, Lb = tt.tree_attn_fwd(bt, bp, qb_, kb_, vb_)
        gq, gk, gv = tt.tree_attn_bwd(bt, bp, qb_, kb_, vb_, Ob, Lb, dob)
        sdq.index_add_(0, rows, gq.float())
        sdk.index_add_(0, rows, gk.float())
        sdv.index_add_(0, rows, gv.float())
        bo[rows] = Ob.float()
        bl[rows] = Lb
    assert bool(owned.all())
    for n, x, y in (("o", O, bo), ("lse", L, bl), ("dq", dq, sdq), ("dk", dk, sdk), ("dv", dv, sdv)):
        ref = y.cpu().double().numpy()
        e, er = rel_err(x, ref), row_rel_err(x, ref)
        print(f"  {n}: tensor {e:.2e}  per-row {er:.2e}", flush=True)
        assert e < TOL and (n == "dq" or er < TOL), (n, e, er)


def test_mfma_past_4gib():
    """Query-side tensors past 4 GiB (a forest of 260 chains of 2048 tokens,
    N = 532,480 rows x 32 heads: Q, dO, O and dQ hold 4.36 GB each), so the
    dK/dV kernel's Q/dO tiles sit beyond any 32-bit byte offset: rows and keys
    at the end of the tensors against the oracle's per-row computation."""
    n_seq, Ls = 260, 2048
    rng = ts.rng_for(61)
    seqs = [np.concatenate([[s_], rng.integers(0, 151936, Ls - 1)]).astype(np.int32)
            for s_ in rng.choice(151936, n_seq, replace=False)]
    tree = tt.Tree(seqs)
    o = dfs_arrays(seqs)
    N = tree.N
    assert N * 32 * 128 * 2 > 4 * 2 ** 30
    g = torch.Generator(device="cuda").manual_seed(62)
    mk = lambda *sh, std=128 ** -0.5: (torch.randn(*sh, device="cuda", generator=g) * std).to(torch.bfloat16)  # noqa
    q, k, v, do = mk(N, 32, 128), mk(N, 8, 128), mk(N, 8, 128), mk(N, 32, 128, std=1.0)
    plan = tree.upload_plan()
    print(f"N={N}", flush=True)
    O, L = tt.tree_attn_fwd(tree, plan, q, k, v)
    dq, dk, dv = tt.tree_attn_bwd(tree, plan, q, k, v, O, L, do)
    torch.cuda.synchronize()

    def get(name, idx):
        src = {"q": q, "k": k, "v": v, "do": do}[name]
        return src[torch.as_tensor(np.asarray(idx, dtype=np.int64), device="cuda")].double().cpu().numpy()

    rows = np.array([N - 1, N - 2, N - 64, N - 65, N - Ls + 3, N // 2 + 5, 17])
    Or, Lr = OA.forward_rows(o, None, None, None, rows, get=get)
    ri = torch.as_tensor(rows, device="cuda")
    assert rel_err(O[ri], Or) < TOL and rel_err(L[ri], Lr) < TOL
    assert rel_err(dq[ri], OA.dq_rows(o, None, None, None, None, rows, get=get)) < TOL
    keys = np.array([N - 1, N - 3, N - 20, N - 64])
    rk, rv = OA.dkdv_keys(o, None, None, None, None, keys, get=get)
    ki = torch.as_tensor(keys, device="cuda")
    assert rel_err(dk[ki], rk) < TOL and rel_err(dv[ki], rv) < TOL
