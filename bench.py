#!/usr/bin/env python3
"""Benchmark of the prefix-tree attention hot path on one MI355X.

Headline workload (one "step"): forward + backward tree attention over the
8B-class agentic tree (32 query heads, 8 kv heads, head dim 128, bf16,
RoPE at depth): beam of depth 10 from a 4096-token root, branch 2, 16 kept,
segments U[512, 2048], random leaves dropped until <= 67.2k unique tokens.
Inputs are resident in HBM before the timed region; the host trie build and
plan upload happen once, outside it, and are reported separately.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  value = unique tree tokens per second of the
forward+backward step; useful TFLOP/s counts visible (query, key) pairs only:
forward 4 d Hq P, backward 10 d Hq P (P = sum over rows of depth + 1).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "tree attn fwd+bwd unique tokens/s + useful TFLOP/s (% bf16 MFMA peak), 8B shape"

# HBM traffic of the roofline kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs (scaled by the same counters' reading for a plain copy of known size),
# valid only for the kernel source and the host scheduler (which sets the
# workgroups' launch order) it was measured on.
MEASURED_TRAFFIC = {"kernel": "attn_bwd_mfma", "source_sha1": "93ae87b661496ab5379cc8f17ad4dd61b4f5ae3a",
                    "bytes_per_launch": 19766407624}


def _source_sha(*paths):
    """sha1 of source code (the files in order): // comments and blank lines
    removed, so that a comment edit does not invalidate a traffic measurement."""
    lines = []
    for path in paths:
        with open(path, encoding="utf-8") as f:
            lines += [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha1("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def _bf16(t):
    import torch
    return t.to(torch.bfloat16)


def _make_inputs(N, hq, hkv, d, seed, device="cuda"):
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    s = d ** -0.5
    q = _bf16(torch.randn(N, hq, d, device=device, generator=g) * s)
    k = _bf16(torch.randn(N, hkv, d, device=device, generator=g) * s)
    v = _bf16(torch.randn(N, hkv, d, device=device, generator=g) * s)
    do = _bf16(torch.randn(N, hq, d, device=device, generator=g))
    return q, k, v, do


class Step:
    """Preallocated fwd+bwd over one tree (or one chunk of a path); the
    backward takes the forward's rotated q and k from the shared workspace."""

    def __init__(self, tt, tree, plan, q, k, v, do, q_off=0, accumulate=False, d_k=None, d_v=None):
        import torch
        self.tt, self.tree, self.plan = tt, tree, plan
        self.q, self.k, self.v, self.do, self.q_off = q, k, v, do, q_off
        self.o = torch.empty_like(q)
        self.lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
        self.dq = torch.empty_like(q)
        self.accumulate = accumulate
        self.dk = d_k if d_k is not None else torch.empty_like(k)
        self.dv = d_v if d_v is not None else torch.empty_like(v)
        nb = max(tt.attn_workspace_bytes(tree, plan, q, k, v, True, q_off=q_off),
                 tt.attn_workspace_bytes(tree, plan, q, k, v, False, q_off=q_off))
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)

    def fwd(self):
        self.tt.tree_attn_fwd(self.tree, self.plan, self.q, self.k, self.v, q_off=self.q_off, o=self.o,
                              lse=self.lse, workspace=self.ws)

    def bwd(self):
        self.tt.tree_attn_bwd(self.tree, self.plan, self.q, self.k, self.v, self.o, self.lse, self.do,
                              q_off=self.q_off, d_q=self.dq, d_k=self.dk, d_v=self.dv,
                              accumulate=self.accumulate, workspace=self.ws, reuse_rotated=True)


def _time(fn, steps, warmup, min_warm_s=0.1):
    """Mean time of `steps` calls between two events.  The warm-up runs at
    least `warmup` calls and at least min_warm_s of wall time, so that a
    sub-millisecond call is timed at the clock the chip reaches under load,
    not while it ramps up from idle."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        fn()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _graph(fn):
    """fn captured into a HIP graph (after two warm-up calls on a side stream)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _graph_time(fn, steps, warmup):
    """_time of fn's graph replay, or None (with the reason on stderr) when
    capture is not available: the measurement is an extra beside the
    eager one, not a reason to stop the run."""
    try:
        return _time(_graph(fn).replay, steps, warmup)
    except Exception as e:  # noqa: BLE001
        print(f"graph replay not measured: {e}", file=sys.stderr, flush=True)
        return None


def secondary(tt, ts, steps):
    """Shorter measurements of the other configurations (not the headline)."""
    import numpy as np
    import torch
    out = {}
    # tiny tree, fp32, 1 head, d 64: forward + backward + weighted NLL over vocab 1000
    case = ts.tiny_tree(0)
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    g = torch.Generator(device="cuda").manual_seed(13)
    q, k, v, do = (torch.randn(tree.N, 1, 64, device="cuda", generator=g) for _ in range(4))
    z = torch.randn(tree.N, 1000, device="cuda", generator=g)
    a = tree.export()
    rp, tid, tw = (torch.from_numpy(np.ascontiguousarray(a[n])).cuda() for n in ("tgt_row_ptr", "tgt_token", "tgt_w"))

    def tiny():
        o, lse = tt.tree_attn_fwd(tree, plan, q, k, v)
        tt.tree_attn_bwd(tree, plan, q, k, v, o, lse, do)
        tt.tree_weighted_nll(rp, tid, tw, logits=z)

    ms = _time(tiny, 20, 3)
    # the same step with preallocated outputs, captured once and replayed as a HIP graph
    o, lse = torch.empty_like(q), torch.empty(tree.N, 1, dtype=torch.float32, device="cuda")
    dq, dk, dv, dz = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z)

    def tiny_pre():
        tt.tree_attn_fwd(tree, plan, q, k, v, o=o, lse=lse)
        tt.tree_attn_bwd(tree, plan, q, k, v, o, lse, do, d_q=dq, d_k=dk, d_v=dv)
        tt.tree_weighted_nll(rp, tid, tw, logits=z, d_logits=dz)

    ms_pre = _time(tiny_pre, 20, 3)
    ms_graph = _graph_time(tiny_pre, 20, 3)
    out["tiny_tree_fp32"] = dict(N=tree.N, pairs=tree.info["pairs"], ms=round(ms, 4), ms_preallocated=round(ms_pre, 4),
                                 ms_graph_replay=round(ms_graph, 4) if ms_graph is not None else None,
                                 note="fwd + bwd + NLL (vocab 1000): outputs allocated per call, preallocated, "
                                      "and the preallocated step replayed as a HIP graph; launch-bound")
    d = 128
    # 1.7B-class forward on the RL forest (16 q heads, 8 kv heads)
    case = ts.rl_forest_accepted(0)
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    q, k, v, do = _make_inputs(tree.N, 16, 8, d, 11)
    st = Step(tt, tree, plan, q, k, v, do)
    ms = _time(st.fwd, steps, 2)
    fl = 4 * d * 16 * tree.info["pairs"]
    out["rl_forest_1p7b_fwd"] = dict(N=tree.N, seed=case.seed, compression=round(case.seq_tokens / tree.N, 3),
                                     ms=round(ms, 4), tokens_per_s=round(tree.N / ms * 1e3),
                                     useful_tflops=round(fl / ms / 1e9, 1),
                                     pct_bf16_peak=round(fl / ms / 1e9 / PEAK_BF16_TFLOPS * 100, 2))

    dense = per_branch_dense(tt, ts, tree, case, q, k, v, do, steps, fwd_only=True)
    out["rl_forest_1p7b_fwd"]["per_branch_dense"] = dict(dense, tree_speedup=round(dense["ms"] / ms, 3),
                                                         pair_ratio=round(tree.info["dense_pairs"] /
                                                                          tree.info["pairs"], 3))

    def fwd_bwd():
        st.fwd()
        st.bwd()

    # the same forest through forward + backward (not part of the forward-only
    # configuration; the GQA-2 backward runs as separate dQ and dK/dV launches)
    ms2 = _time(fwd_bwd, steps, 2)
    fl2 = 14 * d * 16 * tree.info["pairs"]
    out["rl_forest_1p7b_fwd_bwd"] = dict(ms=round(ms2, 4), useful_tflops=round(fl2 / ms2 / 1e9, 1),
                                         pct_bf16_peak=round(fl2 / ms2 / 1e9 / PEAK_BF16_TFLOPS * 100, 2))
    del st, q, k, v, do
    # path mode: 49,152-token chain, 16k suffix in 2048-token chunks right to left against a 32k prefix
    case = ts.long_chain(0)
    tree = tt.Tree(case.seqs)
    plan = tree.upload_plan()
    L, prefix, chunk = 49152, 32768, 2048
    q, k, v, do = _make_inputs(L, 32, 8, d, 12)
    dk = torch.zeros(L, 8, d, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    steps_c = []
    for s in reversed(range(prefix, L, chunk)):
        e = min(L, s + chunk)
        steps_c.append(Step(tt, tree, plan, q[s:e], k[:e], v[:e], do[s:e], q_off=s, accumulate=True,
                            d_k=dk[:e], d_v=dv[:e]))

    def path_step():
        for sc in steps_c:
            sc.fwd()
            sc.bwd()

    ms = _time(path_step, max(2, steps // 2), 1)
    P = sum(chunk * (s + 1) + chunk * (chunk - 1) // 2 for s in range(prefix, L, chunk))
    fl = 14 * d * 32 * P
    out["chain_path_mode_8b"] = dict(chunks=len(steps_c), chunk=chunk, prefix=prefix, pairs_per_head=P,
                                     ms=round(ms, 3), ms_per_chunk=round(ms / len(steps_c), 3),
                                     useful_tflops=round(fl / ms / 1e9, 1),
                                     pct_bf16_peak=round(fl / ms / 1e9 / PEAK_BF16_TFLOPS * 100, 2))
    del steps_c, q, k, v, do, dk, dv
    torch.cuda.empty_cache()
    out["lmhead_weighted_nll"] = lmhead_bench(tt, ts, steps)
    return out


def path_mode_bench(tt, tree, plan, q, k, v, do, steps, tree_ms):
    """Path mode on the headline tree: depth-first walk with a stack of the
    current path, each segment's forward on entry and backward (right-to-left
    chunks) on exit.  The pages' chunk sizes 2048 and 4096 and both child
    orders; time against tree mode, recompute (pad rows) and workspace.
    vs_tree_mode compares each walk with the tree-mode step timed right
    before it (same number of calls), so that both run at the same clock;
    vs_tree_mode_headline compares it with the headline step, timed seconds
    earlier."""
    import torch
    d, hq = q.shape[2], q.shape[1]
    P = tree.info["pairs"]
    useful = 14 * d * hq * P
    o, lse = torch.empty_like(q), torch.empty(q.shape[0], hq, dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    out = {"tree_mode_ms": round(tree_ms, 3),
           "tree_mode_workspace_bytes": tt.attn_workspace_bytes(tree, plan, q, k, v, True)}
    tree_step = Step(tt, tree, plan, q, k, v, do)

    def tree_fwd_bwd():
        tree_step.fwd()
        tree_step.bwd()

    for chunk, order in ((2048, 0), (4096, 0), (2048, 1), (4096, 1)):
        path = tt.Path(tree, chunk, order)
        nbytes = tt.path_workspace_bytes(path, q, k, v, True)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)

        def walk():
            tt.tree_attn_path(path, q, k, v, d_o=do, o=o, lse=lse, d_q=dq, d_k=dk, d_v=dv, workspace=ws)

        n = max(2, steps // 2)
        ms_tree = _time(tree_fwd_bwd, n, 1)
        ms = _time(walk, n, 1)
        # the whole walk (about 180 launches) captured once and replayed as a HIP graph
        ms_graph = _graph_time(walk, n, 1) if (chunk, order) == (2048, 0) else None
        tt.timing_enable(True)
        walk()
        torch.cuda.synchronize()
        tt.timing_enable(False)
        kt = tt.timing_collect()
        inf = path.info
        out[f"chunk{chunk}_{'dfs' if order == 0 else 'greedy'}"] = dict(
            ms=round(ms, 3), tree_mode_ms_adjacent=round(ms_tree, 3), vs_tree_mode=round(ms / ms_tree, 3),
            vs_tree_mode_headline=round(ms / tree_ms, 3), kernel_ms=round(sum(x[1] for x in kt.values()), 3),
            launches=int(sum(x[0] for x in kt.values())), segments=inf["n_segments"], calls=inf["fwd_calls"],
            bwd_calls=inf["bwd_calls"], max_path=inf["max_path"], pad_rows=inf["pad_rows"],
            pad_pairs_per_head=inf["pad_pairs"], recompute_pct=round(100.0 * inf["pad_pairs"] / (2 * P), 3),
            useful_tflops=round(useful / ms / 1e9, 1),
            pct_bf16_peak=round(useful / ms / 1e9 / PEAK_BF16_TFLOPS * 100, 2), workspace_bytes=nbytes,
            kernels={n_: {"launches": x[0], "total_ms": round(x[1], 3)} for n_, x in kt.items()})
        if ms_graph is not None:  # measured for chunk 2048, DFS order only
            out[f"chunk{chunk}_dfs"].update(ms_graph_replay=round(ms_graph, 3),
                                             graph_vs_tree_mode=round(ms_graph / ms_tree, 3))
        del ws, path
    del tree_step
    return out


def lmhead_bench(tt, ts, steps, dense=True):
    """Fused lm-head + weighted NLL: 16384 tree tokens x 4096 -> 151936 vocabulary,
    32-leaf tree (compression about 5.5); loss, dH and dW (fp32)."""
    import numpy as np
    import torch
    case = ts.lmhead_tree(0)
    tree = tt.Tree(case.seqs)
    a = tree.export()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    rp, tid, tw = dev(a["tgt_row_ptr"]), dev(a["tgt_token"]), dev(a["tgt_w"])
    N, dm, V = tree.N, 4096, 151936
    g = torch.Generator(device="cuda").manual_seed(21)
    H = _bf16(torch.randn(N, dm, device="cuda", generator=g))
    W = _bf16(torch.randn(dm, V, device="cuda", generator=g) * 0.02)
    ws = None
    out = tt.tree_weighted_nll(rp, tid, tw, hidden=H, w_vocab=W)
    dh, dw = out["d_hidden"], out["d_w_vocab"]

    def call():
        nonlocal ws
        o = tt.tree_weighted_nll(rp, tid, tw, hidden=H, w_vocab=W, workspace=ws)
        return o

    # keep one workspace alive across calls
    import ctypes  # noqa: F401
    nb = tt.NllArgs(n_rows=N, d_model=dm, vocab=V, n_tgt=int(tid.numel()), hidden=1, w_vocab=1)
    n = ctypes.c_size_t()
    tt.lib().tree_nll_workspace_bytes(ctypes.byref(nb), ctypes.byref(n))
    ws = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    del dh, dw, out
    call()
    torch.cuda.synchronize()
    tt.timing_enable(True)
    ms = _time(call, max(2, steps // 3), 0)
    tt.timing_enable(False)
    kt = tt.timing_collect()
    fl = 6 * N * dm * V
    red = kt.get("nll_rows", (1, 0.0, 0.0))
    red_ms = red[1] / max(1, red[0])
    zbytes = 2 * N * V * 2  # read Z once, write dZ once (bf16)
    res = dict(rows=N, d_model=dm, vocab=V, compression=round(case.seq_tokens / N, 3), ms=round(ms, 3),
               useful_tflops=round(fl / ms / 1e9, 1), pct_bf16_peak=round(fl / ms / 1e9 / PEAK_BF16_TFLOPS * 100, 2),
               nll_reduce_ms=round(red_ms, 3), nll_reduce_gbs=round(zbytes / red_ms / 1e6, 1),
               kernels={k_: {"launches": c, "avg_ms": round(t / c, 3)} for k_, (c, t, _) in kt.items()})
    del ws
    torch.cuda.empty_cache()
    if dense:
        try:
            res["per_branch_dense"] = lmhead_dense(tt, tree, case, H, W, res["ms"],
                                                   float(out_loss(rp, tid, tw, H, W, tt)))
        except torch.cuda.OutOfMemoryError as e:  # ~35 GB of device memory
            res["per_branch_dense"] = {"error": f"not measured: {e}"}
            torch.cuda.empty_cache()
    del H, W
    torch.cuda.empty_cache()
    return res


def out_loss(rp, tid, tw, H, W, tt):
    return tt.tree_weighted_nll(rp, tid, tw, hidden=H, w_vocab=W)["loss"].item()


def lmhead_dense(tt, tree, case, H, W, tree_ms, tree_loss):
    """The per-branch equivalent of the fused lm-head: every input sequence's
    rows on their own (the tree rows gathered through seq_pos_to_dfs), each
    position's target the sequence's next token with weight 1/B.  Its loss is
    the tree loss (the branch average) up to rounding; the time is what the
    tree saves."""
    import numpy as np
    import torch
    a = tree.export()
    B = len(case.seqs)
    rows = torch.as_tensor(a["seq_pos_to_dfs"].astype("int64"), device="cuda")
    Hd = H[rows].contiguous()
    ptr, tok = [0], []
    for s_ in case.seqs:
        for k_ in range(len(s_)):
            if k_ + 1 < len(s_):
                tok.append(int(s_[k_ + 1]))
            ptr.append(len(tok))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    rp = dev(np.asarray(ptr, dtype=np.int32))
    tid = dev(np.asarray(tok, dtype=np.int32))
    tw = dev(np.full(len(tok), np.float32(1.0) / np.float32(B), dtype=np.float32))
    loss = tt.tree_weighted_nll(rp, tid, tw, hidden=Hd, w_vocab=W)["loss"].item()

    def call():
        tt.tree_weighted_nll(rp, tid, tw, hidden=Hd, w_vocab=W)

    ms = _time(call, 2, 1)
    n = int(rows.numel())
    res = dict(rows=n, ms=round(ms, 3), rows_per_s=round(n / ms * 1e3), tree_speedup=round(ms / tree_ms, 3),
               row_ratio=round(n / tree.N, 3), loss=round(loss, 4), tree_loss=round(tree_loss, 4),
               loss_rel_diff=float(abs(loss - tree_loss) / abs(tree_loss)))
    del Hd
    torch.cuda.empty_cache()
    return res


def per_branch_dense(tt, ts, tree, case, q, k, v, do, steps, fwd_only=False):
    """The same kernels run on every input sequence as its own chain (no prefix sharing)."""
    import torch
    arr = tree.export()
    offs = [0]
    for s in case.seqs:
        offs.append(offs[-1] + len(s))
    steps_b = []
    for b, s in enumerate(case.seqs):
        rows = torch.as_tensor(arr["seq_pos_to_dfs"][offs[b]:offs[b + 1]].astype("int64"), device="cuda")
        bt = tt.Tree([s])
        bp = bt.upload_plan()
        steps_b.append((bt, Step(tt, bt, bp, q[rows].contiguous(), k[rows].contiguous(), v[rows].contiguous(),
                                 do[rows].contiguous())))

    def run():
        for _, sb in steps_b:
            sb.fwd()
            if not fwd_only:
                sb.bwd()

    ms = _time(run, max(2, steps // 2), 1)
    branch_tokens = sum(len(s) for s in case.seqs)
    del steps_b
    torch.cuda.empty_cache()
    return dict(branches=len(case.seqs), branch_tokens=branch_tokens, ms=round(ms, 3),
                branch_tokens_per_s=round(branch_tokens / ms * 1e3))


def compression_study(tt, ts, steps, prefixes=(7168, 6144, 4096, 2048, 1024, 512, 0)):
    """Where the tree stops paying off: 8 branches of 8192 tokens sharing a
    prefix of p tokens, p from 7168 down to 0 (compression to exactly 1).
    Tree mode (one fwd+bwd over the tree) against the same kernels per branch
    (AReaL-DTA summary, Main Findings: gains shrink as sharing falls)."""
    import types
    import torch
    B, L, hq, hkv, d = 8, 8192, 32, 8, 128
    points = []
    for p in prefixes:
        prefix = list(range(p))
        seqs = [prefix + [200000 + b * L + j for j in range(L - p)] for b in range(B)]
        tree = tt.Tree(seqs)
        plan = tree.upload_plan()
        q, k, v, do = _make_inputs(tree.N, hq, hkv, d, 21)
        st = Step(tt, tree, plan, q, k, v, do)

        def step():
            st.fwd()
            st.bwd()

        ms = _time(step, max(2, steps // 2), 1)
        dense = per_branch_dense(tt, ts, tree, types.SimpleNamespace(seqs=seqs), q, k, v, do, steps)
        inf = tree.info
        points.append(dict(shared_prefix=p, compression=round(B * L / tree.N, 3), unique_tokens=tree.N,
                           tree_ms=round(ms, 3), dense_ms=dense["ms"], tree_speedup=round(dense["ms"] / ms, 3),
                           pair_ratio=round(inf["dense_pairs"] / inf["pairs"], 3)))
        del st, q, k, v, do, tree, plan
        torch.cuda.empty_cache()
    return points


def cpu_baseline(ts, case, seed, budget_s):
    """The fp64 oracle's whole step (forward + backward) on a bounded sample of
    the headline tree, extrapolated to the full step.

    The oracle computes every branch on its own (textbook causal attention of
    L x L per head), so its cost grows with sum over branches of L^2 times
    the query heads.  Sample: a prefix of the longest branch, of L rows, for
    one kv head's group of 4 query heads, forward then backward; L doubles
    from 1024 until one call takes a quarter of the budget, then calls repeat
    until the budget is spent.  Full step = mean call time x (sum_s |s|^2 /
    L^2) x 8 groups; value = unique tree tokens / that time.  A second,
    shorter sample on one BLAS thread gives value_1core the same way."""
    import numpy as np
    from oracle import attention as OA
    from oracle.tree import dfs_arrays
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = 1
    N = len(dfs_arrays(case.seqs)["token"])
    longest = max(case.seqs, key=len)
    rng = ts.rng_for(seed + 77)
    sq = float(sum(len(x) ** 2 for x in case.seqs))
    draw = lambda shape, std: ts.bf16_bits_to_f64(ts.normal_bf16(rng, shape, std))  # noqa: E731

    def one(L):
        o = dfs_arrays([longest[:L]])
        q, k, v, do = draw((L, 4, 128), 128 ** -0.5), draw((L, 1, 128), 128 ** -0.5), \
            draw((L, 1, 128), 128 ** -0.5), draw((L, 4, 128), 1.0)
        t0 = time.perf_counter()
        OA.forward(o, q, k, v)
        OA.backward(o, q, k, v, do)
        return time.perf_counter() - t0

    def measure(budget, L_max):
        L = min(1024, len(longest))
        t = one(L)
        while t < budget / 4 and 2 * L <= min(len(longest), L_max):
            L *= 2
            t = one(L)
        times, t_all = [t], t
        while t_all + t < budget:
            times.append(one(L))
            t_all += times[-1]
        mean = float(np.mean(times))
        full = mean * (sq / L ** 2) * 8
        return L, len(times), mean, full

    L, n, mean, full = measure(budget_s, 8192)
    one_core = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            L1, n1, mean1, full1 = measure(budget_s / 3, 4096)
        one_core = round(N / full1, 3)
    return {"value": round(N / full, 3), "unit": "unique tokens/s (forward + backward, extrapolated)",
            "cores": threads, "value_1core": one_core, "kind": "oracle",
            "extrapolated_step_s": round(full, 1),
            "sample": f"{n} oracle calls (fp64 numpy per-branch forward + backward) on the first {L} rows of the "
                      f"longest branch for one kv head's 4 query heads, {mean:.2f} s each; the full step (all "
                      f"{len(case.seqs)} branches of the {N}-row tree, 32 heads) is extrapolated by "
                      f"sum_s |s|^2 / L^2 = {sq / L ** 2:.1f} and 8 head groups to {full:.0f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-dense", action="store_true", help="skip the per-branch dense comparison")
    ap.add_argument("--no-path", action="store_true", help="skip the path-mode walk of the headline tree")
    ap.add_argument("--lmhead-only", action="store_true",
                    help="only run the lm-head measurement and print it (for profiling its kernels)")
    ap.add_argument("--study", action="store_true",
                    help="only run the compression sweep (tree vs per-branch dense) and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        x = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": x.numel() * 2, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (sharding across GPUs is "
                                   "described in the design notes, not implemented)"}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import prefix_tree_attention_dfs_amd as tt
    import treesynth as ts

    torch.cuda.set_device(0)
    if args.lmhead_only:
        print(json.dumps({"lmhead_weighted_nll": lmhead_bench(tt, ts, args.steps, dense=not args.no_dense)}),
              flush=True)
        return
    if args.study:
        print(json.dumps({"study": "compression_sweep", "workload": "8 branches x 8192 tokens, shared prefix p, "
                          "Hq 32, Hkv 8, d 128, bf16 fwd+bwd", "points": compression_study(tt, ts, args.steps)}),
              flush=True)
        return
    t0 = time.perf_counter()
    case = ts.agentic_beam_tree(args.seed)
    gen_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    tree = tt.Tree(case.seqs)
    build_ms = (time.perf_counter() - t0) * 1e3
    plan = tree.upload_plan()
    info = tree.info
    N, hq, hkv, d = tree.N, 32, 8, 128
    P = info["pairs"]
    q, k, v, do = _make_inputs(N, hq, hkv, d, args.seed + 1)
    st = Step(tt, tree, plan, q, k, v, do)

    def step():
        st.fwd()
        st.bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tt.timing_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    tt.timing_enable(False)
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    ms_median = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]))
    kt = tt.timing_collect()
    sustained = tt.probe_mfma()  # dense bf16 MFMA rate the chip sustains (clock under load included)

    useful = 14 * d * hq * P  # forward 4 d Hq P + backward 10 d Hq P (S recompute counted)
    value = N / (ms * 1e-3)
    tflops = useful / (ms * 1e-3) / 1e12
    tflops_strict = 12 * d * hq * P / (ms * 1e-3) / 1e12  # backward counted as 8 d Hq P
    # roofline of the dominant kernel (largest share of the step's device time)
    algo = {"attn_fwd_mfma": 4 * d * hq * P, "attn_bwd_dkdv_mfma": 8 * d * hq * P,
            "attn_bwd_dq_mfma": 6 * d * hq * P,
            "attn_bwd_mfma": 14 * d * hq * P}  # dQ (S, dP recomputed; dQ) and dK/dV (S, dP, dV, dK) in one launch
    dom = max(kt, key=lambda n: kt[n][1])
    launches, tot, mx = kt[dom]
    avg_ms = tot / launches
    achieved = algo.get(dom, 0) / (avg_ms * 1e-3) / 1e12
    csrc = os.path.join(ROOT, "prefix_tree_attention_dfs_amd", "csrc")
    src = os.path.join(csrc, "attn_mfma.hip" if dom == "attn_fwd_mfma" else "attn_mfma_bwd.hip")
    traffic = None
    if MEASURED_TRAFFIC and MEASURED_TRAFFIC.get("kernel") == dom and \
            MEASURED_TRAFFIC.get("source_sha1") == _source_sha(src, os.path.join(csrc, "tree_host.cpp")):
        traffic = MEASURED_TRAFFIC["bytes_per_launch"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "avg_launch_ms": round(avg_ms, 4),
                "algorithmic_flops_per_launch": algo.get(dom, 0),
                "peak_sustained": round(sustained, 1), "frac_sustained": round(achieved / sustained, 4)}
    kernels = {n: {"launches": c, "avg_ms": round(t / c, 4), "max_ms": round(m, 4),
                   "share": round(t / sum(x[1] for x in kt.values()), 4)} for n, (c, t, m) in kt.items()}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "unique tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_median, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "8B-class agentic tree fwd+bwd (Hq 32, Hkv 8, d 128, RoPE at depth)",
                   "unique_tokens": N, "seq_tokens": info["seq_tokens"], "leaves": info["n_leaves"],
                   "max_depth": info["max_depth"], "pairs_per_head": P, "seed": args.seed,
                   "tiles_64x64": info["n_tiles"], "full_tiles": info["n_full_tiles"],
                   "generator": dict(name="agentic_beam_tree", rng="numpy PCG64", seed=case.seed, **case.params),
                   "tensors": "torch CUDA generator seeded seed+1: q, k, v ~ N(0,1)/sqrt(128), dO ~ N(0,1), bf16"},
        "useful_tflops": round(tflops, 1), "pct_bf16_peak": round(tflops / PEAK_BF16_TFLOPS * 100, 2),
        "useful_tflops_strict": round(tflops_strict, 1),
        "pct_bf16_peak_strict": round(tflops_strict / PEAK_BF16_TFLOPS * 100, 2),
        "sustained_mfma_tflops": round(sustained, 1),
        "pct_sustained_mfma": round(tflops / sustained * 100, 2),
        "roofline": roofline, "kernels": kernels,
        "tree_build_ms": round(build_ms, 2), "tree_gen_s": round(gen_s, 2),
    }
    if not args.no_dense:
        dense = per_branch_dense(tt, ts, tree, case, q, k, v, do, args.steps)
        dense["tree_speedup"] = round(dense["ms"] / ms, 3)
        result["per_branch_dense"] = dense
    if not args.no_path:
        result["path_mode"] = path_mode_bench(tt, tree, plan, q, k, v, do, args.steps, ms)
    del st
    torch.cuda.empty_cache()
    if not args.no_secondary:
        result["secondary"] = secondary(tt, ts, args.steps)
        result["study"] = {"name": "compression_sweep", "workload": "8 branches x 8192 tokens sharing a prefix of "
                           "p tokens, Hq 32, Hkv 8, d 128, bf16 fwd+bwd; tree mode vs the same kernels per branch",
                           "points": compression_study(tt, ts, args.steps, prefixes=(7168, 4096, 1024, 0))}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(ts, case, args.seed, args.cpu_seconds)
        cb["gpu_over_cpu"] = round(value / cb["value"], 1)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
