"""Host side of libtreeattn against the oracle (CPU only, no GPU needed).

* tree_build's DFS arrays are bit-exact with the oracle's (lexicographic
  prefix order) on random sets and on every workload generator;
* the tile schedule equals brute-force enumeration of visible pairs;
* the library exports every symbol declared in include/tt.h;
* every host-checkable error path returns its negative status.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle.metrics import metrics
from oracle.schedule import tiles as oracle_tiles
from oracle.tree import dfs_arrays

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _compare(seqs, block_q=0, block_k=0):
    t = tt.Tree(seqs, block_q=block_q, block_k=block_k)
    a = t.export()
    o = dfs_arrays(seqs)
    assert t.N == o["N"]
    for key in ("token", "depth", "end", "parent", "n_pass", "seq_pos_to_dfs", "tgt_row_ptr", "tgt_dfs"):
        np.testing.assert_array_equal(a[key].astype(np.int64), o[key], err_msg=key)
    assert a["weight"].tobytes() == o["weight"].tobytes()          # bit-exact float32
    np.testing.assert_array_equal(a["tgt_token"], o["token"][o["tgt_dfs"]])
    assert a["tgt_w"].tobytes() == o["weight"][o["tgt_dfs"]].tobytes()
    m = metrics(seqs, o)
    inf = t.info
    assert inf["n_seqs"] == len(seqs)
    assert inf["n_roots"] == o["n_roots"] and inf["n_leaves"] == o["n_leaves"]
    assert inf["max_depth"] == o["max_depth"]
    assert inf["seq_tokens"] == m["seq_tokens"] and inf["leaf_tokens"] == m["leaf_tokens"]
    assert inf["pairs"] == m["pairs"] and inf["dense_pairs"] == m["dense_pairs"]
    assert inf["n_targets"] == len(o["tgt_dfs"])
    return t, o


RANDOM = [ts.random_small_tree(s, n_seqs=n, max_len=L, vocab=v, p_empty=pe)
          for s, (n, L, v, pe) in enumerate(
              [(1, 1, 3, 0.0), (4, 30, 2, 0.0), (9, 40, 3, 0.1), (15, 20, 4, 0.2), (30, 60, 5, 0.05),
               (3, 200, 1000, 0.0), (50, 10, 2, 0.0), (8, 120, 3, 0.0)] * 3)]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: f"seed{c.seed}")
def test_tree_bit_exact_random(case):
    _compare(case.seqs)


def test_tree_bit_exact_workloads():
    _compare(ts.tiny_tree(0).seqs)
    _compare(ts.rl_forest_accepted(0).seqs)
    _compare(ts.agentic_beam_tree(0).seqs)
    _compare(ts.long_chain(0).seqs)
    _compare(ts.lmhead_tree(0).seqs)


def test_tree_edge_cases():
    # no sequences; only empty sequences; duplicates; one token
    t, _ = _compare([])
    assert t.N == 0 and t.info["max_depth"] == -1 and t.info["n_tiles"] == 0
    t, _ = _compare([np.zeros(0, np.int32)] * 3)
    assert t.N == 0 and t.info["n_seqs"] == 3
    t, o = _compare([np.array([5, 6, 7])] * 4 + [np.array([5])])
    assert t.N == 3 and list(o["n_pass"]) == [5, 4, 4]
    _compare([np.array([0])])
    # large token ids near INT32_MAX
    _compare([np.array([2**31 - 1, 0, 2**31 - 2]), np.array([2**31 - 1, 1])])


@pytest.mark.parametrize("case", RANDOM[:12], ids=lambda c: f"seed{c.seed}")
@pytest.mark.parametrize("blocks", [(16, 16), (32, 16), (16, 64), (64, 64)])
def test_schedule_equals_bruteforce(case, blocks):
    bq, bk = blocks
    t = tt.Tree(case.seqs, block_q=bq, block_k=bk)
    o = dfs_arrays(case.seqs)
    s = t.schedule()
    assert s["bq"] == bq and s["bk"] == bk
    assert s["tiles"] == oracle_tiles(o["parent"], bq, bk)
    assert t.info["n_tiles"] == len(s["tiles"]) and t.info["n_full_tiles"] == sum(s["tiles"].values())
    np.testing.assert_array_equal(s["depth"], o["depth"])
    np.testing.assert_array_equal(s["end"], o["end"])
    # per key block: rows that see some key of it are exactly [first key, max end)
    N = o["N"]
    for kb in range(len(s["kb_qlo"])):
        keys = range(kb * bk, min(N, kb * bk + bk))
        seen = {i for j in keys for i in range(j, int(o["end"][j]))}
        assert seen == set(range(s["kb_qlo"][kb], s["kb_qhi"][kb]))
        assert s["kb_minend"][kb] == min(int(o["end"][j]) for j in keys)
    # launch orders: q-blocks from the last row up; groups of 256 keys by the
    # end of the rows that see them, latest first, ties in key order
    nqb = len(s["qb_ptr"]) - 1
    assert list(s["qb_order"]) == list(range(nqb - 1, -1, -1))
    gb = max(1, 256 // bk)
    ng = -(-len(s["kb_qlo"]) // gb)
    gend = [max(int(o["end"][j]) for j in range(g * gb * bk, min(N, (g + 1) * gb * bk))) for g in range(ng)]
    assert list(s["kb_order"]) == sorted(range(ng), key=lambda g: (-gend[g], g))


def test_schedule_workload_chain_and_tiny():
    t = tt.Tree(ts.long_chain(0, length=1000).seqs)
    s = t.schedule()
    nb = (1000 + 63) // 64
    assert set(s["tiles"]) == {(q, k) for q in range(nb) for k in range(q + 1)}
    assert all(v == (k < q) for (q, k), v in s["tiles"].items())
    t = tt.Tree(ts.tiny_tree(0).seqs)
    o = dfs_arrays(ts.tiny_tree(0).seqs)
    assert t.schedule()["tiles"] == oracle_tiles(o["parent"], 64, 64)


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "tt.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"^\s*(?:int|void|const char\*)\s+(\w+)\s*\(", hdr, flags=re.M))
    assert {"tree_build", "tree_attn_fwd", "tree_attn_bwd", "tree_weighted_nll"} <= names
    lib = ctypes.CDLL(tt.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(tt.EXPORTED) == names


# ------------------------------------------------------------------ error paths (host only)
def _build_raw(tokens, offs, n_seqs, bq=0, bk=0):
    lib = tt.lib()
    h = ctypes.c_void_p()
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    off = None if offs is None else np.ascontiguousarray(offs, dtype=np.int64)
    rc = lib.tree_build(None if tok is None else tok.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                        None if off is None else off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                        n_seqs, bq, bk, ctypes.byref(h))
    if rc == 0:
        lib.tree_free(h)
    else:
        assert not h.value
    return rc


def test_tree_build_errors():
    assert _build_raw([1, 2], [0, 2], 1) == tt.TT_OK
    assert _build_raw([1, 2], [1, 2], 1) == tt.TT_EINVAL            # offsets[0] != 0
    assert _build_raw([1, 2], [0, 2, 1], 2) == tt.TT_EINVAL         # decreasing
    assert _build_raw([1, -2], [0, 2], 1) == tt.TT_EINVAL           # negative token
    assert _build_raw(None, [0, 2], 1) == tt.TT_EINVAL              # tokens NULL
    assert _build_raw([1], None, 1) == tt.TT_EINVAL                 # offsets NULL
    assert _build_raw([1], [0, 1], -1) == tt.TT_EINVAL
    assert _build_raw([1], [0, 1], 1 << 24) == tt.TT_EOVERFLOW      # B too large for exact weights
    assert _build_raw([1], [0, 1], 1, bq=48) == tt.TT_EINVAL
    assert _build_raw([1], [0, 1], 1, bk=512) == tt.TT_EINVAL
    assert _build_raw(None, [0], 0) == tt.TT_OK                     # empty input is fine
    assert "non-decreasing" in (_build_raw([1, 2], [0, 2, 1], 2) and tt.last_error())
    lib = tt.lib()
    assert lib.tree_build(None, None, 0, 0, 0, None) == tt.TT_EINVAL
    inf = tt.TreeInfo()
    assert lib.tree_info(None, ctypes.byref(inf)) == tt.TT_EINVAL
    t = tt.Tree([np.arange(10)])
    small = np.zeros(4, dtype=np.int32)
    assert lib.tree_plan_copy(t.handle, small.ctypes.data_as(ctypes.c_void_p), 16) == tt.TT_EWORKSPACE


FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced: validation fails first


def _attn(t, **kw):
    a = tt.AttnArgs(tree=t.handle, plan=FAKE, q_off=0, n_q=t.N, n_k=t.N, h_q=4, h_kv=2, d=128, dtype=tt.TT_BF16,
                    scale=0.0, rope_base=10000.0, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, workspace=FAKE,
                    workspace_bytes=1 << 40)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_attention_argument_errors():
    lib = tt.lib()
    t = tt.Tree([np.arange(100), np.arange(50)])
    cases = [
        (dict(h_q=3, h_kv=2), tt.TT_EINVAL),
        (dict(h_kv=0), tt.TT_EINVAL),
        (dict(d=100), tt.TT_EUNSUPPORTED),
        (dict(d=7), tt.TT_EINVAL),
        (dict(d=512), tt.TT_EUNSUPPORTED),
        (dict(dtype=7), tt.TT_EINVAL),
        (dict(n_k=t.N + 1), tt.TT_EINVAL),
        (dict(q_off=64, n_q=t.N), tt.TT_EINVAL),          # q_off + n_q > n_k
        (dict(q_off=32, n_q=10), tt.TT_EINVAL),           # q_off not a multiple of block_q
        (dict(q_off=-64), tt.TT_EINVAL),
        (dict(q=0), tt.TT_EINVAL),
        (dict(v=0), tt.TT_EINVAL),
        (dict(lse=0), tt.TT_EINVAL),
        (dict(plan=0), tt.TT_EINVAL),
        (dict(tree=0), tt.TT_EINVAL),
        (dict(k=FAKE + 2), tt.TT_EINVAL),                 # misaligned
        (dict(scale=-1.0), tt.TT_EINVAL),
        (dict(rope_base=float("nan")), tt.TT_EINVAL),
        (dict(workspace_bytes=16), tt.TT_EWORKSPACE),
        (dict(workspace=0), tt.TT_EWORKSPACE),
    ]
    for kw, want in cases:
        a = _attn(t, **kw)
        assert lib.tree_attn_fwd(ctypes.byref(a), None) == want, kw
        b = tt.AttnBwdArgs(a=a, d_o=FAKE, d_q=FAKE, d_k=FAKE, d_v=FAKE, flags=0)
        assert lib.tree_attn_bwd(ctypes.byref(b), None) == want, kw
    a = _attn(t)
    for kw in (dict(d_o=0), dict(d_k=0), dict(d_q=FAKE + 8), dict(flags=4)):
        b = tt.AttnBwdArgs(a=a, d_o=FAKE, d_q=FAKE, d_k=FAKE, d_v=FAKE, flags=0)
        for k_, v_ in kw.items():
            setattr(b, k_, v_)
        assert lib.tree_attn_bwd(ctypes.byref(b), None) == tt.TT_EINVAL, kw
    assert lib.tree_attn_fwd(None, None) == tt.TT_EINVAL
    n = ctypes.c_size_t()
    assert lib.tree_attn_workspace_bytes(ctypes.byref(_attn(t)), 1, ctypes.byref(n)) == 0
    q_bytes = t.N * 4 * 128 * 2
    assert n.value >= q_bytes + t.N * 2 * 128 * 2 + t.N * 4 * 4 + t.N * 4 * 128 * 4
    # without RoPE the matrix-core forward still needs its scaled query copy; the vector kernels need nothing
    assert lib.tree_attn_workspace_bytes(ctypes.byref(_attn(t, rope_base=0.0)), 0, ctypes.byref(n)) == 0
    assert n.value == (q_bytes + 255) // 256 * 256
    assert lib.tree_attn_workspace_bytes(ctypes.byref(_attn(t, rope_base=0.0, dtype=tt.TT_F32)), 0,
                                         ctypes.byref(n)) == 0
    assert n.value == 0


def test_nll_argument_errors():
    lib = tt.lib()

    def nll(**kw):
        a = tt.NllArgs(n_rows=10, d_model=0, vocab=100, n_tgt=9, logits=FAKE, logits_dtype=tt.TT_F32,
                       tgt_row_ptr=FAKE, tgt_id=FAKE, tgt_w=FAKE, loss=FAKE, workspace=FAKE,
                       workspace_bytes=1 << 30)
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return lib.tree_weighted_nll(ctypes.byref(a), None)

    assert nll(hidden=FAKE, w_vocab=FAKE, d_model=8) == tt.TT_EINVAL     # both modes
    assert nll(logits=0) == tt.TT_EINVAL                                  # no mode
    assert nll(logits=0, hidden=FAKE) == tt.TT_EINVAL                     # fused without w_vocab
    assert nll(vocab=0) == tt.TT_EINVAL
    assert nll(vocab=1 << 20) == tt.TT_EUNSUPPORTED
    assert nll(n_rows=-1) == tt.TT_EINVAL
    assert nll(loss=0) == tt.TT_EINVAL
    assert nll(tgt_id=0) == tt.TT_EINVAL
    assert nll(logits_dtype=5) == tt.TT_EINVAL
    assert nll(d_hidden=FAKE) == tt.TT_EINVAL                             # needs fused mode
    assert nll(loss=FAKE + 4) == tt.TT_EINVAL                             # misaligned
    assert nll(workspace_bytes=8) == tt.TT_EWORKSPACE
    assert nll(logits=0, hidden=FAKE, w_vocab=FAKE, d_model=8, vocab=104, d_logits=FAKE) == tt.TT_EINVAL
    assert nll(logits=0, hidden=FAKE, w_vocab=FAKE, d_model=8, vocab=100) == tt.TT_EUNSUPPORTED  # vocab % 8
    assert nll(logits=0, hidden=FAKE, w_vocab=FAKE, d_model=12, vocab=104) == tt.TT_EUNSUPPORTED  # d_model % 8

    # the no-allocation variant: the same checks, then logits mode only and at most TT_NOALLOC_MAX_ROWS rows
    def noalloc(**kw):
        a = tt.NllArgs(n_rows=10, d_model=0, vocab=100, n_tgt=9, logits=FAKE, logits_dtype=tt.TT_F32,
                       tgt_row_ptr=FAKE, tgt_id=FAKE, tgt_w=FAKE, loss=FAKE)
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return lib.tree_weighted_nll_noalloc(ctypes.byref(a), None)

    assert noalloc(loss=0) == tt.TT_EINVAL
    assert noalloc(vocab=1 << 20) == tt.TT_EUNSUPPORTED
    assert noalloc(logits=0, hidden=FAKE, w_vocab=FAKE, d_model=8, vocab=104) == tt.TT_EUNSUPPORTED
    assert b"logits mode only" in lib.tt_last_error()
    assert noalloc(n_rows=(1 << 20) + 1) == tt.TT_EWORKSPACE
    assert b"static scratch" in lib.tt_last_error()


def test_probe_mfma_validates_before_launch():
    """The matrix-core probe rejects bad sizes and NULL pointers on the host."""
    lib = tt.lib()
    fl = ctypes.c_double()
    dummy = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    assert lib.tt_probe_mfma(0, 10, dummy, None, ctypes.byref(fl)) == tt.TT_EINVAL
    assert lib.tt_probe_mfma(65537, 10, dummy, None, ctypes.byref(fl)) == tt.TT_EINVAL
    assert lib.tt_probe_mfma(4, 0, dummy, None, ctypes.byref(fl)) == tt.TT_EINVAL
    assert lib.tt_probe_mfma(4, (1 << 20) + 1, dummy, None, ctypes.byref(fl)) == tt.TT_EINVAL
    assert lib.tt_probe_mfma(4, 10, None, None, ctypes.byref(fl)) == tt.TT_EINVAL
    assert lib.tt_probe_mfma(4, 10, dummy, None, None) == tt.TT_EINVAL
    assert b"tt_probe_mfma" in lib.tt_last_error()


def _fnv1a_words(words):
    h = 2166136261
    for b in np.asarray(words, dtype="<i4").tobytes():
        h = ((h ^ b) * 16777619) & 0xFFFFFFFF
    return h


def test_plan_identity_word():
    """Header word 17 of the plan image is the FNV-1a hash of the image with
    that word zeroed (the kernels compare it with the tree's own copy before
    reading any plan array).  The image holds structure only, so trees of
    different shape get different identities and trees of one shape (other
    token ids) share one, together with identical, interchangeable images."""
    ids = {}
    for name, seqs in (("tiny", ts.tiny_tree(0).seqs), ("fork", [[1, 2, 3], [1, 2, 4]]),
                       ("fork_other_tokens", [[1, 2, 3], [1, 2, 5]]), ("chain", [[1, 2, 3, 4]]),
                       ("random", ts.random_small_tree(3, n_seqs=6, max_len=90, vocab=4).seqs)):
        p = tt.Tree(seqs).plan_host()
        q = p.copy()
        q[17] = 0
        assert (int(p[17]) & 0xFFFFFFFF) == _fnv1a_words(q)
        ids[name] = (int(p[17]), p.tobytes())
    assert ids["fork"] == ids["fork_other_tokens"]
    shapes = [ids[n][0] for n in ("tiny", "fork", "chain", "random")]
    assert len(set(shapes)) == 4


def test_kernel_envelope_and_plan_registry_on_host():
    """Which shapes the bf16 matrix-core kernels take, decided on the host
    before any launch: head dim 128 at 64-row blocks for any GQA group (1, 2,
    3, 4, 8, 16) goes on to the plan check; another bf16 head dim fails with
    TT_EUNSUPPORTED unless TT_ALLOW_GENERIC asks for the vector kernels;
    float32 always runs the vector kernels.  A plan address the library never
    filled is rejected (TT_EINVAL) after every other check passed."""
    lib = tt.lib()
    t = tt.Tree([np.arange(100), np.arange(50)])
    t32 = tt.Tree([np.arange(100), np.arange(50)], block_q=32, block_k=32)

    def both(a):
        rf = lib.tree_attn_fwd(ctypes.byref(a), None)
        b = tt.AttnBwdArgs(a=a, d_o=FAKE, d_q=FAKE, d_k=FAKE, d_v=FAKE, flags=0)
        rb = lib.tree_attn_bwd(ctypes.byref(b), None)
        assert rf == rb, (rf, rb)
        return rf, tt.last_error()

    for hq, hkv in ((4, 4), (4, 2), (6, 2), (8, 2), (32, 4), (32, 2)):
        rc, msg = both(_attn(t, h_q=hq, h_kv=hkv))
        assert rc == tt.TT_EINVAL and "tree_plan_upload" in msg, (hq, hkv, msg)
    for kw in (dict(d=64), dict(d=256), dict(tree=t32.handle)):
        rc, msg = both(_attn(t, **kw))
        assert rc == tt.TT_EUNSUPPORTED and "TT_ALLOW_GENERIC" in msg, kw
        rc, msg = both(_attn(t, flags=tt.TT_ALLOW_GENERIC, **kw))
        assert rc == tt.TT_EINVAL and "tree_plan_upload" in msg, kw
    rc, msg = both(_attn(t, d=64, dtype=tt.TT_F32))
    assert rc == tt.TT_EINVAL and "tree_plan_upload" in msg
    rc, _ = both(_attn(t, flags=2))
    assert rc == tt.TT_EINVAL and "flags" in tt.last_error()


def test_binding_rejects_bad_tensors_before_the_library():
    """The Python binding checks dtype, shape, contiguity and device of every
    tensor and raises ValueError before anything reaches the library (here
    the tensors live on the CPU, so a check that slipped would fail later on
    the device check, not pass)."""
    import torch
    t = tt.Tree([np.arange(70), np.arange(40)])
    N = t.N
    plan = torch.zeros(t.plan_bytes(), dtype=torch.uint8)
    q = torch.zeros(N, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(N, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros_like(k)

    def raises(fn, text):
        with pytest.raises(ValueError, match=text):
            fn()

    raises(lambda: tt.tree_attn_fwd(t, plan, q.float(), k, v), "k has dtype")
    raises(lambda: tt.tree_attn_fwd(t, plan, q, k, v[:, :1].contiguous()), "v has shape")
    raises(lambda: tt.tree_attn_fwd(t, plan, q, k[:, :, :64].contiguous(), v), "k must be")
    raises(lambda: tt.tree_attn_fwd(t, plan, q.transpose(0, 1).contiguous().transpose(0, 1), k, v), "contiguous")
    raises(lambda: tt.tree_attn_fwd(t, plan, q.half(), k.half(), v.half()), "q has dtype")
    raises(lambda: tt.tree_attn_fwd(t, plan[:10], q, k, v), "device|plan holds")
    raises(lambda: tt.tree_attn_fwd(t, plan, q, k, v), "CUDA")
    lse = torch.zeros(N, 4)
    o = torch.zeros_like(q)
    raises(lambda: tt.tree_attn_bwd(t, plan, q, k, v, o, lse.double(), q), "lse has dtype")
    raises(lambda: tt.tree_attn_bwd(t, plan, q, k, v, o, lse, q, d_k=torch.zeros_like(k), accumulate=True),
           "d_k has dtype")
    raises(lambda: tt.tree_attn_bwd(t, plan, q, k, v, o, lse, q, d_k=torch.zeros(N, 2, 128)), "d_k has dtype")
    raises(lambda: tt.tree_attn_bwd(t, plan, q, k, v, o, lse, q[:-1]), "d_o has shape")
    # weighted NLL: the target CSR must be int32 / float32, logits 2-D
    z = torch.zeros(N, 50)
    rp = torch.zeros(N + 1, dtype=torch.int32)
    tid = torch.zeros(N - 2, dtype=torch.int32)
    tw = torch.zeros(N - 2)
    raises(lambda: tt.tree_weighted_nll(rp.long(), tid, tw, logits=z), "tgt_row_ptr has dtype")
    raises(lambda: tt.tree_weighted_nll(rp, tid.long(), tw, logits=z), "tgt_id has dtype")
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw.double(), logits=z), "tgt_w has dtype")
    raises(lambda: tt.tree_weighted_nll(rp[:-1], tid, tw, logits=z), "tgt_row_ptr has shape")
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw, logits=z.t()), "contiguous|shape")
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw, logits=z, hidden=z), "exactly one")
    h = torch.zeros(N, 16, dtype=torch.bfloat16)
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw, hidden=h, w_vocab=torch.zeros(8, 64, dtype=torch.bfloat16)),
           "w_vocab must be")
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw, hidden=h.float(), w_vocab=torch.zeros(16, 64)),
           "hidden has dtype")
    raises(lambda: tt.tree_weighted_nll(rp, tid, tw, logits=z), "CUDA")
    # path mode: one row per tree row
    p = tt.Path(t, 64, 0)
    raises(lambda: tt.tree_attn_path(p, q[:-1], k, v), "one row per tree row")
    raises(lambda: tt.tree_attn_path(p, q, k.float(), v), "k has dtype")
    raises(lambda: tt.tree_attn_path(p, q, k, v, d_o=q, d_k=torch.zeros(N, 2, 128)), "d_k has dtype")
