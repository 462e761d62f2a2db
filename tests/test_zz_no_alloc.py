"""The no-allocation entry point, tree_weighted_nll_noalloc, called through
the C ABI: its loss, logp and dZ equal tree_weighted_nll's (the same kernels
on the same inputs, per-row losses in the static scratch instead of the
workspace) bit for bit, on two calls in a row, the second on a smaller tree
(the scratch keeps the first call's rows past the second's end; they must not
leak into the sum)."""
import ctypes

import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p()


def _case(seed, n_seqs, max_len, vocab, dtype):
    case = ts.random_small_tree(seed, n_seqs=n_seqs, max_len=max_len, vocab=vocab)
    tree = tt.Tree(case.seqs)
    a = tree.export()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    rp, tid, tw = dev(a["tgt_row_ptr"]), dev(a["tgt_token"]), dev(a["tgt_w"])
    g = torch.Generator(device="cuda").manual_seed(seed)
    z = (torch.randn(tree.N, vocab, device="cuda", generator=g) * 2.0).to(dtype)
    return rp, tid, tw, z


def _noalloc(rp, tid, tw, z):
    n, V = z.shape
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    logp = torch.empty(tid.numel(), dtype=torch.float32, device="cuda")
    dz = torch.empty_like(z)
    a = tt.NllArgs(n_rows=n, d_model=0, vocab=V, n_tgt=tid.numel(), logits=_p(z),
                   logits_dtype=tt.TT_F32 if z.dtype == torch.float32 else tt.TT_BF16,
                   tgt_row_ptr=_p(rp), tgt_id=_p(tid), tgt_w=_p(tw), loss=_p(loss), logp=_p(logp),
                   d_logits=_p(dz), workspace=None, workspace_bytes=0)
    rc = tt.lib().tree_weighted_nll_noalloc(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == tt.TT_OK, tt.last_error()
    return loss, logp, dz


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_nll_equals_workspace_nll(dtype):
    for seed, n_seqs, max_len, vocab in ((31, 40, 120, 3000), (32, 6, 40, 3000)):
        rp, tid, tw, z = _case(seed, n_seqs, max_len, vocab, dtype)
        print(f"rows={z.shape[0]} vocab={vocab} dtype={dtype}", flush=True)
        loss, logp, dz = _noalloc(rp, tid, tw, z)
        ref = tt.tree_weighted_nll(rp, tid, tw, logits=z)
        torch.cuda.synchronize()
        assert torch.equal(loss, ref["loss"]), (loss.item(), ref["loss"].item())
        assert torch.equal(logp, ref["logp"])
        assert torch.equal(dz, ref["d_logits"])
        assert np.isfinite(loss.item()) and loss.item() > 0
