"""GPU parity of the fused lm-head + weighted tree NLL (bf16) against the fp64 oracle.

z = H W is formed in bf16 on the GPU (the oracle forms it exactly), so the
tolerance is the bf16 one, 2e-2, on loss, logp, dH and dW.
"""
import numpy as np
import pytest
import torch

import prefix_tree_attention_dfs_amd as tt
import treesynth as ts
from oracle.nll import lmhead, lmhead_rows, lmhead_lse, lmhead_target_logp, lmhead_dw_columns
from oracle.tree import dfs_arrays
from tests.gpu_util import rel_err, row_rel_err, bf16_input

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _tree_targets(seqs):
    tree = tt.Tree(seqs)
    a = tree.export()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    return tree, a, dev(a["tgt_row_ptr"]), dev(a["tgt_token"]), dev(a["tgt_w"])


@pytest.mark.parametrize("sizes", [(200, 1000, 7), (512, 4096, 11), (72, 264, 3)])
@pytest.mark.parametrize("dw", [torch.float32, torch.bfloat16])
def test_fused_lmhead_ragged(sizes, dw):
    d_model, vocab, seed = sizes
    case = ts.random_small_tree(seed, n_seqs=9, max_len=70, vocab=vocab)
    tree, a, rp, tid, tw = _tree_targets(case.seqs)
    o = dfs_arrays(case.seqs)
    rng = ts.rng_for(seed + 1)
    H, Hn = bf16_input(rng, (tree.N, d_model), 1.0)
    W, Wn = bf16_input(rng, (d_model, vocab), 0.02)
    print(f"N={tree.N} d_model={d_model} vocab={vocab} dw={dw}", flush=True)
    out = tt.tree_weighted_nll(rp, tid, tw, hidden=H, w_vocab=W, dw_dtype=dw)
    loss, logp, dz, dH, dW = lmhead(Hn, Wn, o["parent"], o["token"], o["weight"].astype(np.float64))
    assert abs(out["loss"].item() - loss) / abs(loss) < TOL
    assert rel_err(out["logp"], logp[a["tgt_dfs"]]) < TOL
    assert rel_err(out["d_hidden"], dH) < TOL
    assert rel_err(out["d_w_vocab"], dW) < TOL


def test_fused_lmhead_full_shape():
    """16384 tree tokens x 4096 -> 151936 vocabulary, 32-leaf tree, as timed:
    the total loss and every target's logp against the oracle's per-row LSE
    over all 16,384 rows (z formed in fp64 one block of rows at a time); dW
    on 16 vocabulary columns (every row of dZ contributes, so this covers the
    whole dW GEMM's reduction and its XCD-region tile walk); dH on sampled
    rows.  The weighted loss equals the branch average (Tree Training,
    Abstract), which the oracle's pins tie to this form."""
    import time
    case = ts.lmhead_tree(0)
    tree, a, rp, tid, tw = _tree_targets(case.seqs)
    o = dfs_arrays(case.seqs)
    N, dm, V = tree.N, 4096, 151936
    rng = ts.rng_for(4000)
    hb = ts.normal_bf16(rng, (N, dm), 1.0)
    wb = ts.normal_bf16(rng, (dm, V), 0.02)
    dev = lambda b: torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    out = tt.tree_weighted_nll(rp, tid, tw, hidden=dev(hb), w_vocab=dev(wb))
    torch.cuda.synchronize()
    Hn = ts.bf16_bits_to_f64(hb)
    Wn = ts.bf16_bits_to_f64(wb)
    w = o["weight"].astype(np.float64)
    t0 = time.perf_counter()
    lse = lmhead_lse(Hn, Wn, row_block=512)
    print(f"oracle LSE of {N} rows: {time.perf_counter() - t0:.1f} s", flush=True)
    loss, logp = lmhead_target_logp(Hn, Wn, lse, o["parent"], o["token"], w)
    got_loss = out["loss"].item()
    print(f"loss gpu {got_loss:.6f} oracle {loss:.6f}", flush=True)
    assert abs(got_loss - loss) / abs(loss) < TOL
    lp = logp[a["tgt_dfs"]]
    e = rel_err(out["logp"], lp)
    print(f"logp: rel {e:.2e}, max abs {np.max(np.abs(out['logp'].cpu().numpy() - lp)):.2e}", flush=True)
    assert e < TOL
    cols = np.unique(np.concatenate([[0, 1, V - 1, V // 2], a["tgt_token"][:6], ts.rng_for(4001).integers(0, V, 6)]))
    dwr = lmhead_dw_columns(Hn, Wn, lse, o["parent"], o["token"], w, cols)
    dwg = out["d_w_vocab"][:, torch.as_tensor(cols, device="cuda")]
    e = rel_err(dwg, dwr)
    print(f"dW on {len(cols)} columns: tensor {e:.2e}, per column "
          f"{row_rel_err(dwg.t().contiguous(), dwr.T.copy()):.2e}", flush=True)
    assert e < TOL
    rows = [r for r in np.linspace(0, N - 1, 10).astype(int) if a["tgt_row_ptr"][r + 1] > a["tgt_row_ptr"][r]]
    tg = [[(int(a["tgt_token"][t]), float(a["tgt_w"][t])) for t in range(a["tgt_row_ptr"][r], a["tgt_row_ptr"][r + 1])]
          for r in rows]
    ref = lmhead_rows(Hn[rows], Wn, tg)
    dh = out["d_hidden"].float().cpu().numpy()
    for r, (lse_r, lps, dzr, dhr) in zip(rows, ref):
        assert abs(lse_r - lse[r]) < 1e-9 * abs(lse_r)
        assert rel_err(torch.from_numpy(dh[r]), dhr) < TOL
