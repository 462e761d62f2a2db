"""Helpers shared by the GPU parity tests (inputs from treesynth, comparisons)."""
import numpy as np
import torch

import treesynth as ts


def rel_err(gpu, ref):
    """max |gpu - ref| / max |ref| over the whole tensor (ref in fp64)."""
    g = gpu.detach().float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(r)) if r.size else 0.0
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def row_rel_err(gpu, ref, floor=1e-3):
    """Per-row error: max over rows (every index but the last) of
    max |gpu - ref| / max |ref| within that row, so that small rows (the
    gradient of a leaf key beside a root key) are judged on their own scale.
    A row whose own maximum is below `floor` times the tensor's maximum is
    normalised by that floor instead (an all-but-zero row has no scale)."""
    g = gpu.detach().float().cpu().double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if r.size == 0:
        return 0.0
    g = g.reshape(-1, r.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    top = np.max(np.abs(r))
    den = np.maximum(np.max(np.abs(r), axis=1), floor * (top if top > 0 else 1.0))
    return float(np.max(np.max(np.abs(g - r), axis=1) / den))


def f32_input(rng, shape, std=1.0):
    """(device float32 tensor, exact fp64 numpy copy)."""
    x = ts.normal_f32(rng, shape, std)
    return torch.from_numpy(x).cuda(), x.astype(np.float64)


def bf16_input(rng, shape, std=1.0):
    """(device bf16 tensor, exact fp64 numpy copy of its values)."""
    bits = ts.normal_bf16(rng, shape, std)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return t, ts.bf16_bits_to_f64(bits)


def inputs(dtype, seed, n_q, n_k, hq, hkv, d, std):
    """q [n_q,hq,d], k/v [n_k,hkv,d], dO [n_q,hq,d] ~ N(0,1); drawn q, k, v, dO in that order."""
    rng = ts.rng_for(seed)
    mk = f32_input if dtype == torch.float32 else bf16_input
    q = mk(rng, (n_q, hq, d), std)
    k = mk(rng, (n_k, hkv, d), std)
    v = mk(rng, (n_k, hkv, d), std)
    do = mk(rng, (n_q, hq, d), 1.0)
    return q, k, v, do
