"""Dense random inputs: fp32 normals and their bf16 (round-to-nearest-even) images."""
import numpy as np


def rng_for(seed: int) -> np.random.Generator:
    """numpy PCG64 generator for an explicit integer seed."""
    return np.random.Generator(np.random.PCG64(int(seed)))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; returns the uint16 bit patterns.

    Inputs here are finite normals, so no NaN/Inf handling is needed (asserted).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        b = flat_in[s:s + step].view(np.uint32)
        assert np.all((b & 0x7F800000) != 0x7F800000), "non-finite input"
        bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
        flat_out[s:s + step] = ((b + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in float32 (std applied in float32)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) drawn in float32, then rounded once to bf16; returns uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        m = min(step, n - s)
        out[s:s + m] = bf16_round(normal_f32(rng, (m,), std))
    return out.reshape(shape)
