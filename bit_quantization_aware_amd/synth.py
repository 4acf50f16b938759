"""Seeded synthetic inputs for the quantized-linear hot path.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic, so the GPU path and the CPU oracle can both take their
inputs from it.  Generator: numpy PCG64.

Recipe (weights are fp32 shadow weights stored [out, in], row = output channel):
  * tiny      -- one 256x256 matrix, sigma 0.02, ``default_rng(0)`` drawing W,
                 then the upstream gradient G ~ N(0,1), then 8x256 activations
                 X ~ N(0,1) rounded to bf16, in that order.
  * mobilellm_125m -- 30 layers x {q,k,v,o [576,576]; gate,up [1536,576];
                 down [576,1536]}, sigma 0.02 (SwiGLU feed-forward as in the
                 Llama family).
  * mobilellm_1p5b -- 54 layers x {q,o [1600,1600]; k,v [400,1600];
                 gate,up [4352,1600]; down [1600,4352]}, sigma 0.02, with a
                 Bernoulli(0.001) outlier mask that multiplies weights by 10.
  * llama3_8b -- [4096,4096], [1024,4096], [14336,4096], [4096,14336],
                 sigma 0.015.
  * square16k -- one [16384,16384] matrix, sigma 0.02.
Every matrix of the stacked configs draws from its own stream
``SeedSequence([cfg, layer, matrix, tensor])`` with tensor 0 = W, 1 = G,
2 = X, 3 = outlier mask, so any single matrix can be regenerated alone.
"""
from __future__ import annotations

import numpy as np

CFG_IDS = {"tiny": 0, "mobilellm_125m": 1, "mobilellm_1p5b": 2, "llama3_8b": 3, "square16k": 4}
T_W, T_G, T_X, T_OUTLIER = 0, 1, 2, 3


def mobilellm_125m_shapes():
    """[(layer, name, rows, cols)] of the 210 projection matrices."""
    h, f = 576, 1536
    per = [("q", h, h), ("k", h, h), ("v", h, h), ("o", h, h), ("gate", f, h), ("up", f, h),
           ("down", h, f)]
    return [(l, n, r, c) for l in range(30) for (n, r, c) in per]


def mobilellm_1p5b_shapes():
    """[(layer, name, rows, cols)] of the 378 projection matrices (GQA kv width 400)."""
    h, f, kv = 1600, 4352, 400
    per = [("q", h, h), ("k", kv, h), ("v", kv, h), ("o", h, h), ("gate", f, h), ("up", f, h),
           ("down", h, f)]
    return [(l, n, r, c) for l in range(54) for (n, r, c) in per]


def llama3_8b_shapes():
    return [(0, "4096x4096", 4096, 4096), (0, "1024x4096", 1024, 4096),
            (0, "14336x4096", 14336, 4096), (0, "4096x14336", 4096, 14336)]


def square16k_shapes():
    return [(0, "16384x16384", 16384, 16384)]


SHAPES = {"mobilellm_125m": mobilellm_125m_shapes, "mobilellm_1p5b": mobilellm_1p5b_shapes,
          "llama3_8b": llama3_8b_shapes, "square16k": square16k_shapes}
SIGMA = {"tiny": 0.02, "mobilellm_125m": 0.02, "mobilellm_1p5b": 0.02, "llama3_8b": 0.015,
         "square16k": 0.02}


def rng_for(cfg: str, layer: int, matrix: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [CFG_IDS[cfg], int(layer), int(matrix), int(tensor)])))


def normal_f32(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 activations to bf16 (nearest-even) and return the bits as
    uint16.  Input preparation only; uses torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tiny():
    """The 256x256 case: (W, G, X_bf16_bits) from default_rng(0) in that order."""
    rng = np.random.default_rng(0)
    W = normal_f32(rng, (256, 256), 0.02)
    G = normal_f32(rng, (256, 256))
    X = to_bf16_bits(normal_f32(rng, (8, 256)))
    return W, G, X


def matrix_index(cfg: str, k: int):
    """(layer, index-within-layer) of the k-th matrix of a stacked config."""
    shapes = SHAPES[cfg]()
    layer = shapes[k][0]
    first = next(i for i, s in enumerate(shapes) if s[0] == layer)
    return layer, k - first


def weight(cfg: str, k: int) -> np.ndarray:
    """fp32 W of the k-th matrix of a config."""
    layer, name, rows, cols = SHAPES[cfg]()[k]
    _, mi = matrix_index(cfg, k)
    W = normal_f32(rng_for(cfg, layer, mi, T_W), (rows, cols), SIGMA[cfg])
    if cfg == "mobilellm_1p5b":
        mask = rng_for(cfg, layer, mi, T_OUTLIER).random((rows, cols), dtype=np.float32) < 0.001
        W[mask] *= np.float32(10.0)
    return W


def upstream_grad(cfg: str, k: int) -> np.ndarray:
    """fp32 G ~ N(0,1) of the k-th matrix of a config."""
    layer, name, rows, cols = SHAPES[cfg]()[k]
    _, mi = matrix_index(cfg, k)
    return normal_f32(rng_for(cfg, layer, mi, T_G), (rows, cols))


def activations(cfg: str, k: int, M: int, K: int) -> np.ndarray:
    """bf16 bits of X [M, K] ~ N(0,1) for the k-th matrix of a config."""
    layer = SHAPES[cfg]()[k][0] if cfg in SHAPES else 0
    mi = matrix_index(cfg, k)[1] if cfg in SHAPES else 0
    rng = rng_for(cfg, layer, mi, T_X)
    return to_bf16_bits(normal_f32(rng, (M, K)))


def random_case(seed: int, rows: int, cols: int, sigma: float = 0.02):
    """A generic seeded (W, G) pair for parity tests at arbitrary shapes."""
    rng = np.random.default_rng(seed)
    return normal_f32(rng, (rows, cols), sigma), normal_f32(rng, (rows, cols))
