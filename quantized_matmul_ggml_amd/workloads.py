"""Seeded synthetic inputs for the tests and the benchmark.

This module holds no part of the method's arithmetic: it only draws seeded
Gaussian tensors at the shapes of the workloads, and applies the input
roundings the workloads prescribe (fp16 weights for the dense baseline, bf16
activations for the prefill GEMM) with numpy / torch casts.  The same arrays
feed the oracle and the GPU.

Shapes are those of a TinyLLaMA-class decoder layer (hidden 2048, FFN 5632,
KV dimension 256 under grouped-query attention, vocabulary 32000; the
Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §1 and
§4.3), whose 1.1 B parameters make 22 layers of 44,040,192 weights plus the
32000 x 2048 embedding and LM head.  Weights ~ N(0, 0.02), activations
~ N(0, 1).  Seed convention: 10000 * workload + 100 * tensor + replica.
"""
from __future__ import annotations

import numpy as np
import torch

HIDDEN, FFN, KV, VOCAB, LAYERS = 2048, 5632, 256, 32000, 22

# One decoder layer's projections: name, rows M, contraction K, activation slot.
# Slot 0 feeds the Q/K/V projections, 1 the attention output projection, 2 the
# gate and up projections, 3 the down projection.
LAYER = (
    ("wq", HIDDEN, HIDDEN, 0),
    ("wk", KV, HIDDEN, 0),
    ("wv", KV, HIDDEN, 0),
    ("wo", HIDDEN, HIDDEN, 1),
    ("wgate", FFN, HIDDEN, 2),
    ("wup", FFN, HIDDEN, 2),
    ("wdown", HIDDEN, FFN, 3),
)
LAYER_X_K = (HIDDEN, HIDDEN, HIDDEN, FFN)   # K of activation slots 0..3

# The workloads (by what they are).
Q8_GEMV_SMALL = dict(name="q8_0_gemv_512x512_n1", type="Q8_0", M=512, K=512, N=1, id=1)
F16_GEMV_FFN_UP = dict(name="f16_gemv_5632x2048_n1", type="F16", M=FFN, K=HIDDEN, N=1, id=2)
Q4_DECODE_LAYER = dict(name="q4_0_decode_layer_tinyllama", type="Q4_0", id=3)
Q8_LM_HEAD = dict(name="q8_0_lm_head_32000x2048", type="Q8_0", M=VOCAB, K=HIDDEN, Ns=(1, 2, 4, 8), id=4)
Q4_PREFILL_FFN_UP = dict(name="q4_0_prefill_gemm_5632x2048x512", type="Q4_0", M=FFN, K=HIDDEN, N=512, id=5)


def seed(workload: int, tensor: int, replica: int = 0) -> int:
    return 10000 * workload + 100 * tensor + replica


def weights(seed_: int, M: int, K: int) -> np.ndarray:
    """W ~ N(0, 0.02) as float32 (M, K)."""
    g = np.random.default_rng(seed_).standard_normal((M, K), dtype=np.float32)
    return (g * np.float32(0.02)).astype(np.float32)


def activations(seed_: int, N: int, K: int) -> np.ndarray:
    """x ~ N(0, 1) as float32 (N, K), one row per token."""
    return np.random.default_rng(seed_).standard_normal((N, K), dtype=np.float32)


def round_f16(a: np.ndarray) -> np.ndarray:
    """Input rounding of the dense fp16 weights (numpy cast, nearest even)."""
    return a.astype(np.float16)


def round_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Input rounding of the bf16 activations (torch CPU cast, nearest even);
    returns the bfloat16 bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_torch(bits: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns -> torch bfloat16 tensor on `device` (no rounding)."""
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)


def weights_device(seed_: int, M: int, K: int, device) -> torch.Tensor:
    """W ~ N(0, 0.02) drawn on the GPU with a seeded torch generator (large
    benchmark tensors; same distribution as ``weights``)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_)
    return torch.randn((M, K), generator=g, device=device, dtype=torch.float32) * 0.02


def activations_device(seed_: int, N: int, K: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed_)
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32)


# ---------------------------------------------------------------- edge cases
#
# Inputs that reach the corners of the method rather than its typical case:
# weight blocks at many magnitudes (zero blocks, blocks whose fp16 scale is
# subnormal, blocks of exact quarter-steps that make rounding ties, blocks
# scaled by 1000) and blocks holding one large weight among zeros, paired
# with activations whose mean is far from zero and which are tiny exactly
# where those lone weights sit.  Only random draws and masks: no method
# arithmetic.

def adversarial_weights(seed_: int, M: int, K: int, block: int = 32) -> np.ndarray:
    """Gaussian rows at many magnitudes plus blocks of `block` weights that
    hit ties, clamps, zero blocks and subnormal fp16 scales."""
    rng = np.random.default_rng(seed_)
    w = rng.standard_normal((M, K), dtype=np.float32) * np.float32(0.02)
    blocks = w.reshape(-1, block)
    nb = blocks.shape[0]
    sel = rng.random(nb)
    blocks[sel < 0.05] = 0.0
    tiny = (sel >= 0.05) & (sel < 0.10)
    blocks[tiny] *= np.float32(2.0 ** -18)
    ties = (sel >= 0.10) & (sel < 0.20)
    blocks[ties] = (rng.integers(-16, 17, (int(ties.sum()), block)) / np.float32(16)).astype(np.float32)
    big = (sel >= 0.20) & (sel < 0.25)
    blocks[big] *= np.float32(1000.0)
    return blocks.reshape(M, K)


def outlier_column(K: int, seed_: int) -> np.ndarray:
    """For each 32-block of a row of K, the position (0..31) of its lone
    weight in outlier blocks; shared by every row, so that activations can be
    made tiny exactly there."""
    return np.random.default_rng(seed_).integers(0, 32, K // 32)


def outlier_weights(seed_: int, M: int, K: int, frac: float = 0.5) -> np.ndarray:
    """adversarial_weights, with 32-blocks replaced by one weight of
    magnitude 0.02, 0.2 or 2 (random sign) at the block's outlier_column
    position and zeros elsewhere: every block of every third row, and a
    fraction `frac` of the blocks of the other rows."""
    w = adversarial_weights(seed_, M, K)
    rng = np.random.default_rng(seed_ + 1)
    pos = outlier_column(K, seed_ + 2)
    nbk = K // 32
    sel = rng.random((M, nbk)) < frac
    sel[::3] = True
    mag = (rng.choice(np.array([0.02, 0.2, 2.0], np.float32), (M, nbk)) *
           rng.choice(np.array([-1.0, 1.0], np.float32), (M, nbk))).astype(np.float32)
    blocks = w.reshape(M, nbk, 32)
    blocks[sel] = 0.0
    rows, cols = np.nonzero(sel)
    blocks[rows, cols, pos[cols]] = mag[rows, cols]
    return blocks.reshape(M, K)


def shifted_activations(seed_: int, N: int, K: int, outlier_seed: int | None = None,
                        mean: float = 5.0) -> np.ndarray:
    """x ~ N(mean, 1) (N, K); where outlier_seed is given, x = 0.01 (random
    sign) at the outlier_column positions of that seed, and a tenth of the
    other activations of token 1 (if any) are exact zeros."""
    rng = np.random.default_rng(seed_)
    x = (rng.standard_normal((N, K), dtype=np.float32) + np.float32(mean)).astype(np.float32)
    if outlier_seed is not None:
        pos = outlier_column(K, outlier_seed + 2)
        ks = 32 * np.arange(K // 32) + pos
        x[:, ks] = (np.float32(0.01) * rng.choice(np.array([-1.0, 1.0], np.float32), (N, ks.size))).astype(np.float32)
    if N > 1:
        x[1, rng.random(K) < 0.1] = 0.0
    return x
