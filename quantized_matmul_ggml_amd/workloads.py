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
