"""Pins for the oracle's MUL_MAT (not GPU).

The oracle computes y[n][m] = sum_k W'[m][k] x[n][k] in binary64 over the
exactly dequantized weights ("No Python! Building an AI Inference Engine
Exclusively in C++", §6: C_ij = sum_k A_ik B_kj; §4: ne[0] is the contiguous
dimension, so W is ne = [K, M], x is ne = [K, N], y is ne = [M, N]).

Pinned by: a hand-worked 2 x 32 x 2 product, one-hot activations (which
return a column of W' exactly), all-ones activations against the factored
block form sum_b Delta_b * sum_i code_i ("A Complete Guide to llama.cpp ...",
§2.2: the scale factors out of each block's dot product), and brute force
against numpy's binary64 matmul on non-square shapes (a transposed operand or
a dropped term fails it).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from golden_io import read_blocks


def _w(seed, M, K):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)


def _x(seed, N, K):
    return np.random.default_rng(seed).standard_normal((N, K), dtype=np.float32)


def _packed(orc, type_, w):
    if type_ == orc.F16:
        return w.astype(np.float16).view(np.uint8).reshape(w.shape[0], -1)
    return orc.quantize(type_, w)


def test_hand_worked_tiny_product(orc):
    """W' rows = the 'nibble_order' and 'ties_and_clamp' blocks; x rows = all
    ones and e_3.  By hand:
      row 0: W' = (c_i - 8)/8, c = 0..15, 15..0 -> sum = (-8 - 8)/8 = -2,
             sum |.| = (64 + 64)/8 = 16, element 3 = -5/8;
      row 1: W' = 7/16, -1/2, 1/16, -1/16, 1/8, 7/16, 0... -> sum = 8/16 = 1/2,
             sum |.| = 26/16 = 13/8, element 3 = -1/16."""
    blocks = {c["name"]: c for c in read_blocks("q4_0_blocks.txt")}
    w = np.stack([blocks["nibble_order"]["w"], blocks["ties_and_clamp"]["w"]])
    x = np.zeros((2, 32), np.float32)
    x[0] = 1.0
    x[1, 3] = 1.0
    y, a = orc.mul_mat(orc.Q4_0, orc.quantize(orc.Q4_0, w), 32, x)
    assert y.tolist() == [[-2.0, 0.5], [-0.625, -0.0625]]
    assert a.tolist() == [[16.0, 1.625], [0.625, 0.0625]]


@pytest.mark.parametrize("type_name", ["Q8_0", "Q4_0", "F16"])
def test_one_hot_returns_column(orc, type_name):
    t = getattr(orc, type_name)
    M, K = 37, 256
    w = _w(1, M, K)
    p = _packed(orc, t, w)
    deq = orc.dequantize(t, p, K)
    js = [0, 1, 31, 32, 100, 255]
    x = np.zeros((len(js), K), np.float32)
    for n, j in enumerate(js):
        x[n, j] = 1.0
    y, a = orc.mul_mat(t, p, K, x)
    for n, j in enumerate(js):
        assert np.array_equal(y[n], deq[:, j].astype(np.float64))
        assert np.array_equal(a[n], np.abs(deq[:, j]).astype(np.float64))


@pytest.mark.parametrize("type_name", ["Q8_0", "Q4_0"])
def test_all_ones_factored_block_form(orc, type_name):
    """x = 1: y_m = sum_b Delta_b * sum_i code_i, with the block scales and codes
    taken from the block quantizer applied to each 32-block on its own."""
    t = getattr(orc, type_name)
    M, K = 9, 160
    w = _w(2, M, K)
    y, _ = orc.mul_mat(t, orc.quantize(t, w), K, np.ones((1, K), np.float32))
    for m in range(M):
        total = Fraction(0)
        for b in range(K // 32):
            sb, codes = orc.quantize_block(t, w[m, 32 * b: 32 * b + 32])
            d = Fraction(float(orc.f16_bits_to_f32(np.array([sb], np.uint16))[0]))
            ints = codes.astype(np.int64) - (8 if t == orc.Q4_0 else 0)
            total += d * int(ints.sum())
        assert abs(Fraction(y[0, m]) - total) <= abs(total) * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("type_name", ["Q8_0", "Q4_0", "F16"])
@pytest.mark.parametrize("shape", [(7, 96, 3), (64, 512, 1), (33, 2048, 8), (5, 32, 5)])
def test_brute_force_vs_numpy(orc, type_name, shape):
    t = getattr(orc, type_name)
    M, K, N = shape
    w, x = _w(3, M, K), _x(4, N, K)
    p = _packed(orc, t, w)
    deq = orc.dequantize(t, p, K).astype(np.float64)
    y, a = orc.mul_mat(t, p, K, x)
    yr = x.astype(np.float64) @ deq.T
    ar = np.abs(x.astype(np.float64)) @ np.abs(deq).T
    assert y.shape == (N, M)
    assert np.all(np.abs(y - yr) <= 1e-12 * ar + 1e-300)
    assert np.all(np.abs(a - ar) <= 1e-12 * ar)


def test_bf16_activations_and_bf16_weight_variant(orc):
    """x given as bfloat16 bits; the diagnostic variant rounds W' to bfloat16
    first.  Both reduce to numpy binary64 matmul of the converted operands
    (torch's CPU bfloat16 cast provides the independent conversions)."""
    M, K, N = 40, 256, 6
    w = _w(5, M, K)
    xf = _x(6, N, K)
    xb = torch.from_numpy(xf).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    xv = xb.to(torch.float32).numpy().astype(np.float64)
    p = orc.quantize(orc.Q4_0, w)
    deq = orc.dequantize(orc.Q4_0, p, K)
    y, a = orc.mul_mat(orc.Q4_0, p, K, xbits, x_bf16_bits=True)
    yr = xv @ deq.astype(np.float64).T
    ar = np.abs(xv) @ np.abs(deq.astype(np.float64)).T
    assert np.all(np.abs(y - yr) <= 1e-12 * ar)
    yb, _ = orc.mul_mat(orc.Q4_0, p, K, xbits, x_bf16_bits=True, w_to_bf16=True)
    wb = torch.from_numpy(deq).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    assert np.all(np.abs(yb - xv @ wb.T) <= 1e-12 * ar)
    assert not np.array_equal(yb, y)


def test_row_ranges_and_pairs_agree(orc):
    M, K, N = 50, 128, 4
    w, x = _w(7, M, K), _x(8, N, K)
    p = orc.quantize(orc.Q8_0, w)
    y, a = orc.mul_mat(orc.Q8_0, p, K, x)
    y2, _ = orc.mul_mat(orc.Q8_0, p, K, x, rows=(10, 23))
    assert np.array_equal(y2[:, 10:23], y[:, 10:23]) and not y2[:, :10].any()
    ms = np.array([0, 49, 17, 17, 3])
    ns = np.array([0, 3, 1, 2, 3])
    yp, ap = orc.mul_mat_pairs(orc.Q8_0, p, K, x, ms, ns)
    assert np.array_equal(yp, y[ns, ms]) and np.array_equal(ap, a[ns, ms])


def test_empty_contraction(orc):
    y, a = orc.mul_mat(orc.F32, np.zeros((3, 0), np.uint8), 0, np.zeros((2, 0), np.float32))
    assert y.shape == (2, 3) and not y.any() and not a.any()
