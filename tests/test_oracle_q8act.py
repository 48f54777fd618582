"""Pins for the oracle's integer-activation MUL_MAT (not GPU).

"A Complete Guide to llama.cpp and Customization with C++", §2.2: with the
activations quantized per block too, x_i ~= Delta_x * qx_i, the block dot
product is y ~= Delta * Delta_x * sum_i q_i qx_i, and the sum is integer
arithmetic.  The oracle quantizes x with the Q8_0 rule (the same steps as
the weights: Delta_x = fp16(amax/127), qx = roundf(x / Delta_x)).

Pinned by: a hand-worked block; the identity with the exact MUL_MAT over
the dequantized activations (every block term Delta_w q Delta_x qx is exact,
so the two differ only by binary64 summation order); the quantization
bound |y_int - y(x)| <= sum_k |W'_k| Delta_x(k) / 2 against the float
activations; the factored form with all-ones codes; and, for 64-block
weights, the same identity plus the reduction to 32-block weights.
"""
import numpy as np

from quantized_matmul_ggml_amd import workloads as WL


def _f16_bits(v):
    return int(np.array([v], np.float16).view(np.uint16)[0])


def test_hand_worked_block(orc):
    # Q4_0 weights: Delta = 1/2 (0x3800), nibble of element i = i % 16, so
    # q_i = i % 16 - 8; byte j = j | j << 4.  Q8_0 activations: Delta_x = 1
    # (0x3C00), qx_i = 1, 0, -1 repeating (i % 3 = 0, 1, 2).
    # sum_i q_i qx_i over i = 0..31: the terms with i % 3 == 0 (qx = +1) are
    # q = -8, -5, -2, 1, 4, 7 (i = 0..15) and -6, -3, 0, 3, 6 (i = 18..30),
    # sum -3; those with i % 3 == 2 (qx = -1) are q = -6, -3, 0, 3, 6
    # (i = 2..14) and -7, -4, -1, 2, 5 (i = 17..29), sum -5, entering as +5.
    # S = -3 + 5 = 2, y = 1/2 * 1 * 2 = 1.
    w = np.zeros((1, 32), np.uint8)
    w[0, 0:2] = [0x00, 0x38]
    w[0, 16:32] = [j | j << 4 for j in range(16)]
    xq = np.zeros((1, 48), np.uint8)
    xq[0, 0:2] = [0x00, 0x3C]
    xq[0, 16:48] = np.array([(1, 0, -1)[i % 3] for i in range(32)], np.int8).view(np.uint8)
    y, a = orc.mul_mat_q8act(orc.Q4_0, w, 32, xq)
    assert y[0, 0] == 1.0 and a[0, 0] == 1.0
    # the same weights as Q8_0 codes q_i (scale 1/2): identical sum
    w8 = np.zeros((1, 48), np.uint8)
    w8[0, 0:2] = [0x00, 0x38]
    w8[0, 16:48] = np.array([i % 16 - 8 for i in range(32)], np.int8).view(np.uint8)
    y8, _ = orc.mul_mat_q8act(orc.Q8_0, w8, 32, xq)
    assert y8[0, 0] == 1.0


def test_equals_exact_mul_mat_on_dequantized_activations(orc):
    rng = np.random.default_rng(3)
    for type_ in (orc.Q4_0, orc.Q8_0, orc.Q4_B64, orc.Q8_B64):
        for M, K, N in ((7, 128, 3), (33, 2048, 2), (5, 5632, 1)):
            w = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
            x = rng.standard_normal((N, K)).astype(np.float32)
            packed = orc.quantize(type_, w)
            xq = orc.quantize(orc.Q8_0, x)
            y, a = orc.mul_mat_q8act(type_, packed, K, xq)
            xd = orc.dequantize(orc.Q8_0, xq, K)
            y2, a2 = orc.mul_mat(type_, packed, K, xd)
            assert np.all(np.abs(y - y2) <= 1e-12 * a2)
            assert np.all(a <= a2 * (1 + 1e-12))          # |sum within a block| <= sum of |terms|


def test_quantization_bound_against_float_activations(orc):
    rng = np.random.default_rng(4)
    M, K, N = 40, 2048, 3
    w = WL.weights(77, M, K)
    x = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-3, 3, (N, 1)))).astype(np.float32)
    packed = orc.quantize(orc.Q4_0, w)
    xq = orc.quantize(orc.Q8_0, x)
    y, _ = orc.mul_mat_q8act(orc.Q4_0, packed, K, xq)
    yx, _ = orc.mul_mat(orc.Q4_0, packed, K, x)
    wd = np.abs(orc.dequantize(orc.Q4_0, packed, K).astype(np.float64))            # (M, K)
    dx = xq[:, : 2 * K // 32].copy().view(np.float16).astype(np.float64)           # (N, K/32)
    half_step = np.repeat(dx, 32, axis=1) / 2                                     # (N, K)
    bound = half_step @ wd.T                                                      # (N, M)
    # x / Delta_x is one binary32 division: its rounding adds 2^-24 relative
    assert np.all(np.abs(y - yx) <= bound * (1 + 2.0 ** -20) + 1e-300)
    assert np.abs(y - yx).max() > 0                                               # x was approximated


def test_factored_form_all_ones(orc):
    # all codes 1 in both operands: y = sum_b Delta_w(b) Delta_x(b) * 32
    K = 160
    w = np.zeros((1, orc.row_size(orc.Q8_0, K)), np.uint8)
    xq = np.zeros((1, orc.row_size(orc.Q8_0, K)), np.uint8)
    qoff = 16
    dw = [0.5, 0.25, 2.0, 1.0, 0.125]
    dxs = [1.0, 3.0, 0.5, 0.75, 2.0]
    for b in range(5):
        w[0, 2 * b: 2 * b + 2] = [_f16_bits(dw[b]) & 255, _f16_bits(dw[b]) >> 8]
        xq[0, 2 * b: 2 * b + 2] = [_f16_bits(dxs[b]) & 255, _f16_bits(dxs[b]) >> 8]
    w[0, qoff:qoff + K] = 1
    xq[0, qoff:qoff + K] = 1
    y, _ = orc.mul_mat_q8act(orc.Q8_0, w, K, xq)
    assert y[0, 0] == 32 * sum(a * b for a, b in zip(dw, dxs))


def test_64_block_weights_reduce_to_32_blocks(orc):
    """Weights whose 64-block halves share amax quantize to the same codes
    and scales in both forms (pinned in test_oracle_b64), so the integer path
    gives bit-identical results for the two."""
    rng = np.random.default_rng(5)
    M, K, N = 9, 2048, 3
    w = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    b = w.reshape(M, K // 64, 2, 32)
    b[:, :, 1, :] = -b[:, :, 0, ::-1]
    xq = orc.quantize(orc.Q8_0, rng.standard_normal((N, K)).astype(np.float32))
    for t64, t32 in ((orc.Q4_B64, orc.Q4_0), (orc.Q8_B64, orc.Q8_0)):
        y64, a64 = orc.mul_mat_q8act(t64, orc.quantize(t64, w), K, xq)
        y32, a32 = orc.mul_mat_q8act(t32, orc.quantize(t32, w), K, xq)
        assert np.array_equal(y64, y32) and np.array_equal(a64, a32)
