"""Pins for the oracle's 64-weight blocks (not GPU).

"A Complete Guide to llama.cpp and Customization with C++", §2.2: the block
length B is usually 32 or 64, w_i ~= Delta * q_i with Delta from the block's
max |w| (the pages' rule Delta = amax / 7, q in [-8, 7]; the offset-binary
Q4_0 rule divides by 8, Q8_0 by 127).  A 64-block is one fp16 scale over 64
codes; the codes are stored exactly as in the 32-block rows (runs of 32
codes, Q4 byte j of a run = code j | code j+16 << 4), only the scales halve.

Pinned by: hand-worked blocks whose scale is exact in fp16 (every code then
follows from rounding half away from zero by hand), the reduction to the
already pinned 32-block quantizer (a 64-block whose halves share amax is two
32-blocks with one scale; in general its scale is that of its larger half),
an independent decode of the packed rows (numpy float16 scales times the
codes), the rounding bound |w - W'| <= Delta / 2, and MUL_MAT against a plain
float64 product of the independently decoded weights.
"""
import numpy as np
import pytest


def test_row_sizes(orc):
    for K in (64, 128, 2048, 5632):
        assert orc.row_size(orc.Q8_B64, K) == ((2 * K // 64 + 15) // 16) * 16 + K
        assert orc.row_size(orc.Q4_B64, K) == ((2 * K // 64 + 15) // 16) * 16 + K // 2
    with pytest.raises(ValueError):       # K must be a multiple of 64
        orc.quantize(orc.Q4_B64, np.zeros((1, 96), np.float32))


def test_q4_ramp_block_by_hand(orc):
    """w_i = (i - 32) / 4: amax = 8, so Delta = 8 / 8 = 1 exactly (fp16 0x3C00)
    and q_i = round((i - 32) / 4) with halves rounded away from zero, then
    clamped to [-8, 7] and stored as q + 8."""
    w = (np.arange(64, dtype=np.float32) - 32) / 4
    sb, nib = orc.quantize_block64(orc.Q4_B64, w)
    assert sb == 0x3C00
    expect = ([0, 0, 0] + [1] * 4 + [2] * 4 + [3] * 4 + [4] * 4 + [5] * 4 + [6] * 4 + [7] * 4
              + [8] * 3 + [9] * 4 + [10] * 4 + [11] * 4 + [12] * 4 + [13] * 4 + [14] * 4 + [15] * 6)
    assert len(expect) == 64
    # positions checked by hand: -7.5 -> -8 (i=2), -0.5 -> -1 (i=30), -0.25 -> 0
    # (i=31), 0.5 -> 1 (i=34), 7.5 -> 8 clamped to 7 (i=62)
    assert list(nib) == expect
    assert (nib[2], nib[30], nib[31], nib[34], nib[62]) == (0, 7, 8, 9, 15)


def test_q4_ramp_block_pages_rule_by_hand(orc):
    """The same block with the pages' rule: Delta = fp16(8 / 7) = 1 + 146/1024
    (0x3C92, since 0.142857 * 1024 = 146.29); -8 / Delta = -7.0017 -> -7,
    7.75 / Delta = 6.783 -> 7, 0 -> 0."""
    w = (np.arange(64, dtype=np.float32) - 32) / 4
    sb, nib = orc.quantize_block64(orc.Q4_B64, w, rule=orc.RULE_Q4_SYM7)
    assert sb == 0x3C92
    assert (nib[0], nib[32], nib[63]) == (1, 8, 15)


def test_q8_block_by_hand(orc):
    """w_0 = -127 / 64 and w_i = (i - 32) / 32 otherwise: amax = 127 * 2^-6, so
    Delta = 2^-6 exactly (fp16 0x2400) and q_i = 64 w_i: -127, then 2 (i - 32)."""
    w = (np.arange(64, dtype=np.float32) - 32) / 32
    w[0] = -127.0 / 64.0
    sb, q = orc.quantize_block64(orc.Q8_B64, w)
    assert sb == 0x2400
    assert q[0] == -127
    assert np.array_equal(q[1:].astype(np.int64), 2 * (np.arange(1, 64) - 32))


def _halves_share_amax(rng, M, K):
    w = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    b = w.reshape(M, K // 64, 2, 32)
    b[:, :, 1, :] = -b[:, :, 0, ::-1]          # second half: reversed, negated first half
    return w


@pytest.mark.parametrize("pair", [("Q4_B64", "Q4_0"), ("Q8_B64", "Q8_0")])
def test_reduces_to_32_blocks_when_halves_share_amax(orc, pair):
    """Both halves have the same amax, so the 64-block scale equals each
    32-block's scale and every code equals the 32-block code: the code bytes
    of the two rows coincide, and the 64-block row holds every second scale."""
    t64, t32 = getattr(orc, pair[0]), getattr(orc, pair[1])
    rng = np.random.default_rng(31)
    M, K = 5, 2048
    w = _halves_share_amax(rng, M, K)
    r64, r32 = orc.quantize(t64, w), orc.quantize(t32, w)
    q64, q32 = ((2 * K // 64 + 15) // 16) * 16, ((2 * K // 32 + 15) // 16) * 16
    codes = K if t32 == orc.Q8_0 else K // 2
    assert np.array_equal(r64[:, q64:q64 + codes], r32[:, q32:q32 + codes])
    s64 = r64[:, :2 * K // 64].copy().view(np.uint16)
    s32 = r32[:, :2 * K // 32].copy().view(np.uint16)
    assert np.array_equal(s64, s32[:, 0::2]) and np.array_equal(s64, s32[:, 1::2])


@pytest.mark.parametrize("pair", [("Q4_B64", "Q4_0"), ("Q8_B64", "Q8_0")])
def test_scale_is_that_of_the_larger_half(orc, pair):
    t64, t32 = getattr(orc, pair[0]), getattr(orc, pair[1])
    rng = np.random.default_rng(32)
    for _ in range(20):
        w = (rng.standard_normal(64) * rng.choice([1e-3, 0.05, 3.0])).astype(np.float32)
        sb64, _ = orc.quantize_block64(t64, w)
        big = 0 if np.abs(w[:32]).max() >= np.abs(w[32:]).max() else 1
        sb32, _ = orc.quantize_block(t32, w[32 * big:32 * big + 32])
        assert sb64 == sb32


def _decode(q4, rows, M, K):
    """Values of packed 64-block rows from the layout definition alone."""
    qoff = ((2 * K // 64 + 15) // 16) * 16
    scale = rows[:, :2 * K // 64].copy().view(np.float16).astype(np.float64)
    if q4:
        b = rows[:, qoff:qoff + K // 2].reshape(M, K // 32, 16).astype(np.int64)
        codes = (np.concatenate([b & 15, b >> 4], axis=2) - 8).reshape(M, K)
    else:
        codes = rows[:, qoff:qoff + K].copy().view(np.int8).astype(np.int64)
    return np.repeat(scale, 64, axis=1) * codes


@pytest.mark.parametrize("tname", ["Q4_B64", "Q8_B64"])
def test_decode_bound_and_mul_mat(orc, tname):
    t = getattr(orc, tname)
    rng = np.random.default_rng(33)
    M, K, N = 7, 5632, 3
    w = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    rows = orc.quantize(t, w)
    wd = _decode(tname == "Q4_B64", rows, M, K)
    assert np.array_equal(wd, orc.dequantize(t, rows, K).astype(np.float64))
    delta = np.repeat(rows[:, :2 * K // 64].copy().view(np.float16).astype(np.float64), 64, axis=1)
    if tname == "Q8_B64":
        assert np.all(np.abs(w - wd) <= delta / 2 * (1 + 1e-6))
    else:                                   # away from the clamped top code
        ok = w / np.where(delta > 0, delta, 1) < 7.5
        assert np.all(np.abs(w - wd)[ok] <= delta[ok] / 2 * (1 + 1e-6))
    x = rng.standard_normal((N, K)).astype(np.float32)
    y, a = orc.mul_mat(t, rows, K, x)
    ref = x.astype(np.float64) @ wd.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(a, np.abs(x.astype(np.float64))[:, None, :].__mul__(np.abs(wd)[None]).sum(-1),
                       rtol=1e-12, atol=1e-12)


def test_records_and_integer_path_reject_64_blocks(orc):
    assert orc.record_size(orc.Q4_B64) == 0 and orc.record_size(orc.Q8_B64) == 0
