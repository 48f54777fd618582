"""Pins for the oracle's Q8_0 / Q4_0 quantizer and row packing (not GPU).

Pinned by: hand-worked blocks (tests/golden/q4_0_blocks.txt, q8_0_blocks.txt),
closed-form row sizes, the round-trip bounds that follow from the
definition (|W' - w| <= Delta/2 plus the binary32 quotient rounding for
unclamped codes), idempotence, and code-range invariants on ~10^6 random and
adversarial blocks.

Passages: "Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++",
§6.1 (block = 32 values, one FP16 scale, 16 bytes of 4-bit codes) and §6.2
(dequantize = multiply the unpacked code by the scale); "A Complete Guide to
llama.cpp and Customization with C++", §2.2 (w_i ~= Delta * q_i, Delta from
max |w_i|, q_i in [-8, 7]).
"""
import numpy as np
import pytest

from golden_io import read_blocks


def _layout_offsets(K):
    qoff = ((K // 16) + 15) // 16 * 16
    return qoff


@pytest.mark.parametrize("case", read_blocks("q4_0_blocks.txt"), ids=lambda c: c["name"])
def test_q4_0_hand_worked(orc, case):
    sb, codes = orc.quantize_block(orc.Q4_0, case["w"])
    assert sb == case["scale"]
    assert np.array_equal(codes.astype(np.int64), case["codes"])
    row = orc.quantize(orc.Q4_0, case["w"][None, :])
    assert row.shape == (1, 32)
    assert row[0, :2].tobytes() == bytes([case["scale"] & 0xFF, case["scale"] >> 8])
    assert not row[0, 2:16].any()                      # padding to the 16-byte quant offset
    assert row[0, 16:32].tobytes() == case["bytes"]
    deq = orc.dequantize(orc.Q4_0, row, 32)[0]
    assert np.array_equal(deq, case["deq"])


@pytest.mark.parametrize("case", read_blocks("q8_0_blocks.txt"), ids=lambda c: c["name"])
def test_q8_0_hand_worked(orc, case):
    sb, codes = orc.quantize_block(orc.Q8_0, case["w"])
    assert sb == case["scale"]
    assert np.array_equal(codes.astype(np.int64), case["codes"])
    row = orc.quantize(orc.Q8_0, case["w"][None, :])
    assert row.shape == (1, 48)
    assert row[0, :2].tobytes() == bytes([case["scale"] & 0xFF, case["scale"] >> 8])
    assert not row[0, 2:16].any()
    assert np.array_equal(row[0, 16:48].view(np.int8).astype(np.int64), case["codes"])
    deq = orc.dequantize(orc.Q8_0, row, 32)[0]
    assert np.array_equal(deq, case["deq"])


def test_row_sizes_closed_form(orc):
    # Q8_0 keeps 34 bytes per 32 weights, Q4_0 18 (one fp16 scale each); the
    # row-planar packing pads scales and codes to 16 bytes each.
    for K in (512, 2048, 5632, 256, 4096):
        assert orc.row_size(orc.Q8_0, K) == 17 * K // 16
        assert orc.row_size(orc.Q4_0, K) == 9 * K // 16
    assert orc.row_size(orc.Q4_0, 32) == 32 and orc.row_size(orc.Q8_0, 32) == 48
    assert orc.row_size(orc.Q4_0, 96) == 64 and orc.row_size(orc.Q8_0, 96) == 112
    assert orc.row_size(orc.F16, 2048) == 4096 and orc.row_size(orc.F32, 7) == 28


def test_multi_block_row_layout(orc):
    """Blocks of one row: scale b at bytes 2b, codes of block b at qoff + 16b (Q4_0)
    or qoff + 32b (Q8_0), so each block keeps its hand-worked bytes."""
    q4 = read_blocks("q4_0_blocks.txt")
    w = np.concatenate([c["w"] for c in q4])
    K = w.size
    row = orc.quantize(orc.Q4_0, w[None, :])[0]
    qoff = _layout_offsets(K)
    for b, c in enumerate(q4):
        assert int(row[2 * b]) | (int(row[2 * b + 1]) << 8) == c["scale"]
        assert row[qoff + 16 * b: qoff + 16 * b + 16].tobytes() == c["bytes"]
    assert not row[2 * len(q4): qoff].any()
    q8 = read_blocks("q8_0_blocks.txt")
    w = np.concatenate([c["w"] for c in q8])
    K = w.size
    row = orc.quantize(orc.Q8_0, w[None, :])[0]
    qoff = _layout_offsets(K)
    for b, c in enumerate(q8):
        assert int(row[2 * b]) | (int(row[2 * b + 1]) << 8) == c["scale"]
        assert np.array_equal(row[qoff + 32 * b: qoff + 32 * b + 32].view(np.int8), c["codes"])


def _random_blocks(n_blocks, seed):
    """Gaussian blocks at many magnitudes, plus adversarial ones: a single
    outlier, uniform values, exact multiples of a power of two (quotient ties)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((n_blocks, 32), dtype=np.float32)
    mag = np.float32(2.0) ** rng.integers(-12, 6, (n_blocks, 1)).astype(np.float32)
    w = g * mag
    k = n_blocks // 8
    w[:k, :] *= np.float32(1e-3)
    w[:k, 0] = rng.standard_normal(k).astype(np.float32) * 4
    w[k:2 * k] = rng.uniform(-1, 1, (k, 32)).astype(np.float32)
    w[2 * k:3 * k] = (rng.integers(-64, 65, (k, 32)) / np.float32(64)).astype(np.float32)
    return w.astype(np.float32)


def _scales(orc, type_, packed, nblk):
    sb = packed[:, : 2 * nblk].copy().view(np.uint16)
    return orc.f16_bits_to_f32(sb).astype(np.float64)


@pytest.mark.parametrize("type_name", ["Q8_0", "Q4_0"])
def test_round_trip_bounds(orc, type_name):
    t = getattr(orc, type_name)
    blocks = _random_blocks(1 << 20, 11 if t == orc.Q8_0 else 12)   # ~10^6 blocks
    w = blocks.reshape(-1, 32 * 64)        # rows of 64 blocks (K = 2048)
    packed = orc.quantize(t, w)
    deq = orc.dequantize(t, packed, w.shape[1]).astype(np.float64)
    d = np.repeat(_scales(orc, t, packed, 64), 32, axis=1)
    err = np.abs(deq - w.astype(np.float64))
    normal = d >= 2.0 ** -14                 # normal fp16 scales
    if t == orc.Q8_0:
        # |w/d| <= 127.06 -> binary32 quotient error <= 127.06 * 2^-24 < 2^-17
        assert (err[normal] <= d[normal] * (0.5 + 2.0 ** -17)).all()
        codes = packed[:, 128:].view(np.int8)
        assert codes.min() >= -127 and codes.max() <= 127
    else:
        q = np.where(d > 0, deq / np.where(d > 0, d, 1), 0)
        unclamped = normal & (w.astype(np.float64) < 7.5 * d)
        assert (err[unclamped] <= d[unclamped] * (0.5 + 2.0 ** -21)).all()
        clamped = normal & ~unclamped
        assert clamped.any()
        assert (q[clamped] == 7).all()
        assert (err[clamped] <= d[clamped] * (1 + 2.0 ** -7)).all()
    # the stored scale is the block maximum divided by 127 (Q8_0) or 8 (Q4_0),
    # up to the fp16 rounding (relative 2^-11) for normal scales
    amax = np.abs(w.reshape(w.shape[0], 64, 32)).max(axis=2).astype(np.float64)
    ds = _scales(orc, t, packed, 64)
    div = 127.0 if t == orc.Q8_0 else 8.0
    nz = ds >= 2.0 ** -14
    assert (np.abs(ds[nz] - amax[nz] / div) <= (amax[nz] / div) * 2.0 ** -11).all()


def test_q8_0_idempotent(orc):
    """quant(deq(quant(w))) == quant(w) bitwise for normal scales: the block
    maximum becomes 127 * Delta exactly, and (127 * Delta) / 127 = Delta."""
    w = _random_blocks(1 << 16, 21).reshape(-1, 32)
    p1 = orc.quantize(orc.Q8_0, w)
    d = _scales(orc, orc.Q8_0, p1, 1)[:, 0]
    sel = d >= 2.0 ** -14
    assert sel.sum() > 30000
    p2 = orc.quantize(orc.Q8_0, orc.dequantize(orc.Q8_0, p1[sel], 32))
    assert np.array_equal(p1[sel], p2)


def test_q4_0_idempotent_when_code_minus8_present(orc):
    """Q4_0 re-quantization reproduces the codes when the block holds the code
    -8 (its maximum magnitude is then exactly 8 * Delta); otherwise the
    re-derived scale shrinks, so the statement is only made for such blocks."""
    w = _random_blocks(1 << 16, 22).reshape(-1, 32)
    p1 = orc.quantize(orc.Q4_0, w)
    has_min = (p1[:, 16:32] & 0x0F == 0).any(axis=1) | (p1[:, 16:32] >> 4 == 0).any(axis=1)
    d = _scales(orc, orc.Q4_0, p1, 1)[:, 0]
    sel = has_min & (d >= 2.0 ** -14)
    assert sel.sum() > 1000
    p2 = orc.quantize(orc.Q4_0, orc.dequantize(orc.Q4_0, p1[sel], 32))
    assert np.array_equal(p1[sel], p2)


def test_zero_and_tiny_rows(orc):
    w = np.zeros((3, 64), np.float32)
    w[1, 5] = np.float32(2.0 ** -30)        # scale underflows to fp16 zero
    for t, zero_code in ((orc.Q8_0, 0x00), (orc.Q4_0, 0x88)):
        p = orc.quantize(t, w)
        assert not p[:, :4].any()
        qoff = 16
        codes = p[:, qoff: qoff + (64 if t == orc.Q8_0 else 32)]
        assert (codes == zero_code).all()
        assert not orc.dequantize(t, p, 64).any()
