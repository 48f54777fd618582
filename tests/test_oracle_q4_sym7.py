"""Pins for the oracle's symmetric /7 Q4 rule (not GPU).

"A Complete Guide to llama.cpp and Customization with C++", §2.2: each block
is approximated as w_i ~= Delta * q_i with q_i in [-8, 7] and Delta =
max |w| / 7.  Stored as Q4_0 is ("Development Guide for Small AI Models
(TinyLLaMA, etc.) Using C++", §6.1): the fp16 Delta and the nibble q + 8.

Pinned by: hand-worked blocks (tests/golden/q4_sym7_blocks.txt); the bound
the rule guarantees and the /8 rule cannot (|W' - w| <= Delta/2 for every
weight: no code clamps) on random and adversarial blocks; the code range
[1, 15] (q = -8 is never produced); and agreement with the default rule's
packing on the bytes that do not depend on the divisor (layout, padding).
"""
import numpy as np
import pytest

from golden_io import read_blocks


@pytest.mark.parametrize("case", read_blocks("q4_sym7_blocks.txt"), ids=lambda c: c["name"])
def test_hand_worked(orc, case):
    sb, codes = orc.quantize_block("q4_sym7", case["w"])
    assert sb == case["scale"]
    assert np.array_equal(codes.astype(np.int64), case["codes"])
    row = orc.quantize(orc.Q4_0, case["w"][None, :], rule=orc.RULE_Q4_SYM7)
    assert row[0, :2].tobytes() == bytes([case["scale"] & 0xFF, case["scale"] >> 8])
    assert not row[0, 2:16].any()
    assert row[0, 16:32].tobytes() == case["bytes"]
    assert np.array_equal(orc.dequantize(orc.Q4_0, row, 32)[0], case["deq"])


def _blocks(seed, n):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, 32)).astype(np.float32) * np.float32(0.02)
    scale = np.float32(2.0) ** rng.integers(-12, 8, n).astype(np.float32)
    w *= scale[:, None]
    w[::17] = 0.0
    w[5::23, 3] = -np.abs(w[5::23]).max(axis=1) * 1.0001     # a negative extreme
    return w.astype(np.float32)


def test_round_trip_bound_and_code_range(orc):
    w = _blocks(21, 20000)
    rows = orc.quantize(orc.Q4_0, w, rule=orc.RULE_Q4_SYM7)
    deq = orc.dequantize(orc.Q4_0, rows, 32)
    scale = rows[:, :2].copy().view(np.float16)[:, 0].astype(np.float64)
    err = np.abs(deq.astype(np.float64) - w.astype(np.float64))
    # |w / Delta_fp16| <= 7 (1 + 2^-11) < 7.5: every code is the rounded
    # quotient, so the error is half a step, plus the binary32 rounding of
    # the quotient (relative 2^-24 of at most 7.5 steps)
    assert (err <= scale[:, None] * (0.5 + 7.5 * 2.0 ** -24)).all()
    codes = np.concatenate([rows[:, 16:32] & 15, rows[:, 16:32] >> 4], axis=1)
    nonzero = scale > 0
    assert codes[nonzero].min() >= 1 and codes.max() <= 15
    assert (codes[~nonzero] == 8).all()


def test_differs_from_default_rule_only_in_scale_and_codes(orc):
    w = _blocks(22, 64).reshape(2, 1024)
    a = orc.quantize(orc.Q4_0, w)
    b = orc.quantize(orc.Q4_0, w, rule=orc.RULE_Q4_SYM7)
    assert a.shape == b.shape
    qoff = ((1024 // 16) + 15) // 16 * 16
    assert not a[:, 64:qoff].any() and not b[:, 64:qoff].any()
    sa = a[:, :64].copy().view(np.float16).astype(np.float64)
    sb = b[:, :64].copy().view(np.float16).astype(np.float64)
    normal = sa >= 2.0 ** -14           # fp16 normal: 11 significant bits
    assert normal.sum() > 40
    # amax/7 against amax/8: the ratio is 8/7 up to the two fp16 roundings
    assert np.allclose(sb[normal] / sa[normal], 8.0 / 7.0, rtol=2.0 ** -10)


def test_rule_rejected_for_q8(orc):
    with pytest.raises(ValueError):
        orc.quantize(orc.Q8_0, np.zeros((1, 32), np.float32), rule=orc.RULE_Q4_SYM7)
