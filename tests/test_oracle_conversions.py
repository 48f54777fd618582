"""Pins for the oracle's IEEE conversions (not GPU).

The oracle converts binary32 to binary16 / bfloat16 from the format
definitions.  It is pinned here against (a) hand-worked boundary points
(tests/golden/conversion_points.txt) and (b) two independent implementations:
numpy's float16 cast and torch's CPU bfloat16 cast, over every upper 16-bit
half of binary32 combined with the lower halves that decide rounding (ties,
just-below / just-above ties, sticky bits), plus all 2^16 narrow -> binary32
patterns.  Setting QMM_EXHAUSTIVE=1 also sweeps all 2^32 binary32 inputs.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from golden_io import read_conversion_points

# Lower 16-bit halves that exercise every rounding decision of both targets:
# binary16 keeps 10 fraction bits (round bit = bit 12, sticky = bits 0..11);
# bfloat16 keeps 7 (round bit = bit 15, sticky = bits 0..14).  Bit 13 (the
# binary16 LSB) and the sticky bits vary independently.
_LOW = sorted({0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001,
               0x2FFF, 0x3000, 0x3001, 0x4000, 0x7FFF, 0x8000, 0x8001, 0x9000,
               0xA000, 0xB000, 0xBFFF, 0xC000, 0xE000, 0xEFFF, 0xF000, 0xFFFF}
              | set(np.random.default_rng(7).integers(0, 1 << 16, 40).tolist()))


def _f32_patterns() -> np.ndarray:
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    low = np.array(_LOW, np.uint32)
    return (hi[:, None] | low[None, :]).reshape(-1)


def _is_nan16(bits, exp_mask, man_mask):
    return ((bits & exp_mask) == exp_mask) & ((bits & man_mask) != 0)


def _check_f16(orc, bits32: np.ndarray):
    f = bits32.view(np.float32)
    got = orc.f32_to_f16_bits(f)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert _is_nan16(got[nan], 0x7C00, 0x03FF).all()
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, [(hex(int(bits32[i])), hex(int(got[i])), hex(int(ref[i]))) for i in bad[:8]]


def _check_bf16(orc, bits32: np.ndarray):
    f = bits32.view(np.float32)
    got = orc.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert _is_nan16(got[nan], 0x7F80, 0x007F).all()
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, [(hex(int(bits32[i])), hex(int(got[i])), hex(int(ref[i]))) for i in bad[:8]]


def test_hand_worked_points(orc):
    for target, fbits, expect in read_conversion_points():
        f = np.array([fbits], np.uint32).view(np.float32)
        got = orc.f32_to_f16_bits(f)[0] if target == "f16" else orc.f32_to_bf16_bits(f)[0]
        assert int(got) == expect, (target, hex(fbits), hex(int(got)), hex(expect))


def test_f32_to_f16_every_upper_half(orc):
    _check_f16(orc, _f32_patterns())


def test_f32_to_bf16_every_upper_half(orc):
    _check_bf16(orc, _f32_patterns())


def test_f16_to_f32_all_patterns(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_all_patterns(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_bits_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_round_trip_narrow_values(orc):
    """Every finite binary16 / bfloat16 value converts to binary32 and back unchanged."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin16 = (h & 0x7C00) != 0x7C00
    assert np.array_equal(orc.f32_to_f16_bits(orc.f16_bits_to_f32(h[fin16])), h[fin16])
    fin_b = (h & 0x7F80) != 0x7F80
    assert np.array_equal(orc.f32_to_bf16_bits(orc.bf16_bits_to_f32(h[fin_b])), h[fin_b])


@pytest.mark.skipif(os.environ.get("QMM_EXHAUSTIVE") != "1",
                    reason="all 2^32 inputs take minutes; set QMM_EXHAUSTIVE=1")
def test_exhaustive_all_binary32(orc):
    chunk = 1 << 24

    def run(c):
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        _check_f16(orc, bits)
        _check_bf16(orc, bits)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(run, range((1 << 32) // chunk)))
