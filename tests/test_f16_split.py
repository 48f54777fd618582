"""The arithmetic fact the matrix-core GEMV relies on for F16 weights, checked
on the CPU over every binary16 value: a half f splits exactly into
hi = f rounded to bfloat16 (nearest even) and lo = f - hi, with lo itself a
bfloat16 value, never a bfloat16 subnormal (f has 11 significant bits and hi
keeps 8, so |lo| is at most 4 units in f's last place: at most 2 significant
bits); NaN stays NaN in hi, and an infinite half gives lo = NaN.  The kernel feeds hi and lo to two matrix instructions, so the sum
of their products equals f times the activation part exactly.

No GPU and no oracle: this pins the reading of the number formats, not a
kernel (the kernel itself is compared with the oracle by the GPU tests).
"""
import numpy as np


def _rne_bf16(a: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 (as binary32), round to nearest even; NaN kept."""
    b = a.view(np.uint32).astype(np.uint64)
    r = (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    out = r.view(np.float32).copy()
    out[np.isnan(a)] = np.nan
    return out


def _all_halves() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)


def test_every_finite_half_splits_exactly():
    f = _all_halves()
    fin = np.isfinite(f)
    with np.errstate(invalid="ignore"):
        hi = _rne_bf16(f)
        lo = (f - hi).astype(np.float32)
    assert fin.sum() == 63488
    # hi is a bfloat16 value, lo too (its low 16 bits are zero)
    assert ((hi.view(np.uint32) & 0xFFFF)[fin] == 0).all()
    assert ((lo.view(np.uint32) & 0xFFFF)[fin] == 0).all()
    # and the two add back to f exactly (checked in binary64)
    assert (hi[fin].astype(np.float64) + lo[fin].astype(np.float64) == f[fin].astype(np.float64)).all()
    # lo keeps at most 2 significant bits, and is never a bfloat16 subnormal
    nz = fin & (lo != 0)
    assert (np.abs(lo[nz]) >= 2.0 ** -126).all()
    mant = (lo[nz].view(np.uint32) >> 16) & 0x7F
    assert (mant & 0x3F == 0).all()
    assert float(np.max(np.abs(lo[nz]) / np.abs(f[nz]))) < 2.0 ** -8


def test_non_finite_halves():
    f = _all_halves()
    with np.errstate(invalid="ignore"):
        hi = _rne_bf16(f)
        lo = (f - hi).astype(np.float32)
    nan = np.isnan(f)
    inf = np.isinf(f)
    assert nan.sum() == 2046 and inf.sum() == 2
    assert np.isnan(hi[nan]).all()
    assert np.isinf(hi[inf]).all() and (np.sign(hi[inf]) == np.sign(f[inf])).all()
    # Inf - Inf: the row's outputs become NaN on the matrix cores
    assert np.isnan(lo[inf]).all()


def test_rounding_helper_is_nearest_even():
    # ties go to the even bfloat16 neighbour; values in between to the nearest
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, one + 3 * ulp / 4], np.float32)
    assert _rne_bf16(x).tolist() == [1.0, 1.0 + 2 * 2.0 ** -7, 1.0, 1.0 + 2.0 ** -7]
