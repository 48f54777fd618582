"""GPU parity: libqmm's HIP kernels against the CPU oracle, through the C ABI.

Bars:
  * quantize / dequantize: bit-exact (bytes of the packed rows, bits of W');
  * GEMV (fp32 activations): |y - y_ref| <= 1e-4 * a + 1e-6 per output;
  * GEMM (bf16 activations, bf16 matrix cores): |y - y_ref| <= 1e-2 * a + 1e-5,
    and against the oracle's bf16-weight variant within the binary32
    summation bound 1.1 * K * 2^-24 * a + 1e-7 (the kernel rounds W' to bf16
    and accumulates in fp32; nothing else may differ);
where y_ref = sum_k W'[m][k] x[n][k] and a = sum_k |W'[m][k] x[n][k]| come from
the oracle in binary64.  Inputs are seeded (quantized_matmul_ggml_amd.workloads).
Outputs are written into guard-banded buffers whose margins must stay intact.
"""
import ctypes

import numpy as np
import pytest
import torch

import quantized_matmul_ggml_amd as Q
from quantized_matmul_ggml_amd import binding as B
from quantized_matmul_ggml_amd import workloads as WL
from golden_io import read_blocks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TYPES = {"Q8_0": (B.Q8_0, 3), "Q4_0": (B.Q4_0, 4), "F16": (B.F16, 1),   # (qmm, oracle) ids
         "Q8_B64": (B.Q8_B64, 5), "Q4_B64": (B.Q4_B64, 6)}
CANARY = np.float32(np.array([0x7FC0DEAD], np.uint32).view(np.float32)[0])


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _guarded_out(rows, cols, pad_rows=2, pad_cols=8):
    buf = torch.full((rows + 2 * pad_rows, cols + 2 * pad_cols), float(CANARY),
                     dtype=torch.float32, device=DEV)
    view = buf[pad_rows:pad_rows + rows, pad_cols:pad_cols + cols]
    return buf, view


def _check_guard(buf, pad_rows=2, pad_cols=8):
    b = buf.cpu().numpy().view(np.uint32)
    canary = np.uint32(0x7FC0DEAD)
    inner = np.zeros(b.shape, bool)
    inner[pad_rows:b.shape[0] - pad_rows, pad_cols:b.shape[1] - pad_cols] = True
    assert (b[~inner] == canary).all(), "kernel wrote outside its output"


def _assert_tol(y, yref, a, rel, abs_, what):
    y = np.asarray(y, np.float64)
    err = np.abs(y - yref)
    bound = rel * a + abs_
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    assert ratio.max() <= 1.0, (f"{what}: worst |err|/bound = {ratio.max():.3g} at {worst}, "
                                f"y={y[worst]!r} ref={yref[worst]!r} a={a[worst]!r}")


def _oracle_weight(orc, tname, w32):
    """Oracle-side packed rows (or fp16 rows as bytes) of fp32 weights."""
    if tname == "F16":
        return WL.round_f16(w32).view(np.uint8).reshape(w32.shape[0], 2 * w32.shape[1])
    return orc.quantize(TYPES[tname][1], w32)


def _gpu_weight(tname, w32, pitch=None):
    if tname == "F16":
        h = torch.from_numpy(WL.round_f16(w32)).to(DEV)
        if pitch is not None:
            buf = torch.zeros((w32.shape[0], pitch // 2), dtype=torch.float16, device=DEV)
            buf[:, : w32.shape[1]] = h
            h = buf
        return B.Weight(h, B.F16, w32.shape[1], w32.shape[0])
    return Q.quantize(torch.from_numpy(w32).to(DEV), TYPES[tname][0], pitch=pitch)


# ---------------------------------------------------------------- quantize

QUANT_SHAPES = [(1, 32), (3, 96), (257, 160), (64, 2048), (129, 5632), (5, 32768)]


def _adversarial(M, K, seed):
    """Gaussian rows at many magnitudes plus blocks that hit ties, clamps,
    zero blocks and subnormal fp16 scales."""
    return WL.adversarial_weights(seed, M, K)


@pytest.mark.parametrize("tname", ["Q8_0", "Q4_0"])
@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_bit_exact(orc, tname, shape):
    M, K = shape
    _banner(f"quantize {tname} {M}x{K}")
    w = _adversarial(M, K, 100 + M + K)
    ref = orc.quantize(TYPES[tname][1], w)
    got = Q.quantize(torch.from_numpy(w).to(DEV), TYPES[tname][0])
    torch.cuda.synchronize()
    assert np.array_equal(got.data.cpu().numpy(), ref)


@pytest.mark.parametrize("tname", ["Q8_0", "Q4_0"])
def test_quantize_padded_pitch(orc, tname):
    M, K = 33, 2048 + 32
    _banner(f"quantize padded pitch {tname}")
    w = _adversarial(M, K, 7)
    rs = B.row_size(TYPES[tname][0], K)
    got = Q.quantize(torch.from_numpy(w).to(DEV), TYPES[tname][0], pitch=rs + 48)
    torch.cuda.synchronize()
    g = got.data.cpu().numpy()
    assert np.array_equal(g[:, :rs], orc.quantize(TYPES[tname][1], w))
    assert not g[:, rs:].any()


@pytest.mark.parametrize("tname,fixture", [("Q4_0", "q4_0_blocks.txt"), ("Q8_0", "q8_0_blocks.txt")])
def test_quantize_hand_worked_blocks(tname, fixture):
    _banner(f"quantize hand-worked {tname}")
    cases = read_blocks(fixture)
    w = np.stack([c["w"] for c in cases])
    got = Q.quantize(torch.from_numpy(w).to(DEV), TYPES[tname][0]).data.cpu().numpy()
    for i, c in enumerate(cases):
        assert int(got[i, 0]) | (int(got[i, 1]) << 8) == c["scale"], c["name"]
        if tname == "Q4_0":
            assert got[i, 16:32].tobytes() == c["bytes"], c["name"]
        else:
            assert np.array_equal(got[i, 16:48].view(np.int8).astype(np.int64), c["codes"]), c["name"]


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_q4_amax7_bit_exact(orc, shape):
    """The pages' symmetric rule (amax / 7) against the oracle, byte for byte."""
    M, K = shape
    _banner(f"quantize q4 amax7 {M}x{K}")
    w = _adversarial(M, K, 500 + M + K)
    ref = orc.quantize(orc.Q4_0, w, rule=orc.RULE_Q4_SYM7)
    got = Q.quantize(torch.from_numpy(w).to(DEV), B.Q4_0, rule=B.QUANT_Q4_AMAX7)
    torch.cuda.synchronize()
    assert np.array_equal(got.data.cpu().numpy(), ref)


def test_quantize_q4_amax7_hand_worked():
    _banner("quantize q4 amax7 hand-worked")
    cases = read_blocks("q4_sym7_blocks.txt")
    w = np.stack([c["w"] for c in cases])
    got = Q.quantize(torch.from_numpy(w).to(DEV), B.Q4_0, rule=B.QUANT_Q4_AMAX7).data.cpu().numpy()
    for i, c in enumerate(cases):
        assert int(got[i, 0]) | (int(got[i, 1]) << 8) == c["scale"], c["name"]
        assert got[i, 16:32].tobytes() == c["bytes"], c["name"]


def test_q4_amax7_weights_through_gemv_and_gemm(orc):
    """amax/7 rows are ordinary Q4_0 rows: the GEMV and the GEMM read them
    unchanged (the Wdown shape, one token and 300 tokens)."""
    M, K = 2048, 5632
    _banner("q4 amax7 weights: gemv + gemm")
    w = WL.weights(WL.seed(3, 6), M, K)
    packed = orc.quantize(orc.Q4_0, w, rule=orc.RULE_Q4_SYM7)
    wt = Q.quantize(torch.from_numpy(w).to(DEV), B.Q4_0, rule=B.QUANT_Q4_AMAX7)
    assert np.array_equal(wt.data.cpu().numpy(), packed)
    x = WL.activations(WL.seed(3, 10), 1, K)
    yref, a = orc.mul_mat(orc.Q4_0, packed, K, x)
    y = Q.gemv(wt, torch.from_numpy(x).to(DEV)).cpu().numpy()
    _assert_tol(y, yref, a, 1e-4, 1e-6, "gemv amax7")
    xb = WL.round_bf16_bits(WL.activations(WL.seed(3, 11), 300, K))
    ms = np.repeat(np.arange(0, M, 37), 4)            # sampled rows ...
    ns = np.tile(np.array([0, 1, 150, 299]), ms.size // 4)   # ... and tokens
    yr, ar = orc.mul_mat_pairs(orc.Q4_0, packed, K, xb, ms, ns, x_bf16_bits=True)
    yg = Q.gemm(wt, WL.bf16_bits_to_torch(xb, DEV)).cpu().numpy()
    assert (np.abs(yg[ns, ms] - yr) <= 1e-2 * ar + 1e-5).all()


def test_quantize_full_size_weights(orc):
    _banner("quantize full-size LM head (Q8_0) and decoder layer (Q4_0)")
    w = WL.weights(WL.seed(4, 0), WL.VOCAB, WL.HIDDEN)
    got = Q.quantize(torch.from_numpy(w).to(DEV), B.Q8_0).data.cpu().numpy()
    assert np.array_equal(got, orc.quantize(orc.Q8_0, w))
    for t, (name, M, K, _) in enumerate(WL.LAYER):
        w = WL.weights(WL.seed(3, t), M, K)
        got = Q.quantize(torch.from_numpy(w).to(DEV), B.Q4_0).data.cpu().numpy()
        assert np.array_equal(got, orc.quantize(orc.Q4_0, w)), name


@pytest.mark.parametrize("tname", ["Q8_0", "Q4_0", "F16"])
def test_dequantize_bit_exact(orc, tname):
    M, K = 67, 2048 + 96
    _banner(f"dequantize {tname}")
    w = _adversarial(M, K, 3)
    packed = _oracle_weight(orc, tname, w)
    ref = orc.dequantize(TYPES[tname][1], packed, K)
    if tname == "F16":
        wt = B.Weight(torch.from_numpy(WL.round_f16(w)).to(DEV), B.F16, K, M)
    else:
        wt = B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)
    got = Q.dequantize(wt).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


QUANT_SHAPES_B64 = [(1, 64), (3, 128), (257, 192), (64, 2048), (129, 5632), (5, 32768)]


@pytest.mark.parametrize("tname,rule", [("Q8_B64", 0),
                                        ("Q4_B64", 0), ("Q4_B64", 1)])
@pytest.mark.parametrize("shape", QUANT_SHAPES_B64, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_64_blocks_bit_exact(orc, tname, rule, shape):
    """64-weight blocks, both Q4 rules (rule 1: the pages' amax/7)."""
    M, K = shape
    _banner(f"quantize {tname} rule {rule} {M}x{K}")
    w = _adversarial(M, K, 300 + M + K)
    ref = orc.quantize(TYPES[tname][1], w, rule=rule)
    got = Q.quantize(torch.from_numpy(w).to(DEV), TYPES[tname][0], rule=rule)
    torch.cuda.synchronize()
    assert np.array_equal(got.data.cpu().numpy(), ref)


@pytest.mark.parametrize("tname", ["Q8_B64", "Q4_B64"])
def test_dequantize_64_blocks_bit_exact(orc, tname):
    M, K = 67, 2048 + 192
    _banner(f"dequantize {tname}")
    w = _adversarial(M, K, 5)
    packed = orc.quantize(TYPES[tname][1], w)
    ref = orc.dequantize(TYPES[tname][1], packed, K)
    rs = B.row_size(TYPES[tname][0], K)
    buf = torch.full((M, rs + 32), 0x7F, dtype=torch.uint8, device=DEV)   # padded pitch, junk padding
    buf[:, :rs] = torch.from_numpy(packed).to(DEV)
    got = Q.dequantize(B.Weight(buf, TYPES[tname][0], K, M)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- GEMV

GEMV_CASES = [
    # (type, M, K, N)
    ("Q8_0", 512, 512, 1),          # the 512 x 512 Q8_0 decode GEMV
    ("Q8_0", 1, 32, 1), ("Q8_0", 3, 96, 3), ("Q8_0", 257, 160, 5), ("Q8_0", 4097, 2048, 2),
    ("Q8_0", 130, 4096, 8), ("Q8_0", 64, 16384, 1), ("Q8_0", 300, 2048, 7),
    ("Q4_0", 1, 32, 1), ("Q4_0", 257, 5632, 1), ("Q4_0", 4100, 2048, 1), ("Q4_0", 100, 2048, 3),
    ("Q4_0", 33, 32768, 1), ("Q4_0", 5, 8192, 4), ("Q4_0", 300, 2048, 8), ("Q4_0", 4099, 2048, 2),
    # rows over 4096 at one token on more row groups than the 512 workgroups
    ("Q4_0", 4100, 8192, 1), ("Q8_0", 3000, 5632, 1),
    ("F16", 5632, 2048, 1),         # the fp16 FFN up-projection GEMV
    ("F16", 1, 7, 1), ("F16", 65, 1000, 2), ("F16", 4101, 2048, 1), ("F16", 10, 8192, 1),
    ("F16", 77, 520, 8),
    # 5+ tokens with K <= 4096 run on the matrix cores: partial block groups
    # (K = 96, 160, 1056, 2080), 4 and 8 waves per row range, and K just
    # past that kernel's range
    ("Q4_0", 40, 96, 5), ("Q4_0", 257, 160, 6), ("Q4_0", 17, 1056, 5), ("Q4_0", 1000, 4096, 6),
    ("Q8_0", 31, 2080, 6), ("Q8_0", 1001, 4096, 5), ("Q8_0", 64, 4128, 8),
    # 3 and 4 tokens over more than 2048 rows take the matrix cores too;
    # 2048 rows stay on the VALU kernel
    ("Q4_0", 8200, 2048, 3), ("Q8_0", 8195, 1024, 4), ("Q4_0", 2049, 2048, 3), ("Q8_0", 2600, 1024, 4),
    ("Q4_0", 2048, 2048, 3),
    # K of 129..192 blocks: one twelve-wave launch (16-row Q4_0 tiles, 8-row
    # Q8_0 tiles), from 3 tokens; the down projection itself at 8 tokens
    ("Q4_0", 300, 5632, 6), ("Q4_0", 2048, 5632, 8), ("Q4_0", 37, 4128, 3), ("Q8_0", 300, 5632, 5),
    ("Q8_0", 45, 6144, 4), ("Q8_0", 2048, 5632, 8),
    # K beyond 192 blocks: passes of 128 blocks that add to y (7-8 tokens;
    # fewer stay on the VALU kernel)
    ("Q4_0", 100, 6176, 7), ("Q8_0", 77, 16384, 8), ("Q8_0", 77, 16384, 5),
    # the streaming kernel (F16 rows; two tokens; Q8_0 over 8192 rows at one
    # token) with ragged groups and grids, and shapes past its limits that
    # stay on the other kernel (more than 8 row groups per wave; wide rows)
    ("Q8_0", 9001, 2048, 1), ("Q8_0", 70001, 512, 1), ("F16", 4097, 1024, 2), ("F16", 33, 4096, 1),
    ("Q4_0", 4099, 4096, 2), ("Q8_0", 8193, 2048, 2), ("F16", 70001, 256, 1),
    # 64-weight blocks (one scale per two 32-code runs)
    ("Q4_B64", 5632, 2048, 1), ("Q8_B64", 300, 5632, 3), ("Q4_B64", 100, 192, 8), ("Q8_B64", 4099, 2048, 2),
    ("Q4_B64", 64, 16384, 5), ("Q8_B64", 1, 64, 1), ("Q4_B64", 8200, 2048, 4),
    ("Q4_B64", 129, 5632, 7), ("Q8_B64", 64, 4160, 8), ("Q4_B64", 64, 16384, 8),
    # F16 rows (K a multiple of 32) on the matrix cores from 5 tokens: the
    # 5632 x 2048 up-projection at 8, 4 and 16 blocks per wave (8-row
    # tiles), K past 4096 in two passes (16 then 8 blocks per wave, 8- then
    # 16-row tiles); from 3 tokens over 16384 rows or K above 8192 (three
    # passes); K not a multiple of 32 stays on the VALU kernel
    ("F16", 5632, 2048, 8), ("F16", 37, 96, 6), ("F16", 1001, 4096, 5), ("F16", 300, 5632, 7),
    ("F16", 16400, 256, 3), ("F16", 64, 8224, 3), ("F16", 129, 1040, 6),
    # F16 rows past 2048 on the VALU kernel: four waves per row of 2 or 4
    # chunks per lane (two rows per group at one token)
    ("F16", 5632, 2048, 3), ("F16", 2049, 1024, 4), ("F16", 1000, 4096, 1), ("F16", 1000, 4096, 2),
    ("F16", 300, 5632, 2), ("F16", 999, 4096, 4),
    # Q8_0 rows past 4096 at one and two tokens: four waves per row (2 and 4
    # chunks per lane, two rows per group)
    ("Q8_0", 1000, 8192, 1), ("Q8_0", 501, 8192, 2), ("Q8_0", 300, 11008, 1), ("Q8_B64", 257, 8192, 2),
]


def _run_gemv(orc, tname, M, K, N, seed, w_pitch=None, x_pad=0, y_pad=8):
    w = WL.weights(seed, M, K)
    x = WL.activations(seed + 1, N, K)
    packed = _oracle_weight(orc, tname, w)
    yref, a = orc.mul_mat(TYPES[tname][1], packed, K, x)
    wt = _gpu_weight(tname, w, pitch=w_pitch)
    xbuf = torch.zeros((N, K + x_pad), dtype=torch.float32, device=DEV)
    xbuf[:, :K] = torch.from_numpy(x).to(DEV)
    buf, yv = _guarded_out(N, M, pad_cols=y_pad)
    Q.gemv(wt, xbuf[:, :K], out=yv)
    torch.cuda.synchronize()
    _check_guard(buf, pad_cols=y_pad)
    return yv.cpu().numpy(), yref, a


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_parity(orc, case):
    tname, M, K, N = case
    _banner(f"gemv {tname} M={M} K={K} N={N}")
    y, yref, a = _run_gemv(orc, tname, M, K, N, seed=10 * M + K + N)
    _assert_tol(y, yref, a, 1e-4, 1e-6, f"gemv {case}")


def test_gemv_strided_operands(orc):
    """Padded weight pitch, x rows with a larger pitch, y rows with a larger pitch."""
    for tname in ("Q8_0", "Q4_0", "F16"):
        K = 2048
        _banner(f"gemv strided {tname}")
        pitch = B.row_size(TYPES[tname][0], K) + 64 if tname != "F16" else 2 * K + 64
        for N in (3, 6):
            y, yref, a = _run_gemv(orc, tname, 70, K, N, seed=5, w_pitch=pitch, x_pad=12, y_pad=5)
            _assert_tol(y, yref, a, 1e-4, 1e-6, f"gemv strided {tname} N={N}")


@pytest.mark.parametrize("K,N", [(7, 3), (1003, 3), (2051, 3), (1024, 6)])
def test_gemv_f16_tail_with_nan_padding(orc, K, N):
    """F16 rows whose K is not a multiple of 8 (and, at 6 tokens on the
    matrix cores, whole 32-blocks), stored with a row pitch whose padding
    holds NaN: only the halves inside each row may contribute."""
    M = 37
    _banner(f"gemv f16 tail K={K} N={N} nan padding")
    w = WL.weights(900 + K, M, K)
    x = WL.activations(901 + K, N, K)
    pitch = (K + 7) // 8 * 8 + 8            # halves; the pitch is 16-byte aligned
    buf = torch.full((M, pitch), float("nan"), dtype=torch.float16, device=DEV)
    buf[:, :K] = torch.from_numpy(WL.round_f16(w)).to(DEV)
    wt = B.Weight(buf, B.F16, K, M)
    y = Q.gemv(wt, torch.from_numpy(x).to(DEV)).cpu().numpy()
    yref, a = orc.mul_mat(TYPES["F16"][1], _oracle_weight(orc, "F16", w), K, x)
    _assert_tol(y, yref, a, 1e-4, 1e-6, f"gemv f16 tail K={K}")


@pytest.mark.parametrize("N", [1, 6])
def test_gemv_f16_special_weights(orc, N):
    """F16 weights at the edges of the format: the largest finite half,
    subnormal halves and signed zeros everywhere else; rows holding an
    infinite or NaN weight give non-finite outputs (one token on the VALU
    kernel: IEEE Inf or NaN; six on the matrix cores: NaN), every other row
    stays within the bound."""
    M, K = 96, 2048
    _banner(f"gemv f16 special weights N={N}")
    w = WL.round_f16(WL.weights(77, M, K))
    rng = np.random.default_rng(78)
    w[0:8, rng.integers(0, K, 8)] = np.float16(65504.0)
    w[8:16, :] = (rng.integers(-1023, 1024, (8, K)) * 2.0 ** -24).astype(np.float16)   # subnormal halves
    w[16:24, :] = np.where(rng.random((8, K)) < 0.5, np.float16(0.0), np.float16(-0.0))
    w[24, 5] = np.float16(np.inf)
    w[25, 900] = -np.float16(np.inf)
    w[26, 2047] = np.float16(np.nan)
    x = WL.activations(79, N, K)
    packed = w.view(np.uint8).reshape(M, 2 * K)
    wt = B.Weight(torch.from_numpy(w).to(DEV), B.F16, K, M)
    y = Q.gemv(wt, torch.from_numpy(x).to(DEV)).cpu().numpy().astype(np.float64)
    bad = [24, 25, 26]
    assert not np.isfinite(y[:, bad]).any()
    ok = np.setdiff1d(np.arange(M), bad)
    yref, a = orc.mul_mat(TYPES["F16"][1], packed[ok], K, x)
    _assert_tol(y[:, ok], yref, a, 1e-4, 1e-6, f"gemv f16 special N={N}")
    assert (y[:, 16:24] == 0.0).all()


def _swiglu_tol(orc, gref, ga, uref, ua, h):
    """Bound of the fused gate/up SwiGLU: the GEMV bound of each sum carried
    through Swish (|Swish'| <= 1.1) and the product, plus binary32 rounding of
    the epilogue (a few ulps of h)."""
    eg = 1e-4 * ga + 1e-6
    eu = 1e-4 * ua + 1e-6
    sg = np.array([orc.swish(v) for v in gref.ravel()]).reshape(gref.shape)
    return 1.1 * eg * (np.abs(uref) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(h)


SWIGLU_CASES = [
    ("Q4_0", 5632, 2048, 1),       # the TinyLLaMA feed-forward gate/up pair
    ("Q4_0", 37, 96, 1), ("Q4_0", 300, 1024, 2), ("Q4_0", 129, 2048, 3),
    ("Q8_0", 513, 512, 8), ("Q8_0", 64, 4096, 5), ("Q8_0", 1, 32, 1),
    ("F16", 77, 1003, 2), ("F16", 260, 2048, 4),
    ("Q4_B64", 300, 2048, 2), ("Q8_B64", 65, 192, 1),
    # from 3 tokens the matrix-core kernel (8 gate + 8 up rows per tile, K
    # up to 4096); longer rows stay on the VALU kernel
    ("Q4_0", 5632, 2048, 8), ("Q4_0", 300, 1024, 5), ("Q4_B64", 130, 4096, 6), ("Q8_B64", 77, 512, 4),
    ("Q4_0", 37, 4128, 8),
]


@pytest.mark.parametrize("case", SWIGLU_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_swiglu_parity(orc, case):
    tname, M, K, N = case
    _banner(f"gemv swiglu {tname} M={M} K={K} N={N}")
    seed = 7 * M + K + N
    wg, wu = WL.weights(seed, M, K), WL.weights(seed + 1, M, K)
    x = WL.activations(seed + 2, N, K)
    gref, ga = orc.mul_mat(TYPES[tname][1], _oracle_weight(orc, tname, wg), K, x)
    uref, ua = orc.mul_mat(TYPES[tname][1], _oracle_weight(orc, tname, wu), K, x)
    href = orc.swiglu(gref, uref)
    pitch = (2 * K + 15) // 16 * 16 if tname == "F16" else None   # F16 rows 16-byte aligned
    h = Q.gemv_swiglu(_gpu_weight(tname, wg, pitch), _gpu_weight(tname, wu, pitch),
                      torch.from_numpy(x).to(DEV))
    h = h.cpu().numpy().astype(np.float64)
    tol = _swiglu_tol(orc, gref, ga, uref, ua, href)
    err = np.abs(h - href)
    assert np.isfinite(h).all()
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


def test_gemv_swiglu_saturated_and_separate_pitches(orc):
    """|gate| in the hundreds (e^{-z} overflows for the negative ones), the
    up matrix stored with a padded pitch, and rows and tokens that fill no
    whole group."""
    M, K, N = 203, 256, 3
    _banner("gemv swiglu saturated, separate pitches")
    wg, wu = WL.weights(41, M, K), WL.weights(42, M, K)
    x = (WL.activations(43, N, K) * np.float32(400.0)).astype(np.float32)
    gref, ga = orc.mul_mat(orc.Q8_0, orc.quantize(orc.Q8_0, wg), K, x)
    uref, ua = orc.mul_mat(orc.Q8_0, orc.quantize(orc.Q8_0, wu), K, x)
    assert np.abs(gref).max() > 100.0 and gref.min() < -88.0
    href = orc.swiglu(gref, uref)
    gw = Q.quantize(torch.from_numpy(wg).to(DEV), B.Q8_0)
    uw = Q.quantize(torch.from_numpy(wu).to(DEV), B.Q8_0, pitch=B.row_size(B.Q8_0, K) + 48)
    h = Q.gemv_swiglu(gw, uw, torch.from_numpy(x).to(DEV)).cpu().numpy().astype(np.float64)
    tol = _swiglu_tol(orc, gref, ga, uref, ua, href)
    assert np.isfinite(h).all()
    assert (np.abs(h - href) <= tol).all()


def test_gemv_decoder_layer_full_size(orc):
    """The seven projections of one TinyLLaMA-shaped layer, Q4_0, one token."""
    xs = [WL.activations(WL.seed(3, 7 + s), 1, k) for s, k in enumerate(WL.LAYER_X_K)]
    for t, (name, M, K, slot) in enumerate(WL.LAYER):
        _banner(f"gemv layer {name} {M}x{K}")
        w = WL.weights(WL.seed(3, t), M, K)
        packed = orc.quantize(orc.Q4_0, w)
        yref, a = orc.mul_mat(orc.Q4_0, packed, K, xs[slot])
        wt = B.Weight(torch.from_numpy(packed).to(DEV), B.Q4_0, K, M)
        y = Q.gemv(wt, torch.from_numpy(xs[slot]).to(DEV)).cpu().numpy()
        _assert_tol(y, yref, a, 1e-4, 1e-6, f"layer {name}")


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_gemv_lm_head_full_size(orc, N):
    """The 32000 x 2048 Q8_0 LM head with 1, 2, 4 and 8 tokens."""
    _banner(f"gemv lm head N={N}")
    w = WL.weights(WL.seed(4, 0), WL.VOCAB, WL.HIDDEN)
    x = WL.activations(WL.seed(4, 1), N, WL.HIDDEN)
    packed = orc.quantize(orc.Q8_0, w)
    yref, a = orc.mul_mat(orc.Q8_0, packed, WL.HIDDEN, x)
    wt = B.Weight(torch.from_numpy(packed).to(DEV), B.Q8_0, WL.HIDDEN, WL.VOCAB)
    y = Q.gemv(wt, torch.from_numpy(x).to(DEV)).cpu().numpy()
    _assert_tol(y, yref, a, 1e-4, 1e-6, f"lm head N={N}")


@pytest.mark.parametrize("tname", ["Q8_0", "Q4_0", "F16"])
@pytest.mark.parametrize("n_tok", [4, 6])
def test_gemv_one_hot_is_exact(orc, tname, n_tok):
    """x = e_j returns column j of W' exactly (one non-zero term), on the
    VALU kernel (4 tokens over 1000 rows) and the matrix cores (6)."""
    M, K = 1000, 2048
    _banner(f"gemv one-hot {tname} N={n_tok}")
    w = WL.weights(11, M, K)
    packed = _oracle_weight(orc, tname, w)
    deq = orc.dequantize(TYPES[tname][1], packed, K)
    js = [0, 31, 1000, 2047, 32, 1999][:n_tok]
    x = np.zeros((len(js), K), np.float32)
    for n, j in enumerate(js):
        x[n, j] = 1.0
    y = Q.gemv(_gpu_weight(tname, w), torch.from_numpy(x).to(DEV)).cpu().numpy()
    for n, j in enumerate(js):
        assert np.array_equal(y[n], deq[:, j])


def test_gemv_batch_columns_match_single_token(orc):
    """Column n of an N-token GEMV equals the one-token GEMV of x_n (within the bar)."""
    M, K = 3000, 2048
    _banner("gemv batch consistency")
    w = WL.weights(12, M, K)
    x = WL.activations(13, 8, K)
    wt = _gpu_weight("Q8_0", w)
    yb = Q.gemv(wt, torch.from_numpy(x).to(DEV)).cpu().numpy()
    packed = orc.quantize(orc.Q8_0, w)
    for n in (0, 3, 7):
        y1 = Q.gemv(wt, torch.from_numpy(x[n:n + 1]).to(DEV)).cpu().numpy()
        _, a = orc.mul_mat(orc.Q8_0, packed, K, x[n:n + 1])
        assert np.all(np.abs(yb[n] - y1[0]) <= 2e-4 * a[0] + 2e-6)


def test_gemv_row_view(orc):
    """A row-range view of W gives the matching slice of the full result."""
    M, K = 2000, 2048
    _banner("gemv row view")
    w = WL.weights(14, M, K)
    x = WL.activations(15, 1, K)
    wt = _gpu_weight("Q4_0", w)
    packed = orc.quantize(orc.Q4_0, w)
    yref, a = orc.mul_mat(orc.Q4_0, packed, K, x)
    xs = torch.from_numpy(x).to(DEV)
    for r0, r1 in ((0, 1), (17, 530), (1999, 2000), (1024, 2000)):
        y = Q.gemv(wt.rows(r0, r1), xs).cpu().numpy()
        _assert_tol(y, yref[:, r0:r1], a[:, r0:r1], 1e-4, 1e-6, f"rows {r0}:{r1}")


def test_gemv_zero_k_and_empty(orc):
    _banner("gemv K=0 and empty operands")
    wt = B.Weight(torch.zeros((5, 16), dtype=torch.uint8, device=DEV), B.Q4_0, 0, 5)
    y = torch.full((2, 5), 7.0, device=DEV)
    Q.gemv(wt, torch.zeros((2, 0), device=DEV), out=y)
    assert not y.cpu().numpy().any()
    wt0 = B.Weight(torch.zeros((0, 1152), dtype=torch.uint8, device=DEV), B.Q4_0, 2048, 0)
    y0 = Q.gemv(wt0, torch.ones((1, 2048), device=DEV))
    assert y0.shape == (1, 0)


def test_gemv_rejects_on_device():
    """Host validation with real device memory: overlap and N range."""
    _banner("gemv validation with device buffers")
    w = Q.quantize(torch.randn(64, 2048, device=DEV) * 0.02, B.Q4_0)
    x = torch.randn(1, 2048, device=DEV)
    with pytest.raises(Q.QmmError) as e:
        Q.gemv(w, x, out=w.data.view(torch.float32)[:1, :64])
    assert e.value.status == B.ERR_ALIAS
    with pytest.raises(Q.QmmError) as e:
        Q.gemv(w, torch.randn(9, 2048, device=DEV))
    assert e.value.status == B.ERR_SHAPE


# ---------------------------------------------------------------- GEMM

GEMM_CASES = [
    # (type, M, K, N)
    ("Q4_0", 1, 32, 1), ("Q4_0", 130, 96, 7), ("Q4_0", 128, 64, 128), ("Q4_0", 257, 2048, 129),
    ("Q4_0", 200, 5632, 300), ("Q4_0", 64, 2048 + 32, 64), ("Q8_0", 130, 2048, 65),
    ("Q8_0", 33, 96, 257),
    ("F16", 130, 2048, 65), ("F16", 33, 96, 257), ("F16", 200, 2048 + 32, 300), ("F16", 1, 32, 1),
    ("Q4_B64", 257, 2048, 129), ("Q4_B64", 130, 64, 7), ("Q8_B64", 200, 5632, 300), ("Q8_B64", 33, 192, 65),
]


def _gemm_inputs(orc, tname, M, K, N, seed):
    w = WL.weights(seed, M, K)
    xbits = WL.round_bf16_bits(WL.activations(seed + 1, N, K))
    packed = _oracle_weight(orc, tname, w)
    if tname == "F16":
        wt = B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
    else:
        wt = B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)
    return packed, xbits, wt


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemm_parity(orc, case):
    tname, M, K, N = case
    _banner(f"gemm {tname} M={M} K={K} N={N}")
    packed, xbits, wt = _gemm_inputs(orc, tname, M, K, N, seed=M + K + N)
    yref, a = orc.mul_mat(TYPES[tname][1], packed, K, xbits, x_bf16_bits=True)
    ydiag, _ = orc.mul_mat(TYPES[tname][1], packed, K, xbits, x_bf16_bits=True, w_to_bf16=True)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    # with the split-K workspace the shapes call for (most of these shapes
    # leave compute units idle, so K is split), and without one
    for ws in ("auto", None):
        buf, yv = _guarded_out(N, M)
        Q.gemm(wt, xt, out=yv, workspace=ws)
        torch.cuda.synchronize()
        _check_guard(buf)
        y = yv.cpu().numpy()
        _assert_tol(y, yref, a, 1e-2, 1e-5, f"gemm {case} workspace={ws}")
        _assert_tol(y, ydiag, a, 1.1 * K * 2.0 ** -24, 1e-7, f"gemm bf16-weight diagnostic {case} workspace={ws}")


@pytest.mark.parametrize("tname", ["Q4_0", "Q8_0", "F16"])
def test_gemm_strided_operands(orc, tname):
    """Padded weight pitch (padding filled with 0xFF bytes, which as scales or
    codes would poison the result if read), x rows with a larger pitch, y rows
    with a larger pitch; K/32 odd so the last K-step is half empty."""
    M, K, N = 150, 2048 + 32, 140
    _banner(f"gemm strided {tname}")
    w = WL.weights(31, M, K)
    xbits = WL.round_bf16_bits(WL.activations(32, N, K))
    packed = _oracle_weight(orc, tname, w)
    yref, a = orc.mul_mat(TYPES[tname][1], packed, K, xbits, x_bf16_bits=True)
    rs = packed.shape[1]
    padded = np.full((M, rs + 80), 0xFF, np.uint8)      # F16: 0xFFFF halves are NaN
    padded[:, :rs] = packed
    if tname == "F16":
        wt = B.Weight(torch.from_numpy(padded.view(np.float16)).to(DEV), B.F16, K, M)
    else:
        wt = B.Weight(torch.from_numpy(padded).to(DEV), TYPES[tname][0], K, M)
    xfull = torch.full((N, K + 24), -3.0e38, dtype=torch.bfloat16, device=DEV)
    xfull[:, :K] = WL.bf16_bits_to_torch(xbits, DEV)
    buf, yv = _guarded_out(N, M, pad_cols=5)
    Q.gemm(wt, xfull[:, :K], out=yv)
    torch.cuda.synchronize()
    _check_guard(buf, pad_cols=5)
    _assert_tol(yv.cpu().numpy(), yref, a, 1e-2, 1e-5, f"gemm strided {tname}")


def test_gemm_prefill_full_size_sampled(orc):
    """The 5632 x 2048 Q4_0 weight times 512 bf16 tokens, checked on 4096
    sampled outputs plus every output of the first and last 128 x 128 tiles."""
    M, K, N = WL.FFN, WL.HIDDEN, 512
    _banner("gemm prefill 5632x2048x512")
    w = WL.weights(WL.seed(5, 0), M, K)
    xbits = WL.round_bf16_bits(WL.activations(WL.seed(5, 1), N, K))
    wt = Q.quantize(torch.from_numpy(w).to(DEV), B.Q4_0)
    packed = orc.quantize(orc.Q4_0, w)
    assert np.array_equal(wt.data.cpu().numpy(), packed)
    y = Q.gemm(wt, WL.bf16_bits_to_torch(xbits, DEV)).cpu().numpy()
    rng = np.random.default_rng(99)
    ms = list(rng.integers(0, M, 4096))
    ns = list(rng.integers(0, N, 4096))
    for m0, n0 in ((0, 0), (M - 128, N - 128)):
        mm, nn = np.meshgrid(np.arange(m0, m0 + 128), np.arange(n0, n0 + 128))
        ms += list(mm.ravel())
        ns += list(nn.ravel())
    ms, ns = np.array(ms), np.array(ns)
    yref, a = orc.mul_mat_pairs(orc.Q4_0, packed, K, xbits, ms, ns, x_bf16_bits=True)
    ydiag, _ = orc.mul_mat_pairs(orc.Q4_0, packed, K, xbits, ms, ns, x_bf16_bits=True,
                                 w_to_bf16=True)
    _assert_tol(y[ns, ms], yref, a, 1e-2, 1e-5, "prefill sampled")
    _assert_tol(y[ns, ms], ydiag, a, 1.1 * K * 2.0 ** -24, 1e-7, "prefill sampled diagnostic")


def test_gemm_prefill_f16_full_size_sampled(orc):
    """The same product with the weights in fp16 (converted to bf16 in the
    multiplying waves, one K-step per staged group), in the launch the bench
    times: 4096 sampled outputs plus the first and last 128 x 128 tiles."""
    M, K, N = WL.FFN, WL.HIDDEN, 512
    _banner("gemm prefill F16 5632x2048x512")
    packed = _oracle_weight(orc, "F16", WL.weights(WL.seed(5, 0), M, K))
    xbits = WL.round_bf16_bits(WL.activations(WL.seed(5, 1), N, K))
    wt = B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
    y = Q.gemm(wt, WL.bf16_bits_to_torch(xbits, DEV)).cpu().numpy()
    rng = np.random.default_rng(101)
    ms = list(rng.integers(0, M, 4096))
    ns = list(rng.integers(0, N, 4096))
    for m0, n0 in ((0, 0), (M - 128, N - 128)):
        mm, nn = np.meshgrid(np.arange(m0, m0 + 128), np.arange(n0, n0 + 128))
        ms += list(mm.ravel())
        ns += list(nn.ravel())
    ms, ns = np.array(ms), np.array(ns)
    t = TYPES["F16"][1]
    yref, a = orc.mul_mat_pairs(t, packed, K, xbits, ms, ns, x_bf16_bits=True)
    ydiag, _ = orc.mul_mat_pairs(t, packed, K, xbits, ms, ns, x_bf16_bits=True, w_to_bf16=True)
    _assert_tol(y[ns, ms], yref, a, 1e-2, 1e-5, "prefill F16 sampled")
    _assert_tol(y[ns, ms], ydiag, a, 1.1 * K * 2.0 ** -24, 1e-7, "prefill F16 sampled diagnostic")


def test_gemm_split_k_full_size_sampled(orc):
    """The 2048 x 5632 down projection times 512 bf16 tokens: 64 output
    tiles, so K is split over four workspace slabs and the slabs added by the
    second kernel; checked on 4096 sampled outputs plus every output of the
    first and last 128 x 128 tiles."""
    M, K, N = WL.HIDDEN, WL.FFN, 512
    _banner("gemm split-K 2048x5632x512")
    w = WL.weights(WL.seed(5, 2), M, K)
    xbits = WL.round_bf16_bits(WL.activations(WL.seed(5, 3), N, K))
    packed = orc.quantize(orc.Q4_0, w)
    wt = B.Weight(torch.from_numpy(packed).to(DEV), B.Q4_0, K, M)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    assert Q.gemm_workspace_size(wt, xt) == 4 * N * M * 4
    y = Q.gemm(wt, xt).cpu().numpy()
    rng = np.random.default_rng(98)
    ms = list(rng.integers(0, M, 4096))
    ns = list(rng.integers(0, N, 4096))
    for m0, n0 in ((0, 0), (M - 128, N - 128)):
        mm, nn = np.meshgrid(np.arange(m0, m0 + 128), np.arange(n0, n0 + 128))
        ms += list(mm.ravel())
        ns += list(nn.ravel())
    ms, ns = np.array(ms), np.array(ns)
    yref, a = orc.mul_mat_pairs(orc.Q4_0, packed, K, xbits, ms, ns, x_bf16_bits=True)
    _assert_tol(y[ns, ms], yref, a, 1e-2, 1e-5, "split-K sampled")


def test_gemm_split_k_workspace_sizes(orc):
    """A workspace smaller than planned gives a smaller split (here two K
    ranges instead of four), a misaligned one is refused, and each split is
    deterministic: the same workspace size always gives the same bits."""
    M, K, N = 300, 4096, 100          # 3 tiles, 64 K-steps
    _banner("gemm split-K workspace sizes")
    packed, xbits, wt = _gemm_inputs(orc, "Q8_0", M, K, N, seed=23)
    yref, a = orc.mul_mat(orc.Q8_0, packed, K, xbits, x_bf16_bits=True)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    full = Q.gemm_workspace_size(wt, xt)
    slab = N * 300 * 4
    assert full == 8 * slab
    outs = {}
    for nbytes in (full, 4 * slab, 2 * slab + 16, slab, 0):
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)[:nbytes]
        y1 = Q.gemm(wt, xt, workspace=ws).cpu().numpy()
        y2 = Q.gemm(wt, xt, workspace=ws).cpu().numpy()
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), nbytes
        _assert_tol(y1, yref, a, 1e-2, 1e-5, f"split-K workspace {nbytes} B")
        outs[nbytes] = y1
    # a workspace of one slab cannot hold a split: the same bits as no workspace
    assert np.array_equal(outs[slab].view(np.uint32), outs[0].view(np.uint32))
    bad = torch.empty(full + 64, dtype=torch.uint8, device=DEV)[4:4 + full]
    with pytest.raises(Q.QmmError) as e:
        Q.gemm(wt, xt, workspace=bad)
    assert e.value.status == B.ERR_LAYOUT
    big = torch.empty(full + slab, dtype=torch.uint8, device=DEV)
    yv = big[:slab].view(torch.float32).view(N, M)
    with pytest.raises(Q.QmmError) as e:     # the workspace overlaps y
        Q.gemm(wt, xt, out=yv, workspace=big)
    assert e.value.status == B.ERR_ALIAS


GEMM_SWIGLU_CASES = [
    ("Q4_0", 300, 640, 130), ("Q8_0", 65, 96, 7), ("F16", 130, 2048 + 32, 65),
    ("Q4_B64", 200, 1024, 129), ("Q8_B64", 64, 192, 300), ("Q4_0", 1, 32, 1),
]


def _gemm_swiglu_tol(orc, gref, ga, uref, ua, h):
    """The fused SwiGLU bound with each sum's GEMM bound (1e-2 * a + 1e-5)
    carried through Swish (|Swish'| <= 1.1) and the product, plus binary32
    rounding of the epilogue."""
    eg = 1e-2 * ga + 1e-5
    eu = 1e-2 * ua + 1e-5
    sg = np.array([orc.swish(v) for v in np.ravel(gref)]).reshape(np.shape(gref))
    return 1.1 * eg * (np.abs(uref) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(h)


@pytest.mark.parametrize("case", GEMM_SWIGLU_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemm_swiglu_parity(orc, case):
    """The fused gate/up prefill projection: h against Swish(g) * u of the
    oracle's sums, every output, guard bands intact."""
    tname, M, K, N = case
    _banner(f"gemm swiglu {tname} M={M} K={K} N={N}")
    seed = 3 * M + K + N
    pg = _oracle_weight(orc, tname, WL.weights(seed, M, K))
    pu = _oracle_weight(orc, tname, WL.weights(seed + 1, M, K))
    xbits = WL.round_bf16_bits(WL.activations(seed + 2, N, K))
    t = TYPES[tname][1]
    gref, ga = orc.mul_mat(t, pg, K, xbits, x_bf16_bits=True)
    uref, ua = orc.mul_mat(t, pu, K, xbits, x_bf16_bits=True)
    href = orc.swiglu(gref, uref)

    def wt(packed):
        if tname == "F16":
            return B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
        return B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)
    buf, hv = _guarded_out(N, M)
    Q.gemm_swiglu(wt(pg), wt(pu), WL.bf16_bits_to_torch(xbits, DEV), out=hv)
    torch.cuda.synchronize()
    _check_guard(buf)
    h = hv.cpu().numpy().astype(np.float64)
    tol = _gemm_swiglu_tol(orc, gref, ga, uref, ua, href)
    assert np.isfinite(h).all()
    err = np.abs(h - href)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


def test_gemm_swiglu_full_size_sampled(orc):
    """The TinyLLaMA gate/up pair (2 x 5632 x 2048, Q4_0) times 512 bf16
    tokens, on 2048 sampled outputs plus the first and last 64 x 128 tiles."""
    M, K, N = WL.FFN, WL.HIDDEN, 512
    _banner("gemm swiglu 5632x2048x512")
    wg_, wu_ = WL.weights(WL.seed(5, 0), M, K), WL.weights(WL.seed(5, 9), M, K)
    xbits = WL.round_bf16_bits(WL.activations(WL.seed(5, 1), N, K))
    pg, pu = orc.quantize(orc.Q4_0, wg_), orc.quantize(orc.Q4_0, wu_)
    h = Q.gemm_swiglu(B.Weight(torch.from_numpy(pg).to(DEV), B.Q4_0, K, M),
                      B.Weight(torch.from_numpy(pu).to(DEV), B.Q4_0, K, M),
                      WL.bf16_bits_to_torch(xbits, DEV)).cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(97)
    ms, ns = list(rng.integers(0, M, 2048)), list(rng.integers(0, N, 2048))
    for m0, n0 in ((0, 0), (M - 64, N - 128)):
        mm, nn = np.meshgrid(np.arange(m0, m0 + 64), np.arange(n0, n0 + 128))
        ms += list(mm.ravel())
        ns += list(nn.ravel())
    ms, ns = np.array(ms), np.array(ns)
    gref, ga = orc.mul_mat_pairs(orc.Q4_0, pg, K, xbits, ms, ns, x_bf16_bits=True)
    uref, ua = orc.mul_mat_pairs(orc.Q4_0, pu, K, xbits, ms, ns, x_bf16_bits=True)
    href = orc.swiglu(gref, uref)
    tol = _gemm_swiglu_tol(orc, gref, ga, uref, ua, href)
    err = np.abs(h[ns, ms] - href)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


def test_gemm_split_k_on_a_side_stream(orc):
    """K split with the binding's automatic workspace, enqueued on a stream
    other than torch's current one, several times in a row: the bits equal
    those of the same call on the current stream."""
    M, K, N = 256, 4096, 300
    _banner("gemm split-K on a side stream")
    packed, xbits, wt = _gemm_inputs(orc, "Q4_0", M, K, N, seed=25)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    assert Q.gemm_workspace_size(wt, xt) > 0
    ref = Q.gemm(wt, xt).cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty((N, M), device=DEV) for _ in range(4)]
    for o in outs:
        Q.gemm(wt, xt, out=o, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_gemm_deterministic_and_token_columns(orc):
    """Repeat calls are bitwise identical (with K split, each call with its
    own workspace, and without); without a split each token column equals
    the GEMM of that token alone (the kernel has no cross-token reduction)."""
    M, K, N = 700, 2048, 200
    _banner("gemm determinism")
    packed, xbits, wt = _gemm_inputs(orc, "Q4_0", M, K, N, seed=21)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    for ws in ("auto", None):
        y1 = Q.gemm(wt, xt, workspace=ws).cpu().numpy()
        y2 = Q.gemm(wt, xt, workspace=ws).cpu().numpy()
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), ws
    for n in (0, 129, 199):
        yn = Q.gemm(wt, xt[n:n + 1], workspace=None).cpu().numpy()
        assert np.array_equal(yn[0].view(np.uint32), y1[n].view(np.uint32))


GEMM_BATCH_CASES = [
    # (type, [M of each item], K, N): query/key/value-like shapes with an
    # empty item; gate/up-like; a single item; the most items
    ("Q4_0", [300, 40, 0, 40], 576, 200),
    ("Q8_0", [130, 130], 1024, 129),
    ("F16", [70, 33, 128], 2048 + 32, 65),
    ("Q4_B64", [257], 640, 7),
    ("Q8_B64", [17, 1, 130, 64, 5, 200, 2, 128], 192, 300),
]


@pytest.mark.parametrize("case", GEMM_BATCH_CASES, ids=lambda c: "%s-%s-k%d-n%d" % (c[0], "_".join(map(str, c[1])), c[2], c[3]))
def test_gemm_batch_parity(orc, case):
    """Every output of a batched launch against the oracle, and bit for bit
    equal to qmm_gemm of the same item without a K split."""
    tname, Ms, K, N = case
    _banner(f"gemm batch {tname} M={Ms} K={K} N={N}")
    shared = tname != "Q8_0"           # the Q8_0 case gives every item its own tokens
    xs = [WL.round_bf16_bits(WL.activations(77 + K + (0 if shared else i), N, K)) for i in range(len(Ms))]
    items, refs, xts = [], [], []
    for i, M in enumerate(Ms):
        xbits = xs[i]
        xt = WL.bf16_bits_to_torch(xbits, DEV)
        xts.append(xt)
        if M == 0:                      # an item with no rows owns no tiles
            code = TYPES[tname][0]
            items.append(B.Weight(torch.empty((0, B.row_size(code, K)), dtype=torch.uint8, device=DEV), code, K, 0))
            refs.append(None)
            continue
        w = WL.weights(700 + 10 * i + M, M, K)
        packed = _oracle_weight(orc, tname, w)
        if tname == "F16":
            wt = B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
        else:
            wt = B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)
        items.append(wt)
        refs.append(orc.mul_mat(TYPES[tname][1], packed, K, xbits, x_bf16_bits=True))
    outs = Q.gemm_batch([(wt, xt, None) for wt, xt in zip(items, xts)])
    torch.cuda.synchronize()
    for i, (wt, y, ref, xt) in enumerate(zip(items, outs, refs, xts)):
        assert tuple(y.shape) == (N, Ms[i])
        if not Ms[i]:
            continue
        yn = y.cpu().numpy()
        _assert_tol(yn, ref[0], ref[1], 1e-2, 1e-5, f"gemm batch {case} item {i}")
        alone = Q.gemm(wt, xt, workspace=None).cpu().numpy()
        assert np.array_equal(yn.view(np.uint32), alone.view(np.uint32)), f"item {i} differs from qmm_gemm"


# ---------------------------------------------------------------- GEMV batch

def test_gemv_batch_decoder_layer(orc):
    """The K = 2048 projections of a layer (Q, K, V, O, gate, up, each with its
    own input as the layer workload gives them) in one batched launch, and
    the down projection alone; every output checked against the oracle."""
    _banner("gemv batch: one decoder layer")
    xs = [WL.activations(WL.seed(3, 7 + s), 1, k) for s, k in enumerate(WL.LAYER_X_K)]
    xt = [torch.from_numpy(x).to(DEV) for x in xs]
    items, refs = [], []
    for t, (name, M, K, slot) in enumerate(WL.LAYER):
        w = WL.weights(WL.seed(3, t, 5), M, K)
        packed = orc.quantize(orc.Q4_0, w)
        refs.append(orc.mul_mat(orc.Q4_0, packed, K, xs[slot]))
        items.append((B.Weight(torch.from_numpy(packed).to(DEV), B.Q4_0, K, M), xt[slot], None))
    outs = Q.gemv_batch(items[:6]) + Q.gemv_batch(items[6:])
    for (name, *_), y, (yref, a) in zip(WL.LAYER, outs, refs):
        _assert_tol(y.cpu().numpy(), yref, a, 1e-4, 1e-6, f"batch {name}")


@pytest.mark.parametrize("tname,K", [("Q8_0", 2048), ("Q4_0", 2048), ("F16", 2048), ("Q4_0", 5632), ("Q8_0", 5632),
                                     ("F16", 4096), ("F16", 5632)])
def test_gemv_batch_ragged_items(orc, tname, K):
    """Items of 1, 0, 300 and 4100 rows sharing one x, N = 5, outputs in
    guard-banded buffers; quantized K = 5632 takes the one-launch
    matrix-core kernel with several items, F16 K = 4096 its 8-row tiles and
    F16 K = 5632 two passes of different tile heights."""
    N = 5
    _banner(f"gemv batch ragged {tname} K={K}")
    x = WL.activations(31, N, K)
    xt = torch.from_numpy(x).to(DEV)
    items, refs, bufs = [], [], []
    for i, M in enumerate((1, 0, 300, 4100)):
        w = WL.weights(40 + i, M, K)
        packed = _oracle_weight(orc, tname, w)
        refs.append(orc.mul_mat(TYPES[tname][1], packed, K, x) if M else None)
        buf, yv = _guarded_out(N, M)
        bufs.append(buf)
        items.append((_gpu_weight(tname, w), xt, yv))
    outs = Q.gemv_batch(items)
    torch.cuda.synchronize()
    for buf in bufs:
        _check_guard(buf)
    for y, ref in zip(outs, refs):
        if ref is not None:
            _assert_tol(y.cpu().numpy(), ref[0], ref[1], 1e-4, 1e-6, f"ragged {tname}")


def test_gemv_batch_matches_single_calls(orc):
    """A batch of eight equals eight single calls within the bar (same kernel,
    possibly a different share of the grid)."""
    K = 2048
    _banner("gemv batch of eight vs single calls")
    items, singles = [], []
    for i in range(8):
        w = WL.weights(60 + i, 256 + 100 * i, K)
        x = torch.from_numpy(WL.activations(70 + i, 2, K)).to(DEV)
        wt = _gpu_weight("Q4_0", w)
        items.append((wt, x, None))
        singles.append(Q.gemv(wt, x).cpu().numpy())
    outs = Q.gemv_batch(items)
    for i, (y, y1) in enumerate(zip(outs, singles)):
        w = WL.weights(60 + i, 256 + 100 * i, K)
        _, a = orc.mul_mat(orc.Q4_0, orc.quantize(orc.Q4_0, w), K, WL.activations(70 + i, 2, K))
        assert np.all(np.abs(y.cpu().numpy() - y1) <= 2e-4 * a + 2e-6)


# ------------------------------------------------------------ block records

RECORD_SHAPES = [(1, 32), (7, 96), (300, 2048), (129, 5632), (3, 8192 + 32)]


@pytest.mark.parametrize("tname", ["Q4_0", "Q8_0"])
@pytest.mark.parametrize("shape", RECORD_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_records_bit_exact(orc, tname, shape):
    """Rows -> records and records -> rows against the oracle, byte for byte;
    bytes past the row size up to the pitch are left untouched."""
    M, K = shape
    _banner(f"records {tname} {M}x{K}")
    ot = TYPES[tname][1]
    rows = orc.quantize(ot, _adversarial(M, K, 300 + M + K))
    ref_rec = orc.rows_to_records(ot, rows, K)
    rs = rows.shape[1]
    # rows -> records
    wt = B.Weight(torch.from_numpy(rows).to(DEV), TYPES[tname][0], K, M)
    rec = Q.rows_to_records(wt).cpu().numpy()
    assert np.array_equal(rec, ref_rec)
    # records -> rows, into a padded pitch prefilled with a marker
    pitch = rs + 48
    buf = torch.full((M, pitch), 0xAB, dtype=torch.uint8, device=DEV)
    dst = B.Weight(buf, TYPES[tname][0], K, M)
    d = dst.desc()
    st = B.lib().qmm_records_to_rows(ctypes.c_void_p(torch.from_numpy(ref_rec).to(DEV).data_ptr()),
                                     ctypes.byref(d), None)
    torch.cuda.synchronize()
    assert st == B.OK
    got = buf.cpu().numpy()
    assert np.array_equal(got[:, :rs], rows)
    assert (got[:, rs:] == 0xAB).all()


def test_records_feed_the_gemv(orc):
    """Weights imported from records give the same GEMV bits as the same
    weights quantized in place (the LM head shape, Q8_0)."""
    _banner("records -> rows -> gemv, LM head")
    w = WL.weights(WL.seed(4, 0), WL.VOCAB, WL.HIDDEN)
    x = torch.from_numpy(WL.activations(WL.seed(4, 1), 2, WL.HIDDEN)).to(DEV)
    q = Q.quantize(torch.from_numpy(w).to(DEV), B.Q8_0)
    rec = Q.rows_to_records(q)
    assert rec.numel() == WL.VOCAB * WL.HIDDEN // 32 * 34
    back = Q.records_to_rows(rec, B.Q8_0, WL.HIDDEN, WL.VOCAB)
    assert torch.equal(back.data, q.data)
    y1 = Q.gemv(q, x)
    y2 = Q.gemv(back, x)
    assert torch.equal(y1, y2)


# ------------------------------------------------- integer activations (Q8_0 x)

I8_CASES = [
    ("Q4_0", 2048, 2048, 1), ("Q4_0", 5632, 2048, 1), ("Q4_0", 2048, 5632, 1),
    ("Q8_0", 32000, 2048, 8), ("Q8_0", 32000, 2048, 1), ("Q4_0", 300, 1024, 3),
    ("Q8_0", 37, 96, 5), ("Q4_0", 1, 32, 1), ("Q8_0", 513, 512, 2), ("Q4_0", 64, 16384, 2),
    ("Q4_0", 130, 8192, 8),
    # Q8_0 weights from 5 tokens over 8192 rows or K over 4096 take the
    # matrix-core kernel (one twelve-wave launch up to K = 6144, passes
    # beyond); the rest stays on the int8 dot-product kernel
    ("Q8_0", 129, 5632, 6), ("Q8_0", 77, 16384, 7), ("Q8_0", 8200, 1024, 5), ("Q8_0", 2048, 2048, 8),
    ("Q4_0", 2048, 5632, 8), ("Q4_0", 2600, 2048, 4), ("Q4_0", 45, 6144, 5),
    # 64-block weights: each 32-block term takes its 64-block's scale
    ("Q4_B64", 5632, 2048, 1), ("Q8_B64", 300, 5632, 3), ("Q4_B64", 37, 128, 8), ("Q8_B64", 513, 512, 2),
    ("Q4_B64", 64, 4160, 8), ("Q8_B64", 100, 5632, 8), ("Q8_B64", 8200, 2048, 5),
]


@pytest.mark.parametrize("case", I8_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_q8_activations(orc, case):
    """The integer-activation GEMV against the oracle's integer path: x is
    quantized on the GPU (bit-exact with the oracle), then y must agree
    within the binary32 summation bound of its block terms."""
    tname, M, K, N = case
    _banner(f"gemv q8 activations {tname} M={M} K={K} N={N}")
    seed = 13 * M + K + N
    w = WL.weights(seed, M, K)
    x = WL.activations(seed + 1, N, K)
    packed = orc.quantize(TYPES[tname][1], w)
    xq_ref = orc.quantize(orc.Q8_0, x)
    wt = B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)
    xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
    assert np.array_equal(xq.data.cpu().numpy(), xq_ref)
    yref, _ = orc.mul_mat_q8act(TYPES[tname][1], packed, K, xq_ref)
    _, a_exact = orc.mul_mat(TYPES[tname][1], packed, K, orc.dequantize(orc.Q8_0, xq_ref, K))
    y = Q.gemv(wt, xq).cpu().numpy().astype(np.float64)
    nchunk = K // 32 if tname.startswith("Q4") else K // 16
    tol = (nchunk + 16) * 2.0 ** -24 * a_exact + 1e-30
    err = np.abs(y - yref)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


I8_BATCH_CASES = [
    # (type, [M of each item], K, N, shared x): a layer's [Wq Wk Wv] on one
    # token; items with their own activations and an empty item; 64-blocks
    ("Q4_0", [2048, 256, 256], 2048, 1, True),
    ("Q8_0", [300, 0, 130, 37], 1024, 5, False),
    ("Q4_B64", [5632, 5632], 2048, 2, True),
    ("Q8_0", [64] * 8, 512, 8, False),
    ("Q4_0", [2048, 300], 5632, 8, False),
    ("Q8_0", [4100, 4100, 17], 2048, 6, False),
]


@pytest.mark.parametrize("case", I8_BATCH_CASES, ids=lambda c: "%s-%s-k%d-n%d" % (c[0], "_".join(map(str, c[1])), c[2], c[3]))
def test_gemv_batch_q8_activations(orc, case):
    """qmm_gemv_batch with Q8_0 activations: every item against the
    oracle's integer path within the bound of qmm_gemv's integer path."""
    tname, Ms, K, N, shared = case
    _banner(f"gemv batch q8 activations {tname} M={Ms} K={K} N={N}")
    code = TYPES[tname][0]
    items, checks = [], []
    xs_shared = WL.activations(900 + K, N, K)
    for i, M in enumerate(Ms):
        x = xs_shared if shared else WL.activations(910 + i, N, K)
        xq_ref = orc.quantize(orc.Q8_0, x)
        xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
        assert np.array_equal(xq.data.cpu().numpy(), xq_ref)
        if M == 0:
            wt = B.Weight(torch.empty((0, B.row_size(code, K)), dtype=torch.uint8, device=DEV), code, K, 0)
            items.append((wt, xq, None))
            checks.append(None)
            continue
        w = WL.weights(920 + 7 * i + M, M, K)
        packed = orc.quantize(TYPES[tname][1], w)
        items.append((B.Weight(torch.from_numpy(packed).to(DEV), code, K, M), xq, None))
        yref, _ = orc.mul_mat_q8act(TYPES[tname][1], packed, K, xq_ref)
        _, a_exact = orc.mul_mat(TYPES[tname][1], packed, K, orc.dequantize(orc.Q8_0, xq_ref, K))
        checks.append((yref, a_exact))
    outs = Q.gemv_batch(items)
    nchunk = K // 32 if tname.startswith("Q4") else K // 16
    for i, (y, chk) in enumerate(zip(outs, checks)):
        assert tuple(y.shape) == (N, Ms[i])
        if chk is None:
            continue
        err = np.abs(y.cpu().numpy().astype(np.float64) - chk[0])
        tol = (nchunk + 16) * 2.0 ** -24 * chk[1] + 1e-30
        assert (err <= tol).all(), f"item {i}: worst err/tol {(err / tol).max():.3g}"
    # a batch mixing fp32 and Q8_0 activations is refused
    w0 = items[0][0]
    with pytest.raises(Q.QmmError) as e:
        Q.gemv_batch([(w0, items[0][1], None), (w0, torch.zeros((N, K), device=DEV), None)])
    assert e.value.status == B.ERR_TYPE


I8_SWIGLU_CASES = [
    ("Q4_0", 5632, 2048, 1),       # the TinyLLaMA feed-forward gate/up pair
    ("Q4_0", 37, 96, 3), ("Q8_0", 513, 512, 8), ("Q8_0", 64, 4096, 5), ("Q4_0", 300, 5632, 2),
    ("Q4_B64", 300, 2048, 2), ("Q8_B64", 65, 192, 1),
]


@pytest.mark.parametrize("case", I8_SWIGLU_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_swiglu_q8_activations(orc, case):
    """The fused gate/up SwiGLU with Q8_0 activations: h against Swish(g) * u
    of the oracle's integer-path sums, within the bound of the fused GEMV
    with each sum's bound that of the integer path."""
    tname, M, K, N = case
    _banner(f"gemv swiglu q8 activations {tname} M={M} K={K} N={N}")
    seed = 5 * M + K + N
    wg, wu = WL.weights(seed, M, K), WL.weights(seed + 1, M, K)
    x = WL.activations(seed + 2, N, K)
    t = TYPES[tname][1]
    pg, pu = orc.quantize(t, wg), orc.quantize(t, wu)
    xq_ref = orc.quantize(orc.Q8_0, x)
    xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
    assert np.array_equal(xq.data.cpu().numpy(), xq_ref)
    gref, _ = orc.mul_mat_q8act(t, pg, K, xq_ref)
    uref, _ = orc.mul_mat_q8act(t, pu, K, xq_ref)
    xd = orc.dequantize(orc.Q8_0, xq_ref, K)
    _, ga = orc.mul_mat(t, pg, K, xd)
    _, ua = orc.mul_mat(t, pu, K, xd)
    href = orc.swiglu(gref, uref)
    code = TYPES[tname][0]
    h = Q.gemv_swiglu(B.Weight(torch.from_numpy(pg).to(DEV), code, K, M),
                      B.Weight(torch.from_numpy(pu).to(DEV), code, K, M), xq)
    h = h.cpu().numpy().astype(np.float64)
    nchunk = K // 32 if tname.startswith("Q4") else K // 16
    eg = (nchunk + 16) * 2.0 ** -24 * ga + 1e-30
    eu = (nchunk + 16) * 2.0 ** -24 * ua + 1e-30
    sg = np.array([orc.swish(v) for v in gref.ravel()]).reshape(gref.shape)
    tol = 1.1 * eg * (np.abs(uref) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(href)
    assert np.isfinite(h).all()
    err = np.abs(h - href)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


def test_gemv_q8_activations_zero_and_strided(orc):
    """Zero activation blocks (scale 0) and padded pitches on both operands."""
    M, K, N = 90, 2048, 4
    _banner("gemv q8 activations zero blocks, strided")
    w = WL.weights(61, M, K)
    x = WL.activations(62, N, K)
    x[1, 64:512] = 0.0
    x[3] = 0.0
    packed = orc.quantize(orc.Q4_0, w)
    rs = packed.shape[1]
    padded = np.full((M, rs + 32), 0xFF, np.uint8)
    padded[:, :rs] = packed
    wt = B.Weight(torch.from_numpy(padded).to(DEV), B.Q4_0, K, M)
    xq_ref = orc.quantize(orc.Q8_0, x)
    xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0, pitch=B.row_size(B.Q8_0, K) + 64)
    yref, _ = orc.mul_mat_q8act(orc.Q4_0, packed, K, xq_ref)
    _, a_exact = orc.mul_mat(orc.Q4_0, packed, K, orc.dequantize(orc.Q8_0, xq_ref, K))
    y = Q.gemv(wt, xq).cpu().numpy().astype(np.float64)
    assert (y[3] == 0).all()
    assert (np.abs(y - yref) <= (K // 32 + 16) * 2.0 ** -24 * a_exact + 1e-30).all()
