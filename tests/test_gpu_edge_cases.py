"""GPU parity on the method's edge cases, through every MUL_MAT path.

The weights are quantized from blocks that reach the corners of the block
rule ("Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++",
§6.1; "A Complete Guide to llama.cpp and Customization with C++", §2.2):
zero blocks (scale 0), blocks whose fp16 scale is subnormal, exact rounding
ties, clamped codes, blocks scaled by 1000, and blocks holding one large
weight among zeros (every block of every third row).  The activations have
mean 5 (or -5), are 0.01 exactly where those lone weights sit, and one token
holds exact zeros.  For such rows the result is a small sum next to large
activations: any path that multiplies codes offset from their signed value
and subtracts the offset afterwards loses the result to cancellation, while
the pages' flow (unpack to the signed code, scale, multiply-add) keeps the
bound.

Bars (the same as the Gaussian parity tests), per output, against the
oracle's binary64 MUL_MAT on the same arrays:
  * fp32 activations: |y - y_ref| <= 1e-4 * a + 1e-6;
  * bf16 GEMM: <= 1e-2 * a + 1e-5, and the binary32 summation bound
    1.1 * K * 2^-24 * a + 1e-7 against the oracle's bf16-weight variant;
  * Q8_0 activations: (chunks + 16) * 2^-24 * a against the oracle's
    integer path;
  * SwiGLU: each sum's bound carried through Swish and the product.
Paths: the VALU GEMV (1-4 tokens), the matrix-core GEMV (3-4 tokens over
8192 rows, 5-8 tokens, K over 4096 in passes), the integer-activation GEMV,
the fused SwiGLU GEMVs, batched GEMVs, the GEMM with and without a K split,
batched GEMMs and the fused SwiGLU GEMM.
"""
import numpy as np
import pytest
import torch

import quantized_matmul_ggml_amd as Q
from quantized_matmul_ggml_amd import binding as B
from quantized_matmul_ggml_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TYPES = {"Q8_0": (B.Q8_0, 3), "Q4_0": (B.Q4_0, 4), "F16": (B.F16, 1),
         "Q8_B64": (B.Q8_B64, 5), "Q4_B64": (B.Q4_B64, 6)}


def _banner(msg):
    print(f"[case] {msg}", flush=True)


def _assert_tol(y, yref, a, rel, abs_, what):
    y = np.asarray(y, np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y - yref)
    ratio = err / (rel * a + abs_)
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{what}: worst |err|/bound = {ratio.max():.3g} at {worst}, "
                                f"y={y[worst]!r} ref={yref[worst]!r} a={a[worst]!r}")


def _inputs(seed, M, K, N, mean=5.0):
    return WL.outlier_weights(seed, M, K), WL.shifted_activations(seed + 7, N, K, outlier_seed=seed, mean=mean)


def _packed(orc, tname, w):
    if tname == "F16":
        return WL.round_f16(w).view(np.uint8).reshape(w.shape[0], 2 * w.shape[1])
    return orc.quantize(TYPES[tname][1], w)


def _weight(tname, packed, K, M):
    if tname == "F16":
        return B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
    return B.Weight(torch.from_numpy(packed).to(DEV), TYPES[tname][0], K, M)


def _swiglu_tol(orc, gref, eg, uref, eu, href):
    sg = np.array([orc.swish(v) for v in np.ravel(gref)]).reshape(np.shape(gref))
    return 1.1 * eg * (np.abs(uref) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(href)


# ------------------------------------------------------------ fp32 GEMV

GEMV_EDGE = [
    # (type, M, K, N, mean): the VALU kernel (1 and 2 tokens; 3-4 tokens
    # up to 2048 rows of at most 4096), one and several waves per row
    ("Q4_0", 300, 2048, 1, 5.0), ("Q4_0", 257, 5632, 1, 5.0), ("Q4_0", 130, 2048, 2, -5.0),
    ("Q4_0", 99, 32768, 1, 5.0), ("Q4_0", 100, 2048, 3, 5.0),
    ("Q8_0", 300, 2048, 1, 5.0), ("Q8_0", 129, 5632, 2, 5.0), ("Q8_0", 77, 1024, 4, -5.0),
    ("Q8_0", 512, 512, 1, 5.0),
    ("F16", 300, 2048, 1, 5.0), ("F16", 65, 1024, 2, 5.0),
    ("Q4_B64", 300, 2048, 1, 5.0), ("Q8_B64", 130, 2048, 2, 5.0),
    # the matrix-core kernel: 3-4 tokens over 2048 rows, 5-8 tokens, K of
    # 129..192 blocks in one launch (from 3 tokens), longer K in passes that
    # add to y (7-8 tokens)
    ("Q4_0", 8200, 2048, 4, 5.0), ("Q8_0", 8195, 1024, 3, 5.0), ("Q4_0", 2600, 2048, 3, -5.0),
    ("Q4_0", 300, 2048, 5, 5.0), ("Q8_0", 300, 2048, 8, -5.0), ("Q4_0", 257, 160, 6, 5.0),
    ("Q4_0", 300, 5632, 6, 5.0), ("Q4_0", 2048, 5632, 3, 5.0), ("Q8_0", 129, 5632, 5, 5.0),
    ("Q8_0", 77, 16384, 7, 5.0), ("Q8_0", 31, 2080, 7, 5.0),
    ("Q4_B64", 64, 4096, 7, 5.0), ("Q8_B64", 8200, 2048, 4, 5.0), ("Q8_B64", 100, 5632, 8, -5.0),
    # F16 rows on the matrix cores (one, two and three passes over K) and
    # on the VALU kernel's four-wave rows
    ("F16", 300, 2048, 6, 5.0), ("F16", 129, 5632, 8, 5.0), ("F16", 40, 8224, 3, -5.0),
    ("F16", 2100, 1024, 3, -5.0), ("F16", 500, 4096, 2, 5.0),
]


@pytest.mark.parametrize("case", GEMV_EDGE, ids=lambda c: "%s-%dx%d-n%d-mean%+g" % c)
def test_gemv_edge_cases(orc, case):
    tname, M, K, N, mean = case
    _banner(f"gemv edge {tname} M={M} K={K} N={N} mean={mean}")
    w, x = _inputs(1000 + M + K + N, M, K, N, mean)
    packed = _packed(orc, tname, w)
    yref, a = orc.mul_mat(TYPES[tname][1], packed, K, x)
    y = Q.gemv(_weight(tname, packed, K, M), torch.from_numpy(x).to(DEV)).cpu().numpy()
    _assert_tol(y, yref, a, 1e-4, 1e-6, f"gemv edge {case}")


@pytest.mark.parametrize("N", [1, 5])
def test_gemv_batch_edge_cases(orc, N):
    """qmm_gemv_batch over edge-case items with their own activations: the
    VALU kernel at one token, the matrix-core kernel at five."""
    K = 2048
    _banner(f"gemv batch edge N={N}")
    items, refs = [], []
    for i, (tname, M) in enumerate((("Q4_0", 2048), ("Q4_0", 256), ("Q4_0", 5632))):
        w, x = _inputs(2000 + 10 * i + N, M, K, N)
        packed = _packed(orc, tname, w)
        refs.append(orc.mul_mat(TYPES[tname][1], packed, K, x))
        items.append((_weight(tname, packed, K, M), torch.from_numpy(x).to(DEV), None))
    outs = Q.gemv_batch(items)
    for i, (y, (yref, a)) in enumerate(zip(outs, refs)):
        _assert_tol(y.cpu().numpy(), yref, a, 1e-4, 1e-6, f"gemv batch edge item {i}")


SWIGLU_EDGE = [("Q4_0", 5632, 2048, 1), ("Q4_0", 300, 1024, 3), ("Q8_0", 513, 512, 2),
               ("Q8_0", 64, 4096, 8), ("F16", 130, 1024, 1), ("Q4_B64", 300, 2048, 2),
               ("Q4_0", 5632, 2048, 8), ("Q4_B64", 130, 2048, 5)]


@pytest.mark.parametrize("case", SWIGLU_EDGE, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_swiglu_edge_cases(orc, case):
    tname, M, K, N = case
    _banner(f"gemv swiglu edge {tname} M={M} K={K} N={N}")
    seed = 3000 + M + K + N
    wg, x = _inputs(seed, M, K, N)
    wu = WL.outlier_weights(seed + 50, M, K)
    pg, pu = _packed(orc, tname, wg), _packed(orc, tname, wu)
    t = TYPES[tname][1]
    gref, ga = orc.mul_mat(t, pg, K, x)
    uref, ua = orc.mul_mat(t, pu, K, x)
    href = orc.swiglu(gref, uref)
    h = Q.gemv_swiglu(_weight(tname, pg, K, M), _weight(tname, pu, K, M),
                      torch.from_numpy(x).to(DEV)).cpu().numpy().astype(np.float64)
    tol = _swiglu_tol(orc, gref, 1e-4 * ga + 1e-6, uref, 1e-4 * ua + 1e-6, href)
    assert np.isfinite(h).all()
    err = np.abs(h - href)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


# ------------------------------------------------- integer activations (Q8_0 x)

I8_EDGE = [("Q4_0", 300, 2048, 1), ("Q4_0", 2048, 5632, 2), ("Q8_0", 1000, 2048, 8),
           ("Q8_0", 77, 1024, 3), ("Q4_B64", 130, 2048, 4),
           # the matrix-core kernel: K = 2048, one launch at K = 5632, passes
           ("Q4_0", 300, 2048, 6), ("Q4_0", 2048, 5632, 8), ("Q8_0", 129, 5632, 5), ("Q4_0", 64, 8192, 7)]


def _i8_bound(K, tname, a):
    nchunk = K // 32 if tname.startswith("Q4") else K // 16
    return (nchunk + 16) * 2.0 ** -24 * a + 1e-30


@pytest.mark.parametrize("case", I8_EDGE, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemv_q8_activations_edge_cases(orc, case):
    tname, M, K, N = case
    _banner(f"gemv q8 activations edge {tname} M={M} K={K} N={N}")
    w, x = _inputs(4000 + M + K + N, M, K, N)
    packed = orc.quantize(TYPES[tname][1], w)
    xq_ref = orc.quantize(orc.Q8_0, x)
    xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
    assert np.array_equal(xq.data.cpu().numpy(), xq_ref)
    yref, _ = orc.mul_mat_q8act(TYPES[tname][1], packed, K, xq_ref)
    _, a = orc.mul_mat(TYPES[tname][1], packed, K, orc.dequantize(orc.Q8_0, xq_ref, K))
    y = Q.gemv(_weight(tname, packed, K, M), xq).cpu().numpy().astype(np.float64)
    err = np.abs(y - yref)
    tol = _i8_bound(K, tname, a)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


def test_gemv_swiglu_q8_activations_edge_cases(orc):
    tname, M, K, N = "Q4_0", 5632, 2048, 1
    _banner("gemv swiglu q8 activations edge")
    wg, x = _inputs(4500, M, K, N)
    wu = WL.outlier_weights(4550, M, K)
    t = TYPES[tname][1]
    pg, pu = orc.quantize(t, wg), orc.quantize(t, wu)
    xq_ref = orc.quantize(orc.Q8_0, x)
    xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
    gref, _ = orc.mul_mat_q8act(t, pg, K, xq_ref)
    uref, _ = orc.mul_mat_q8act(t, pu, K, xq_ref)
    xd = orc.dequantize(orc.Q8_0, xq_ref, K)
    _, ga = orc.mul_mat(t, pg, K, xd)
    _, ua = orc.mul_mat(t, pu, K, xd)
    href = orc.swiglu(gref, uref)
    h = Q.gemv_swiglu(_weight(tname, pg, K, M), _weight(tname, pu, K, M), xq).cpu().numpy().astype(np.float64)
    tol = _swiglu_tol(orc, gref, _i8_bound(K, tname, ga), uref, _i8_bound(K, tname, ua), href)
    err = np.abs(h - href)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"


# ------------------------------------------------------------ GEMM

GEMM_EDGE = [("Q4_0", 257, 2048, 129), ("Q4_0", 300, 5632, 200), ("Q8_0", 130, 2048, 65),
             ("F16", 130, 1024, 65), ("Q4_B64", 200, 2048, 130), ("Q8_B64", 64, 4096, 300),
             ("Q4_0", 64, 4096, 33)]


@pytest.mark.parametrize("case", GEMM_EDGE, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_gemm_edge_cases(orc, case):
    """Every output, with the split-K workspace the shape calls for and
    without one; bf16-rounded shifted activations."""
    tname, M, K, N = case
    _banner(f"gemm edge {tname} M={M} K={K} N={N}")
    w, x = _inputs(5000 + M + K + N, M, K, N)
    xbits = WL.round_bf16_bits(x)
    packed = _packed(orc, tname, w)
    t = TYPES[tname][1]
    yref, a = orc.mul_mat(t, packed, K, xbits, x_bf16_bits=True)
    ydiag, _ = orc.mul_mat(t, packed, K, xbits, x_bf16_bits=True, w_to_bf16=True)
    wt = _weight(tname, packed, K, M)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    for ws in ("auto", None):
        y = Q.gemm(wt, xt, workspace=ws).cpu().numpy()
        _assert_tol(y, yref, a, 1e-2, 1e-5, f"gemm edge {case} workspace={ws}")
        _assert_tol(y, ydiag, a, 1.1 * K * 2.0 ** -24, 1e-7, f"gemm edge diagnostic {case} workspace={ws}")


def test_gemm_batch_and_swiglu_edge_cases(orc):
    """A batched launch ([Wq Wk Wv]-like items) and the fused SwiGLU GEMM on
    edge-case weights and shifted activations."""
    K, N = 2048, 130
    _banner("gemm batch + swiglu edge")
    x = WL.shifted_activations(6007, N, K, outlier_seed=6000)
    xbits = WL.round_bf16_bits(x)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    items, refs = [], []
    for i, M in enumerate((300, 64, 64)):
        packed = orc.quantize(orc.Q4_0, WL.outlier_weights(6000 if i == 0 else 6000 + i, M, K))
        refs.append(orc.mul_mat(orc.Q4_0, packed, K, xbits, x_bf16_bits=True))
        items.append((B.Weight(torch.from_numpy(packed).to(DEV), B.Q4_0, K, M), xt, None))
    outs = Q.gemm_batch(items)
    for i, (y, (yref, a)) in enumerate(zip(outs, refs)):
        _assert_tol(y.cpu().numpy(), yref, a, 1e-2, 1e-5, f"gemm batch edge item {i}")
    M = 300
    pg = orc.quantize(orc.Q4_0, WL.outlier_weights(6000, M, K))
    pu = orc.quantize(orc.Q4_0, WL.outlier_weights(6050, M, K))
    gref, ga = orc.mul_mat(orc.Q4_0, pg, K, xbits, x_bf16_bits=True)
    uref, ua = orc.mul_mat(orc.Q4_0, pu, K, xbits, x_bf16_bits=True)
    href = orc.swiglu(gref, uref)
    h = Q.gemm_swiglu(B.Weight(torch.from_numpy(pg).to(DEV), B.Q4_0, K, M),
                      B.Weight(torch.from_numpy(pu).to(DEV), B.Q4_0, K, M), xt).cpu().numpy().astype(np.float64)
    tol = _swiglu_tol(orc, gref, 1e-2 * ga + 1e-5, uref, 1e-2 * ua + 1e-5, href)
    err = np.abs(h - href)
    assert np.isfinite(h).all()
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"
