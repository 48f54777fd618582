"""GPU parity over seeded random shapes: the decode GEMV (quantized and F16
rows), the fused gate/up SwiGLU GEMV, the integer-activation GEMV and the
prefill GEMM against the CPU oracle, over weight types, ragged row and token counts, K at and around the
GEMV kernels' range limits (128 and 192 blocks), 1 to 8 decode tokens and
padded activation and output pitches.  The shapes come from fixed seeds, so
the set is the same on every run; each case's oracle work is bounded
(M K N <= 2.5e7 for the GEMV, 8e7 for the GEMM).

Bars (as in test_gpu_parity.py):
  * fp32 activations: |y - y_ref| <= 1e-4 * a + 1e-6 per output;
  * SwiGLU: each sum's GEMV bound carried through Swish (|Swish'| <= 1.1)
    and the product, plus a few ulps of h;
  * Q8_0 activations: |y - y_q8| <= (nchunk + 16) 2^-24 a, against the
    oracle's integer path;
  * GEMM (bf16 activations): |y - y_ref| <= 1e-2 a + 1e-5, and the binary32
    summation bound against bf16-rounded weights.
"""
import numpy as np
import pytest
import torch

import quantized_matmul_ggml_amd as Q
from quantized_matmul_ggml_amd import binding as B
from quantized_matmul_ggml_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TYPES = {"Q8_0": (B.Q8_0, 3), "Q4_0": (B.Q4_0, 4), "Q8_B64": (B.Q8_B64, 5), "Q4_B64": (B.Q4_B64, 6)}
CANARY = 0x7FC0DEAD


def _cases(n=42, seed=20261203):
    rng = np.random.default_rng(seed)
    edges = [32, 64, 96, 1024, 2048, 4064, 4096, 4128, 5632, 6144, 6176, 8192]
    out = []
    for i in range(n):
        path = ("gemv", "swiglu", "q8x")[i % 3]
        tname = ("Q4_0", "Q8_0", "Q4_B64", "Q8_B64")[rng.integers(0, 4)]
        blk = 64 if tname.endswith("B64") else 32
        if rng.random() < 0.5:
            K = int(edges[rng.integers(0, len(edges))])
        else:
            K = int(rng.integers(1, 8192 // blk + 1)) * blk
        K = max(blk, K // blk * blk)
        N = int(rng.integers(1, 9))
        M = int(rng.integers(1, 3001))
        M = max(1, min(M, int(2.5e7 // (K * N))))
        x_pad = int(rng.choice([0, 16, 40]))
        out.append((path, tname, M, K, N, x_pad))
    return out


CASES = _cases()


def _guarded(rows, cols, pad=8):
    buf = torch.full((rows + 4, cols + 2 * pad), 0.0, dtype=torch.float32, device=DEV)
    buf.view(torch.int32).fill_(CANARY)
    return buf, buf[2:2 + rows, pad:pad + cols]


def _guard_intact(buf, rows, cols, pad=8):
    b = buf.cpu().numpy().view(np.uint32)
    inner = np.zeros(b.shape, bool)
    inner[2:2 + rows, pad:pad + cols] = True
    return bool((b[~inner] == CANARY).all())


def _x_padded(x, x_pad):
    buf = torch.zeros((x.shape[0], x.shape[1] + x_pad), dtype=torch.float32, device=DEV)
    buf[:, : x.shape[1]] = torch.from_numpy(x).to(DEV)
    return buf[:, : x.shape[1]]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-%dx%d-n%d-pad%d" % c)
def test_random_shape(orc, case):
    path, tname, M, K, N, x_pad = case
    print(f"[case] random {path} {tname} M={M} K={K} N={N} x_pad={x_pad}", flush=True)
    code, otype = TYPES[tname]
    seed = 31 * M + 7 * K + N
    w = WL.outlier_weights(seed, M, K) if seed % 2 else WL.weights(seed, M, K)
    x = WL.activations(seed + 1, N, K)
    packed = orc.quantize(otype, w)
    wt = Q.quantize(torch.from_numpy(w).to(DEV), code)
    assert np.array_equal(wt.data.cpu().numpy()[:, : packed.shape[1]], packed)

    if path == "gemv":
        yref, a = orc.mul_mat(otype, packed, K, x)
        buf, yv = _guarded(N, M)
        Q.gemv(wt, _x_padded(x, x_pad), out=yv)
        torch.cuda.synchronize()
        assert _guard_intact(buf, N, M), "wrote outside the output"
        y = yv.cpu().numpy().astype(np.float64)
        err, tol = np.abs(y - yref), 1e-4 * a + 1e-6
    elif path == "swiglu":
        w2 = WL.weights(seed + 2, M, K)
        packed2 = orc.quantize(otype, w2)
        wt2 = Q.quantize(torch.from_numpy(w2).to(DEV), code)
        gref, ga = orc.mul_mat(otype, packed, K, x)
        uref, ua = orc.mul_mat(otype, packed2, K, x)
        href = orc.swiglu(gref, uref)
        buf, hv = _guarded(N, M)
        Q.gemv_swiglu(wt, wt2, _x_padded(x, x_pad), out=hv)
        torch.cuda.synchronize()
        assert _guard_intact(buf, N, M), "wrote outside the output"
        y = hv.cpu().numpy().astype(np.float64)
        eg, eu = 1e-4 * ga + 1e-6, 1e-4 * ua + 1e-6
        sg = np.array([orc.swish(v) for v in gref.ravel()]).reshape(gref.shape)
        err = np.abs(y - href)
        tol = 1.1 * eg * (np.abs(uref) + eu) + np.abs(sg) * eu + 2.0 ** -20 * np.abs(href)
    else:
        xq_ref = orc.quantize(orc.Q8_0, x)
        xq = Q.quantize(torch.from_numpy(x).to(DEV), B.Q8_0)
        assert np.array_equal(xq.data.cpu().numpy(), xq_ref)
        yref, _ = orc.mul_mat_q8act(otype, packed, K, xq_ref)
        _, a = orc.mul_mat(otype, packed, K, orc.dequantize(orc.Q8_0, xq_ref, K))
        buf, yv = _guarded(N, M)
        Q.gemv(wt, xq, out=yv)
        torch.cuda.synchronize()
        assert _guard_intact(buf, N, M), "wrote outside the output"
        y = yv.cpu().numpy().astype(np.float64)
        nchunk = K // 32 if tname.startswith("Q4") else K // 16
        err, tol = np.abs(y - yref), (nchunk + 16) * 2.0 ** -24 * a + 1e-30
    assert np.isfinite(y).all()
    worst = float((err / tol).max())
    assert worst <= 1.0, f"worst err/bound {worst:.3g}"


# ------------------------------------------------------------------ F16 GEMV

def _f16_cases(n=14, seed=20261205):
    """F16 rows: K on and off the 32-block grid (the matrix cores take whole
    blocks from 3 or 5 tokens, the VALU kernel the rest), 1 to 8 tokens,
    row pitches padded to 16 bytes or further."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(rng.integers(1, 8192 // 32 + 1)) * 32
        if i % 3 == 2:
            K = max(1, K - int(rng.integers(1, 32)))
        N = int(rng.integers(1, 9))
        M = int(rng.integers(1, 4001))
        M = max(1, min(M, int(2.5e7 // (K * N))))
        extra = int(rng.choice([0, 8, 24]))            # halves of padding past 16-byte alignment
        out.append((M, K, N, extra))
    return out


F16_CASES = _f16_cases()


@pytest.mark.parametrize("case", F16_CASES, ids=lambda c: "f16-%dx%d-n%d-pad%d" % c)
def test_random_f16_shape(orc, case):
    """|y - y_ref| <= 1e-4 a + 1e-6, the row padding filled with NaN."""
    M, K, N, extra = case
    print(f"[case] random f16 M={M} K={K} N={N} pad={extra}", flush=True)
    seed = 13 * M + 3 * K + N
    w = WL.weights(seed, M, K)
    x = WL.activations(seed + 1, N, K)
    pitch = (K + 7) // 8 * 8 + extra                 # halves, a multiple of 8
    wbuf = torch.full((M, pitch), float("nan"), dtype=torch.float16, device=DEV)
    wbuf[:, :K] = torch.from_numpy(WL.round_f16(w)).to(DEV)
    wt = B.Weight(wbuf, B.F16, K, M)
    packed = WL.round_f16(w).view(np.uint8).reshape(M, 2 * K)
    yref, a = orc.mul_mat(orc.F16, packed, K, x)
    buf, yv = _guarded(N, M)
    Q.gemv(wt, torch.from_numpy(x).to(DEV), out=yv)
    torch.cuda.synchronize()
    assert _guard_intact(buf, N, M), "wrote outside the output"
    y = yv.cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all()
    worst = float((np.abs(y - yref) / (1e-4 * a + 1e-6)).max())
    assert worst <= 1.0, f"worst err/bound {worst:.3g}"


# ------------------------------------------------------------------ GEMM

def _gemm_cases(n=18, seed=20261204):
    """Prefill GEMM shapes: ragged M, N and K (K a multiple of the block),
    every weight type; bf16 activations."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        tname = ("Q4_0", "Q8_0", "Q4_B64", "Q8_B64", "F16")[i % 5]
        blk = 64 if tname.endswith("B64") else 32
        K = int(rng.integers(1, 6144 // blk + 1)) * blk
        M = int(rng.integers(1, 1500))
        N = int(rng.integers(1, 700))
        while M * K * N > 8e7:                  # halve the larger of M and N
            if N > M:
                N = max(1, N // 2)
            else:
                M = max(1, M // 2)
        out.append((tname, M, K, N))
    return out


GEMM_CASES = _gemm_cases()
GEMM_TYPES = dict(TYPES, F16=(B.F16, 1))


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "%s-%dx%d-n%d" % c)
def test_random_gemm_shape(orc, case):
    """|y - y_ref| <= 1e-2 a + 1e-5, and against the oracle's bf16-weight
    variant within the binary32 summation bound 1.1 K 2^-24 a + 1e-7; with
    the split-K workspace the shape calls for and without one."""
    tname, M, K, N = case
    print(f"[case] random gemm {tname} M={M} K={K} N={N}", flush=True)
    code, otype = GEMM_TYPES[tname]
    seed = 17 * M + 5 * K + N
    w = WL.weights(seed, M, K)
    xbits = WL.round_bf16_bits(WL.activations(seed + 1, N, K))
    if tname == "F16":
        packed = WL.round_f16(w).view(np.uint8).reshape(M, 2 * K)
        wt = B.Weight(torch.from_numpy(packed.view(np.float16)).to(DEV), B.F16, K, M)
    else:
        packed = orc.quantize(otype, w)
        wt = B.Weight(torch.from_numpy(packed).to(DEV), code, K, M)
    yref, a = orc.mul_mat(otype, packed, K, xbits, x_bf16_bits=True)
    ydiag, _ = orc.mul_mat(otype, packed, K, xbits, x_bf16_bits=True, w_to_bf16=True)
    xt = WL.bf16_bits_to_torch(xbits, DEV)
    for ws in ("auto", None):
        buf, yv = _guarded(N, M)
        Q.gemm(wt, xt, out=yv, workspace=ws)
        torch.cuda.synchronize()
        assert _guard_intact(buf, N, M), "wrote outside the output"
        y = yv.cpu().numpy().astype(np.float64)
        assert np.isfinite(y).all()
        r1 = float((np.abs(y - yref) / (1e-2 * a + 1e-5)).max())
        r2 = float((np.abs(y - ydiag) / (1.1 * K * 2.0 ** -24 * a + 1e-7)).max())
        assert r1 <= 1.0 and r2 <= 1.0, f"workspace={ws}: worst {r1:.3g} (bar), {r2:.3g} (bf16-weight diagnostic)"
