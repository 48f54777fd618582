"""qmm_gemm_noalloc, the GEMM whose split-K partial sums live in the
library's static scratch array, against qmm_gemm_ws with a caller workspace
of the same size: bit-identical results on two calls in a row (the second
with a smaller product), the size limit, and no device allocation by the
call."""
import numpy as np
import pytest
import torch

import quantized_matmul_ggml_amd as Q
from quantized_matmul_ggml_amd import binding as B
from quantized_matmul_ggml_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(orc, M, K, N, seed):
    w = WL.weights(seed, M, K)
    packed = orc.quantize(orc.Q4_0, w)
    wt = B.Weight(torch.from_numpy(packed).to(DEV), B.Q4_0, K, M)
    xbits = WL.round_bf16_bits(WL.activations(seed + 1, N, K))
    return packed, xbits, wt, WL.bf16_bits_to_torch(xbits, DEV)


def test_gemm_noalloc_matches_gemm_ws(orc):
    # the down projection at 512 tokens (four K ranges, the whole 16 MiB),
    # then a smaller product (256 x 2048 x 128, four ranges of 128 KiB)
    prev = None
    for M, K, N, seed in ((2048, 5632, 512, 71), (256, 2048, 128, 73)):
        print(f"[case] gemm noalloc {M}x{K}x{N}", flush=True)
        packed, xbits, wt, xt = _case(orc, M, K, N, seed)
        need = Q.gemm_workspace_size(wt, xt)
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert need < prev
        prev = need
        ref = torch.empty((N, M), dtype=torch.float32, device=DEV)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        Q.gemm(wt, xt, out=ref, workspace=ws)
        out = torch.full((N, M), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        Q.gemm_noalloc(wt, xt, out, workspace_bytes=need)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        y = out.cpu().numpy()
        assert np.array_equal(y.view(np.uint32), ref.cpu().numpy().view(np.uint32))
        # and the GEMM bound against the oracle on sampled outputs
        rng = np.random.default_rng(seed)
        ms, ns = rng.integers(0, M, 2048), rng.integers(0, N, 2048)
        yr, a = orc.mul_mat_pairs(orc.Q4_0, packed, K, xbits, ms, ns, x_bf16_bits=True)
        assert (np.abs(y[ns, ms] - yr) <= 1e-2 * a + 1e-5).all()


def test_gemm_noalloc_limits(orc):
    print("[case] gemm noalloc limits", flush=True)
    M, K, N = 300, 4096, 100
    _, _, wt, xt = _case(orc, M, K, N, 75)
    out = torch.empty((N, M), dtype=torch.float32, device=DEV)
    with pytest.raises(Q.QmmError) as e:
        Q.gemm_noalloc(wt, xt, out, workspace_bytes=B.NOALLOC_SCRATCH_BYTES + 16)
    assert e.value.status == B.ERR_SCRATCH
    # without a split it is qmm_gemm
    Q.gemm_noalloc(wt, xt, out, workspace_bytes=0)
    ref = Q.gemm(wt, xt, workspace=None)
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # a size below the full split chooses the same smaller split as qmm_gemm_ws
    need = Q.gemm_workspace_size(wt, xt)
    part = need // 4 + 16
    Q.gemm_noalloc(wt, xt, out, workspace_bytes=part)
    ref2 = Q.gemm(wt, xt, workspace=torch.empty(part, dtype=torch.uint8, device=DEV))
    assert torch.equal(out.view(torch.int32), ref2.view(torch.int32))
