"""The entry points under HIP graph capture (GPU).

The benchmark captures the decode step and the prefill GEMM into HIP graphs
and replays them, so every kernel path it times is checked here the same
way: one graph holds a one-token GEMV, a GEMV batch of eight tokens (the
matrix-core kernel), the fused gate/up SwiGLU projection, an integer-
activation GEMV, the prefill GEMM (its K split over a workspace the binding
allocates during capture), a batched prefill GEMM, the fused gate/up SwiGLU
prefill GEMM and a 64-weight-block GEMV.  The graph is
replayed several times with new inputs written eagerly (and the device
synchronized) between replays; every replay must equal, bit for bit, the
same calls made eagerly on the same inputs (the kernels are deterministic).
The library enqueues no memset, so nothing in the graph depends on one.
"""
import numpy as np
import pytest
import torch

import quantized_matmul_ggml_amd as Q
from quantized_matmul_ggml_amd import workloads as WL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _calls(ops, ins, outs):
    """Enqueue every operation of the graph on the current stream."""
    w4, wg, wu, w64, wq = ops
    Q.gemv(w4, ins["x1"], out=outs["y1"])
    Q.gemv_batch([(wg, ins["x8"], outs["g8"]), (wu, ins["x8"], outs["u8"])])
    Q.gemv_swiglu(wg, wu, ins["x1"], out=outs["h"])
    Q.gemv(wq, ins["xq"], out=outs["yi"])
    Q.gemm(w4, ins["xb"], out=outs["Y"])
    Q.gemm_batch([(w4, ins["xb"], outs["Yb1"]), (wg, ins["xb"], outs["Yb2"])])
    Q.gemm_swiglu(wg, wu, ins["xb"], out=outs["Hb"])
    Q.gemv(w64, ins["x3"], out=outs["y64"])


def _fresh_inputs(ins, seed):
    """New values written in place (the graph keeps the buffers' addresses)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    ins["x1"].copy_(torch.randn(ins["x1"].shape, device=DEV, generator=g))
    ins["x8"].copy_(torch.randn(ins["x8"].shape, device=DEV, generator=g))
    ins["x3"].copy_(torch.randn(ins["x3"].shape, device=DEV, generator=g))
    ins["xb"].copy_(torch.randn(ins["xb"].shape, device=DEV, generator=g).to(torch.bfloat16))
    xq = Q.quantize(torch.randn((2, ins["xq"].K), device=DEV, generator=g), Q.Q8_0)
    ins["xq"].data.copy_(xq.data)


def test_graph_replays_match_eager_calls():
    print("[case] graph capture of gemv / gemv_batch / swiglu / int8 gemv / gemm / gemm_batch / 64-block gemv",
          flush=True)
    K, M, MF = 2048, 1000, 9000
    w4 = Q.quantize(WL.weights_device(WL.seed(8, 0), M, K, DEV), Q.Q4_0)
    wg = Q.quantize(WL.weights_device(WL.seed(8, 1), MF, K, DEV), Q.Q4_0)
    wu = Q.quantize(WL.weights_device(WL.seed(8, 2), MF, K, DEV), Q.Q4_0)
    w64 = Q.quantize(WL.weights_device(WL.seed(8, 3), M, K, DEV), Q.Q8_B64)
    wq = Q.quantize(WL.weights_device(WL.seed(8, 4), M, K, DEV), Q.Q8_0)
    ops = (w4, wg, wu, w64, wq)
    ins = {"x1": torch.empty((1, K), device=DEV), "x8": torch.empty((8, K), device=DEV),
           "x3": torch.empty((3, K), device=DEV),
           "xb": torch.empty((300, K), device=DEV, dtype=torch.bfloat16),
           "xq": Q.quantize(torch.zeros((2, K), device=DEV), Q.Q8_0)}
    shapes = {"y1": (1, M), "g8": (8, MF), "u8": (8, MF), "h": (1, MF), "yi": (2, M),
              "Y": (300, M), "y64": (3, M), "Yb1": (300, M), "Yb2": (300, MF), "Hb": (300, MF)}
    outs = {k: torch.full(s, float("nan"), device=DEV) for k, s in shapes.items()}
    ref = {k: torch.empty(s, device=DEV) for k, s in shapes.items()}

    _fresh_inputs(ins, 1)
    _calls(ops, ins, ref)                        # eager warm-up (sets kernel attributes)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _calls(ops, ins, outs)
    torch.cuda.synchronize()

    for rep, seed in enumerate((11, 12, 13)):
        _fresh_inputs(ins, seed)                 # eager work between replays
        torch.cuda.synchronize()
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _calls(ops, ins, ref)
        torch.cuda.synchronize()
        for k in shapes:
            a, b = outs[k].cpu().numpy(), ref[k].cpu().numpy()
            assert np.isfinite(a).all(), f"replay {rep}: {k} not written"
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {rep}: {k} differs from eager"
