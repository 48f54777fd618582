"""ctypes binding of libqmm (include/qmm.h): argument marshalling only.

Every computation runs in the HIP kernels of libqmm.so; this module only
builds ``qmm_tensor`` descriptors from torch tensors (device memory and the
current stream come from torch) and turns non-zero status codes into
exceptions.  There is no CPU fallback: if the library is missing or a tensor
is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmm.so")

# qmm_type
F32, F16, BF16, Q8_0, Q4_0, Q8_B64, Q4_B64 = 0, 1, 2, 3, 4, 5, 6
TYPE_NAMES = {F32: "F32", F16: "F16", BF16: "BF16", Q8_0: "Q8_0", Q4_0: "Q4_0",
              Q8_B64: "Q8_B64", Q4_B64: "Q4_B64"}

# qmm_status
OK, ERR_NULL, ERR_TYPE, ERR_SHAPE, ERR_LAYOUT, ERR_ALIAS, ERR_UNSUPPORTED, ERR_DEVICE, ERR_SCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ("qmm_row_size", "qmm_quantize", "qmm_quantize_rule", "qmm_dequantize", "qmm_gemv", "qmm_gemv_batch",
           "qmm_gemv_swiglu", "qmm_gemm", "qmm_gemm_ws", "qmm_gemm_noalloc", "qmm_gemm_workspace_size", "qmm_gemm_batch", "qmm_gemm_swiglu", "qmm_record_size", "qmm_records_to_rows",
           "qmm_rows_to_records", "qmm_stream_read", "qmm_clock_probe", "qmm_wall_clock_khz", "qmm_strerror")
GEMV_BATCH_MAX = 8


class QmmTensor(ctypes.Structure):
    """Mirror of ``qmm_tensor`` (ne/nb convention: ne[0] contiguous, nb in bytes)."""
    _fields_ = [("type", ctypes.c_int32), ("n_dims", ctypes.c_int32),
                ("ne", ctypes.c_int64 * 4), ("nb", ctypes.c_uint64 * 4),
                ("data", ctypes.c_void_p)]


class QmmGemvItem(ctypes.Structure):
    """Mirror of ``qmm_gemv_item``."""
    _fields_ = [("w", ctypes.POINTER(QmmTensor)), ("x_f32", ctypes.POINTER(QmmTensor)),
                ("y_f32", ctypes.POINTER(QmmTensor))]


class QmmGemmItem(ctypes.Structure):
    """Mirror of ``qmm_gemm_item``."""
    _fields_ = [("w", ctypes.POINTER(QmmTensor)), ("x_bf16", ctypes.POINTER(QmmTensor)),
                ("y_f32", ctypes.POINTER(QmmTensor))]


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqmm.so from the package directory (build it with build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m quantized_matmul_ggml_amd.build` "
                "(hipcc, gfx950); there is no fallback implementation")
        h = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(QmmTensor)
        h.qmm_row_size.argtypes = [ctypes.c_int32, ctypes.c_int64]
        h.qmm_row_size.restype = ctypes.c_size_t
        h.qmm_quantize.argtypes = [P, P, ctypes.c_void_p]
        h.qmm_quantize_rule.argtypes = [P, P, ctypes.c_int32, ctypes.c_void_p]
        h.qmm_quantize_rule.restype = ctypes.c_int
        h.qmm_dequantize.argtypes = [P, P, ctypes.c_void_p]
        h.qmm_gemv.argtypes = [P, P, P, ctypes.c_void_p]
        h.qmm_gemm.argtypes = [P, P, P, ctypes.c_void_p]
        h.qmm_gemm_ws.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        h.qmm_gemm_ws.restype = ctypes.c_int
        h.qmm_gemm_noalloc.argtypes = [P, P, P, ctypes.c_size_t, ctypes.c_void_p]
        h.qmm_gemm_noalloc.restype = ctypes.c_int
        h.qmm_gemm_workspace_size.argtypes = [P, P]
        h.qmm_gemm_workspace_size.restype = ctypes.c_size_t
        h.qmm_gemm_batch.argtypes = [ctypes.POINTER(QmmGemmItem), ctypes.c_int32, ctypes.c_void_p]
        h.qmm_gemm_batch.restype = ctypes.c_int
        h.qmm_gemm_swiglu.argtypes = [P, P, P, P, ctypes.c_void_p]
        h.qmm_gemm_swiglu.restype = ctypes.c_int
        h.qmm_gemv_swiglu.argtypes = [P, P, P, P, ctypes.c_void_p]
        h.qmm_gemv_swiglu.restype = ctypes.c_int
        h.qmm_record_size.argtypes = [ctypes.c_int32]
        h.qmm_record_size.restype = ctypes.c_size_t
        h.qmm_records_to_rows.argtypes = [ctypes.c_void_p, P, ctypes.c_void_p]
        h.qmm_records_to_rows.restype = ctypes.c_int
        h.qmm_rows_to_records.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
        h.qmm_rows_to_records.restype = ctypes.c_int
        h.qmm_gemv_batch.argtypes = [ctypes.POINTER(QmmGemvItem), ctypes.c_int32, ctypes.c_void_p]
        h.qmm_gemv_batch.restype = ctypes.c_int
        for f in ("qmm_quantize", "qmm_dequantize", "qmm_gemv", "qmm_gemm"):
            getattr(h, f).restype = ctypes.c_int
        h.qmm_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p]
        h.qmm_stream_read.restype = ctypes.c_int
        h.qmm_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
        h.qmm_clock_probe.restype = ctypes.c_int
        h.qmm_wall_clock_khz.argtypes = []
        h.qmm_wall_clock_khz.restype = ctypes.c_int64
        h.qmm_strerror.argtypes = [ctypes.c_int]
        h.qmm_strerror.restype = ctypes.c_char_p
        _lib = h
    return _lib


def strerror(status: int) -> str:
    return lib().qmm_strerror(status).decode()


def row_size(type_: int, K: int) -> int:
    return int(lib().qmm_row_size(type_, K))


def make_desc(type_: int, ne0: int, ne1: int, nb1: int, data_ptr: int, n_dims: int = 2,
              nb0: int | None = None) -> QmmTensor:
    """A raw descriptor (used directly by the boundary tests)."""
    t = QmmTensor()
    t.type = type_
    t.n_dims = n_dims
    t.ne[0], t.ne[1], t.ne[2], t.ne[3] = ne0, ne1, 1, 1
    if nb0 is None:
        nb0 = {F32: 4, F16: 2, BF16: 2}.get(type_, 0)
    t.nb[0], t.nb[1] = nb0, nb1
    t.nb[2] = t.nb[3] = nb1 * max(ne1, 1)
    t.data = data_ptr
    return t


@dataclass
class Weight:
    """A weight matrix W (ne = [K, M]): M rows of K weights on the GPU.

    data is uint8 (M, pitch) for quantized rows (Q8_0, Q4_0, Q8_B64, Q4_B64) in the row-planar layout of
    include/qmm.h, or float16 (M, >= K) for F16 rows."""
    data: torch.Tensor
    type: int
    K: int
    M: int

    @property
    def pitch(self) -> int:
        return self.data.stride(0) * self.data.element_size()

    def desc(self) -> QmmTensor:
        return make_desc(self.type, self.K, self.M, self.pitch, self.data.data_ptr())

    def rows(self, r0: int, r1: int) -> "Weight":
        """Row-range view [r0, r1): no copy, same pitch."""
        return Weight(self.data[r0:r1], self.type, self.K, r1 - r0)


def _need_gpu(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libqmm operates on GPU tensors only")


def _dense_desc(t: torch.Tensor, type_: int) -> QmmTensor:
    """2-D row-major torch tensor (rows, cols) -> ne = [cols, rows]."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    es = t.element_size()
    if t.numel() == 0:                  # empty: strides are meaningless
        return make_desc(type_, t.shape[1], t.shape[0], t.shape[1] * es, t.data_ptr())
    if t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride 1 along the last dimension)")
    return make_desc(type_, t.shape[1], t.shape[0], t.stride(0) * es, t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != OK:
        raise QmmError(status, where)


QUANT_DEFAULT, QUANT_Q4_AMAX7 = 0, 1


def quantize(w: torch.Tensor, type_: int, *, pitch: int | None = None, rule: int = QUANT_DEFAULT,
             stream=None) -> Weight:
    """Quantize fp32 rows w (M, K) on the GPU into Q8_0 / Q4_0 rows, or their
    64-weight-block variants Q8_B64 / Q4_B64 (rule: QUANT_DEFAULT, or
    QUANT_Q4_AMAX7 for the symmetric amax/7 Q4 rule)."""
    _need_gpu(w)
    M, K = w.shape
    rs = row_size(type_, K)
    pitch = rs if pitch is None else pitch
    out = torch.empty((M, pitch), dtype=torch.uint8, device=w.device)
    if pitch > rs:
        out[:, rs:].zero_()
    wt = Weight(out, type_, K, M)
    src, dst = _dense_desc(w, F32), wt.desc()
    _check(lib().qmm_quantize_rule(ctypes.byref(src), ctypes.byref(dst), rule, _stream(stream)),
           "qmm_quantize_rule")
    return wt


def dequantize(w: Weight, *, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """W' as fp32 (M, K)."""
    _need_gpu(w.data)
    if out is None:
        out = torch.empty((w.M, w.K), dtype=torch.float32, device=w.data.device)
    src, dst = w.desc(), _dense_desc(out, F32)
    _check(lib().qmm_dequantize(ctypes.byref(src), ctypes.byref(dst), _stream(stream)),
           "qmm_dequantize")
    return out


def f16_weight(w16: torch.Tensor) -> Weight:
    """Wrap float16 rows (M, K) as an F16 weight."""
    _need_gpu(w16)
    assert w16.dtype == torch.float16
    return Weight(w16, F16, w16.shape[1], w16.shape[0])


def gemv(w: Weight, x, *, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y (N, M) fp32 = x (N, K) times W'^T; 1 <= N <= 8.  x is fp32 (N, K), or
    a Q8_0 Weight of N rows (activations quantized with quantize()) for the
    integer-activation path."""
    if isinstance(x, Weight):
        _need_gpu(w.data, x.data)
        n, dev, xd = x.M, x.data.device, x.desc()
    else:
        _need_gpu(w.data, x)
        n, dev, xd = x.shape[0], x.device, _dense_desc(x, F32)
    if out is None:
        out = torch.empty((n, w.M), dtype=torch.float32, device=dev)
    wd, yd = w.desc(), _dense_desc(out, F32)
    _check(lib().qmm_gemv(ctypes.byref(wd), ctypes.byref(xd), ctypes.byref(yd), _stream(stream)),
           "qmm_gemv")
    return out


def gemv_batch(items, *, stream=None) -> list:
    """Several GEMVs in one launch: items = [(Weight, x, out or None), ...]
    sharing the weight type, K and N; x is fp32 (N, K) in every item, or a
    Q8_0 Weight of N rows in every item (the integer-activation path).
    Returns the outputs."""
    descs, keep, outs = [], [], []
    for w, x, out in items:
        if isinstance(x, Weight):
            _need_gpu(w.data, x.data)
            n, dev, xd = x.M, x.data.device, x.desc()
        else:
            _need_gpu(w.data, x)
            n, dev, xd = x.shape[0], x.device, _dense_desc(x, F32)
        if out is None:
            out = torch.empty((n, w.M), dtype=torch.float32, device=dev)
        wd, yd = w.desc(), _dense_desc(out, F32)
        keep += [wd, xd, yd]
        descs.append(QmmGemvItem(ctypes.pointer(wd), ctypes.pointer(xd), ctypes.pointer(yd)))
        outs.append(out)
    arr = (QmmGemvItem * max(1, len(descs)))(*descs)
    _check(lib().qmm_gemv_batch(arr, len(descs), _stream(stream)), "qmm_gemv_batch")
    return outs


def gemv_swiglu(w_gate: Weight, w_up: Weight, x, *, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """h (N, M) fp32 = Swish(x W_gate'^T) * (x W_up'^T), one fused launch; 1 <= N <= 8.
    x is fp32 (N, K), or a Q8_0 Weight of N rows for the integer-activation path."""
    if isinstance(x, Weight):
        _need_gpu(w_gate.data, w_up.data, x.data)
        n, dev, xd = x.M, x.data.device, x.desc()
    else:
        _need_gpu(w_gate.data, w_up.data, x)
        n, dev, xd = x.shape[0], x.device, _dense_desc(x, F32)
    if out is None:
        out = torch.empty((n, w_gate.M), dtype=torch.float32, device=dev)
    gd, ud, hd = w_gate.desc(), w_up.desc(), _dense_desc(out, F32)
    _check(lib().qmm_gemv_swiglu(ctypes.byref(gd), ctypes.byref(ud), ctypes.byref(xd), ctypes.byref(hd),
                                 _stream(stream)), "qmm_gemv_swiglu")
    return out


def record_size(type_: int) -> int:
    """Bytes of one GGUF-style block record (18 for Q4_0, 34 for Q8_0, else 0)."""
    return int(lib().qmm_record_size(type_))


def records_to_rows(records: torch.Tensor, type_: int, K: int, M: int, *, pitch: int | None = None,
                    stream=None) -> Weight:
    """Packed rows (a Weight) from M * K/32 block records (uint8 device tensor)."""
    _need_gpu(records)
    rs = row_size(type_, K)
    pitch = rs if pitch is None else pitch
    out = torch.zeros((M, pitch), dtype=torch.uint8, device=records.device)
    wt = Weight(out, type_, K, M)
    d = wt.desc()
    _check(lib().qmm_records_to_rows(ctypes.c_void_p(records.data_ptr()), ctypes.byref(d), _stream(stream)),
           "qmm_records_to_rows")
    return wt


def rows_to_records(w: Weight, *, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The M * K/32 block records of a quantized Weight (uint8 device tensor)."""
    _need_gpu(w.data)
    n = w.M * (w.K // 32) * record_size(w.type)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.data.device)
    d = w.desc()
    _check(lib().qmm_rows_to_records(ctypes.byref(d), ctypes.c_void_p(out.data_ptr()), _stream(stream)),
           "qmm_rows_to_records")
    return out


def gemm_workspace_size(w: Weight, x: torch.Tensor) -> int:
    """Bytes of workspace qmm_gemm_ws uses to split K for these shapes (0: no split)."""
    wd, xd = w.desc(), _dense_desc(x, BF16)
    return int(lib().qmm_gemm_workspace_size(ctypes.byref(wd), ctypes.byref(xd)))


def gemm(w: Weight, x: torch.Tensor, *, out: torch.Tensor | None = None, workspace="auto",
         stream=None) -> torch.Tensor:
    """y (N, M) fp32 = x (N, K) bf16 times W'^T on the bf16 matrix cores.

    workspace: "auto" allocates the split-K workspace the shapes call for (a
    torch allocation, so it is graph-capture safe), None runs without one
    (qmm_gemm), or a uint8 device tensor to use as is."""
    _need_gpu(w.data, x)
    if out is None:
        out = torch.empty((x.shape[0], w.M), dtype=torch.float32, device=x.device)
    wd, xd, yd = w.desc(), _dense_desc(x, BF16), _dense_desc(out, F32)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
        n = int(lib().qmm_gemm_workspace_size(ctypes.byref(wd), ctypes.byref(xd)))
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
        if workspace is not None and stream is not None:
            # freed when this call returns: keep the allocator from handing it
            # out again before the kernels on `stream` have run
            workspace.record_stream(stream)
    if workspace is None:
        _check(lib().qmm_gemm(ctypes.byref(wd), ctypes.byref(xd), ctypes.byref(yd), _stream(stream)),
               "qmm_gemm")
    else:
        _need_gpu(workspace)
        _check(lib().qmm_gemm_ws(ctypes.byref(wd), ctypes.byref(xd), ctypes.byref(yd),
                                 ctypes.c_void_p(workspace.data_ptr()),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
               "qmm_gemm_ws")
    return out


def gemm_noalloc(w: Weight, x: torch.Tensor, out: torch.Tensor, *, workspace_bytes: int | None = None,
                 stream=None) -> torch.Tensor:
    """qmm_gemm_noalloc: the GEMM with its split-K partial sums in the
    library's static scratch array (no allocation in the call; `out` is the
    caller's).  workspace_bytes defaults to the full split of these shapes."""
    _need_gpu(w.data, x, out)
    wd, xd, yd = w.desc(), _dense_desc(x, BF16), _dense_desc(out, F32)
    if workspace_bytes is None:
        workspace_bytes = int(lib().qmm_gemm_workspace_size(ctypes.byref(wd), ctypes.byref(xd)))
    _check(lib().qmm_gemm_noalloc(ctypes.byref(wd), ctypes.byref(xd), ctypes.byref(yd),
                                  ctypes.c_size_t(workspace_bytes), _stream(stream)), "qmm_gemm_noalloc")
    return out


def gemm_swiglu(w_gate: Weight, w_up: Weight, x: torch.Tensor, *, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """h (N, M) fp32 = Swish(x W_gate'^T) * (x W_up'^T) for bf16 x (N, K), one fused launch."""
    _need_gpu(w_gate.data, w_up.data, x)
    if out is None:
        out = torch.empty((x.shape[0], w_gate.M), dtype=torch.float32, device=x.device)
    gd, ud, xd, hd = w_gate.desc(), w_up.desc(), _dense_desc(x, BF16), _dense_desc(out, F32)
    _check(lib().qmm_gemm_swiglu(ctypes.byref(gd), ctypes.byref(ud), ctypes.byref(xd), ctypes.byref(hd),
                                 _stream(stream)), "qmm_gemm_swiglu")
    return out


def gemm_batch(items, *, stream=None) -> list:
    """Several prefill GEMMs in one launch: items = [(Weight, x (N, K) bf16, out or None), ...]
    sharing the weight type, K and N.  Returns the outputs."""
    descs, keep, outs = [], [], []
    for w, x, out in items:
        _need_gpu(w.data, x)
        if out is None:
            out = torch.empty((x.shape[0], w.M), dtype=torch.float32, device=x.device)
        wd, xd, yd = w.desc(), _dense_desc(x, BF16), _dense_desc(out, F32)
        keep += [wd, xd, yd]
        descs.append(QmmGemmItem(ctypes.pointer(wd), ctypes.pointer(xd), ctypes.pointer(yd)))
        outs.append(out)
    arr = (QmmGemmItem * max(1, len(descs)))(*descs)
    _check(lib().qmm_gemm_batch(arr, len(descs), _stream(stream)), "qmm_gemm_batch")
    return outs


def call_batch_raw(triples, count=None, stream: int = 0) -> int:
    """qmm_gemv_batch with hand-made descriptors [(w, x, y), ...]; returns the status."""
    items = [QmmGemvItem(*(ctypes.pointer(d) if d is not None else None for d in t)) for t in triples]
    arr = (QmmGemvItem * max(1, len(items)))(*items)
    n = len(items) if count is None else count
    return lib().qmm_gemv_batch(arr, n, ctypes.c_void_p(stream))


def call_raw(name: str, *descs: QmmTensor, stream: int = 0) -> int:
    """Call an entry point with hand-made descriptors; returns the status."""
    fn = getattr(lib(), name)
    return fn(*[ctypes.byref(d) if d is not None else None for d in descs], ctypes.c_void_p(stream))


def stream_read(src: torch.Tensor, sink: torch.Tensor, *, nbytes: int | None = None, workgroups: int = 1024,
                stream=None) -> None:
    """qmm_stream_read over the first nbytes (default: all) of the device
    tensor src; sink: an int32 device tensor of at least `workgroups` words."""
    _need_gpu(src, sink)
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink holds fewer words than workgroups")
    _check(lib().qmm_stream_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_size_t(n),
                                 ctypes.c_void_p(sink.data_ptr()), workgroups, _stream(stream)),
           "qmm_stream_read")


def clock_probe(workgroups: int = 256, iters: int = 20000, mode: int = 0) -> float:
    """Shader clock in MHz under a dependent chain on every wave (mode 0:
    binary32 FMAs, mode 1: bf16 matrix instructions), from the device's
    shader-clock and constant-rate counters; synchronizes."""
    out = torch.zeros(8 * workgroups, dtype=torch.int64, device="cuda")
    _check(lib().qmm_clock_probe(ctypes.c_void_p(out.data_ptr()), workgroups, iters, mode, _stream(None)),
           "qmm_clock_probe")
    d = out.view(-1, 2).cpu()
    wall_khz = int(lib().qmm_wall_clock_khz())
    if wall_khz <= 0:
        raise QmmError(wall_khz, "qmm_wall_clock_khz")
    return float(d[:, 0].sum()) / float(d[:, 1].sum()) * wall_khz / 1e3


def mfma_probe(mode: int, workgroups: int = 256, iters: int = 4000) -> dict:
    """The block-GEMM inner-loop probe (qmm_clock_probe modes 2-4) on every
    CU: multiply-add rate in TFLOP/s over the waves' own clocks, and shader
    clock cycles per round (four 32 x 32 x 32 tile-blocks) per wave: the mean
    over waves and the slowest wave (waves sharing a SIMD do not run in
    lockstep, so the SIMD's rate is that of its last wave to finish)."""
    out = torch.zeros(8 * workgroups, dtype=torch.int64, device="cuda")
    _check(lib().qmm_clock_probe(ctypes.c_void_p(out.data_ptr()), workgroups, iters, mode, _stream(None)),
           "qmm_clock_probe")
    d = out.view(-1, 2).cpu().double()
    wall_khz = int(lib().qmm_wall_clock_khz())
    if wall_khz <= 0:
        raise QmmError(wall_khz, "qmm_wall_clock_khz")
    seconds = float(d[:, 1].mean()) / (wall_khz * 1e3)
    flops = 4.0 * workgroups * iters * 4 * 2 * 32 * 32 * 32
    return {"tflops": flops / seconds / 1e12, "cycles_per_round": float(d[:, 0].mean()) / iters,
            "cycles_per_round_max": float(d[:, 0].max()) / iters}
