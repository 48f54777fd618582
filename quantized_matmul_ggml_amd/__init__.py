"""libqmm: block-quantized MUL_MAT (decode GEMV, prefill GEMM) on MI355X.

The compute lives in hand-written HIP kernels (csrc/, built into libqmm.so by
``python -m quantized_matmul_ggml_amd.build``); ``binding`` is a thin ctypes
layer over the C ABI of include/qmm.h, with torch supplying device memory and
streams.
"""
from .binding import (BF16, F16, F32, Q4_0, Q4_B64, Q8_0, Q8_B64, QUANT_DEFAULT, QUANT_Q4_AMAX7, QmmError, Weight,
                      dequantize, f16_weight,
                      gemm, gemm_batch, gemm_noalloc, gemm_swiglu, gemm_workspace_size, gemv, gemv_batch, gemv_swiglu, quantize, record_size,
                      records_to_rows, stream_read, clock_probe, mfma_probe,
                      row_size, rows_to_records, strerror)

__all__ = ["BF16", "F16", "F32", "Q4_0", "Q4_B64", "Q8_0", "Q8_B64", "QUANT_DEFAULT", "QUANT_Q4_AMAX7", "QmmError",
           "Weight", "dequantize",
           "f16_weight", "gemm", "gemm_batch", "gemm_noalloc", "gemm_swiglu", "gemm_workspace_size", "gemv", "gemv_batch", "gemv_swiglu", "quantize", "record_size",
           "records_to_rows", "stream_read", "clock_probe", "mfma_probe", "row_size", "rows_to_records", "strerror"]
