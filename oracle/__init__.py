"""CPU oracle for block-quantized MUL_MAT (ctypes wrapper over qmm_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never imports, links or calls it, and it shares no code with the GPU
path: the arithmetic lives in plain C (``qmm_oracle.c``), this module only
marshals numpy arrays.

What it computes (the pages it follows are cited in ``qmm_oracle.h``):
  * IEEE binary16 / bfloat16 conversions written from the format definitions;
  * Q8_0 / Q4_0 block quantization of fp32 rows (32-weight blocks, and the
    64-weight variants Q8_B64 / Q4_B64) and the row-planar packing;
  * the exact dequantized weights W';
  * MUL_MAT y[n][m] = sum_k W'[m][k] x[n][k] accumulated in binary64, with
    the magnitude sum a[n][m] = sum_k |W'[m][k] x[n][k]| used by tolerances;
  * the SwiGLU epilogue h = Swish(g) * u of the fused gate/up projection;
  * the GGUF-style block records (scale, then codes) <-> packed rows;
  * the integer-activation MUL_MAT (activations quantized to Q8_0 blocks,
    block dot products in integers).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_SRC_TIMING = os.path.join(_HERE, "oracle_timing.c")
_SO = os.environ.get("QMM_ORACLE_LIB") or os.path.join(_HERE, "libqmm_oracle.so")

# Own type numbering (mirrors qmm_oracle.h, not the GPU library's enum).
F32, F16, BF16, Q8_0, Q4_0, Q8_B64, Q4_B64 = 0, 1, 2, 3, 4, 5, 6
# Quantization rules: the default ones, and the pages' symmetric Q4 rule.
RULE_DEFAULT, RULE_Q4_SYM7 = 0, 1

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(out: str = _SO) -> str:
    """Compile the oracle with gcc (plain -O2, contraction off, no fast-math)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, _SRC_TIMING, "-o", tmp, "-lm", "-lpthread"], check=True)
    os.replace(tmp, out)
    return out


_lib_handle = None


def lib() -> ctypes.CDLL:
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO):
            build()
        h = ctypes.CDLL(_SO)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        vp = ctypes.c_void_p
        sz = ctypes.c_size_t
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        h.orc_f32_to_f16_n.argtypes = [f32p, u16p, sz]
        h.orc_f16_to_f32_n.argtypes = [u16p, f32p, sz]
        h.orc_f32_to_bf16_n.argtypes = [f32p, u16p, sz]
        h.orc_bf16_to_f32_n.argtypes = [u16p, f32p, sz]
        for name in ("orc_f32_to_f16_n", "orc_f16_to_f32_n",
                     "orc_f32_to_bf16_n", "orc_bf16_to_f32_n"):
            getattr(h, name).restype = None
        h.orc_quantize_block_q8_0.argtypes = [f32p, u16p, ctypes.POINTER(ctypes.c_int8)]
        h.orc_quantize_block_q8_0.restype = None
        h.orc_quantize_block_q4_0.argtypes = [f32p, u16p, u8p]
        h.orc_quantize_block_q4_0.restype = None
        h.orc_row_size.argtypes = [ci, i64]
        h.orc_row_size.restype = sz
        h.orc_quantize_rows.argtypes = [ci, f32p, i64, i64, u8p, sz]
        h.orc_quantize_rows.restype = ci
        h.orc_quantize_rows_rule.argtypes = [ci, ci, f32p, i64, i64, u8p, sz]
        h.orc_quantize_rows_rule.restype = ci
        h.orc_quantize_block_q4_sym7.argtypes = [f32p, u16p, u8p]
        h.orc_quantize_block_q4_sym7.restype = None
        h.orc_quantize_block_q8_b64.argtypes = [f32p, u16p, ctypes.POINTER(ctypes.c_int8)]
        h.orc_quantize_block_q8_b64.restype = None
        h.orc_quantize_block_q4_b64.argtypes = [f32p, ci, u16p, u8p]
        h.orc_quantize_block_q4_b64.restype = None
        h.orc_dequantize_rows.argtypes = [ci, u8p, sz, i64, i64, f32p]
        h.orc_dequantize_rows.restype = ci
        h.orc_mul_mat_rows.argtypes = [ci, u8p, sz, i64, i64, vp, ci, i64, ci,
                                       i64, i64, f64p, f64p]
        h.orc_mul_mat_rows.restype = ci
        h.orc_mul_mat_pairs.argtypes = [ci, u8p, sz, i64, i64, vp, ci, i64, ci,
                                        i64p, i64p, i64, f64p, f64p]
        h.orc_mul_mat_pairs.restype = ci
        h.orc_mul_mat_q8act_rows.argtypes = [ci, u8p, sz, i64, i64, u8p, sz, i64, i64, i64,
                                             f64p, f64p]
        h.orc_mul_mat_q8act_rows.restype = ci
        h.orc_record_size.argtypes = [ci]
        h.orc_record_size.restype = sz
        h.orc_rows_to_records.argtypes = [ci, u8p, sz, i64, i64, u8p]
        h.orc_rows_to_records.restype = ci
        h.orc_records_to_rows.argtypes = [ci, u8p, i64, i64, u8p, sz]
        h.orc_records_to_rows.restype = ci
        h.orc_time_mul_mat.argtypes = [ci, u8p, sz, i64, i64, vp, ci, i64, ci, ci, f64p, f64p]
        h.orc_time_mul_mat.restype = ctypes.c_double
        h.orc_online_cpus.argtypes = []
        h.orc_online_cpus.restype = ci
        h.orc_swish.argtypes = [ctypes.c_double]
        h.orc_swish.restype = ctypes.c_double
        h.orc_swiglu_n.argtypes = [f64p, f64p, f64p, sz]
        h.orc_swiglu_n.restype = None
        _lib_handle = h
    return _lib_handle


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---- conversions --------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_n(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


def f32_to_bf16_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def bf16_bits_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_bf16_to_f32_n(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


# ---- blocks and rows ------------------------------------------------------

def quantize_block(type_: int, w32) -> tuple[int, np.ndarray]:
    """One 32-weight block -> (fp16 scale bits, codes).  Q8_0 codes are int8
    in [-127, 127]; Q4_0 codes are the stored nibbles in [0, 15]."""
    w = _c(w32, np.float32).reshape(32)
    sb = np.zeros(1, np.uint16)
    if type_ == Q8_0:
        q = np.zeros(32, np.int8)
        lib().orc_quantize_block_q8_0(_ptr(w, ctypes.c_float), _ptr(sb, ctypes.c_uint16),
                                      _ptr(q, ctypes.c_int8))
    elif type_ == Q4_0:
        q = np.zeros(32, np.uint8)
        lib().orc_quantize_block_q4_0(_ptr(w, ctypes.c_float), _ptr(sb, ctypes.c_uint16),
                                      _ptr(q, ctypes.c_uint8))
    elif type_ == "q4_sym7":
        q = np.zeros(32, np.uint8)
        lib().orc_quantize_block_q4_sym7(_ptr(w, ctypes.c_float), _ptr(sb, ctypes.c_uint16),
                                         _ptr(q, ctypes.c_uint8))
    else:
        raise ValueError("quantize_block: type must be Q8_0 or Q4_0")
    return int(sb[0]), q


def quantize_block64(type_: int, w64, rule: int = RULE_DEFAULT) -> tuple[int, np.ndarray]:
    """One 64-weight block -> (fp16 scale bits, codes): Q8_B64 int8 codes, or
    Q4_B64 nibbles in [0, 15] (rule RULE_Q4_SYM7: the amax/7 scale)."""
    w = _c(w64, np.float32).reshape(64)
    sb = np.zeros(1, np.uint16)
    if type_ == Q8_B64:
        q = np.zeros(64, np.int8)
        lib().orc_quantize_block_q8_b64(_ptr(w, ctypes.c_float), _ptr(sb, ctypes.c_uint16),
                                        _ptr(q, ctypes.c_int8))
    elif type_ == Q4_B64:
        q = np.zeros(64, np.uint8)
        lib().orc_quantize_block_q4_b64(_ptr(w, ctypes.c_float), 7 if rule == RULE_Q4_SYM7 else 8,
                                        _ptr(sb, ctypes.c_uint16), _ptr(q, ctypes.c_uint8))
    else:
        raise ValueError("quantize_block64: type must be Q8_B64 or Q4_B64")
    return int(sb[0]), q


def row_size(type_: int, K: int) -> int:
    return int(lib().orc_row_size(type_, K))


def quantize(type_: int, w, pitch: int | None = None, rule: int = RULE_DEFAULT) -> np.ndarray:
    """Quantize fp32 rows w (M x K) into packed rows: uint8 array (M, pitch)."""
    w = _c(w, np.float32)
    M, K = w.shape
    pitch = row_size(type_, K) if pitch is None else pitch
    out = np.zeros((M, pitch), np.uint8)
    rc = lib().orc_quantize_rows_rule(type_, rule, _ptr(w, ctypes.c_float), K, M,
                                      _ptr(out, ctypes.c_uint8), pitch)
    if rc != 0:
        raise ValueError("orc_quantize_rows rejected its arguments")
    return out


def dequantize(type_: int, packed, K: int) -> np.ndarray:
    """Packed rows (M, pitch) uint8 (or dense rows viewed as bytes) -> W' (M, K) f32."""
    packed = _c(packed, np.uint8)
    M, pitch = packed.shape
    out = np.zeros((M, K), np.float32)
    rc = lib().orc_dequantize_rows(type_, _ptr(packed, ctypes.c_uint8), pitch, K, M,
                                   _ptr(out, ctypes.c_float))
    if rc != 0:
        raise ValueError("orc_dequantize_rows rejected its arguments")
    return out


def _x_args(x, x_bf16_bits: bool):
    if x_bf16_bits:
        xa = _c(x, np.uint16)
        return xa, BF16
    xa = _c(x, np.float32)
    return xa, F32


def mul_mat(type_: int, packed, K: int, x, *, x_bf16_bits: bool = False,
            w_to_bf16: bool = False, rows: tuple[int, int] | None = None):
    """y[n][m] = sum_k W'[m][k] x[n][k] in binary64, and a = sum |W' x|.

    packed: (M, pitch) uint8 rows of the weight type; x: (N, K) float32, or
    (N, K) uint16 bf16 bits when x_bf16_bits.  Returns (y, a), each (N, M)
    float64; only rows [m0, m1) are filled when ``rows`` is given (rest 0)."""
    packed = _c(packed, np.uint8)
    M, pitch = packed.shape
    xa, xt = _x_args(x, x_bf16_bits)
    N = xa.shape[0]
    assert xa.shape[1] == K
    m0, m1 = (0, M) if rows is None else rows
    y = np.zeros((N, M), np.float64)
    a = np.zeros((N, M), np.float64)
    rc = lib().orc_mul_mat_rows(type_, _ptr(packed, ctypes.c_uint8), pitch, K, M,
                                xa.ctypes.data_as(ctypes.c_void_p), xt, N,
                                1 if w_to_bf16 else 0, m0, m1,
                                _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_mul_mat_rows rejected its arguments")
    return y, a


def mul_mat_pairs(type_: int, packed, K: int, x, ms, ns, *, x_bf16_bits: bool = False,
                  w_to_bf16: bool = False):
    """The same sums for the (m, n) pairs only; returns (y, a) of shape (count,)."""
    packed = _c(packed, np.uint8)
    M, pitch = packed.shape
    xa, xt = _x_args(x, x_bf16_bits)
    N = xa.shape[0]
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    y = np.zeros(ms.shape, np.float64)
    a = np.zeros(ms.shape, np.float64)
    rc = lib().orc_mul_mat_pairs(type_, _ptr(packed, ctypes.c_uint8), pitch, K, M,
                                 xa.ctypes.data_as(ctypes.c_void_p), xt, N,
                                 1 if w_to_bf16 else 0,
                                 _ptr(ms, ctypes.c_int64), _ptr(ns, ctypes.c_int64), ms.size,
                                 _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_mul_mat_pairs rejected its arguments")
    return y, a


# ---- SwiGLU ---------------------------------------------------------------

def swish(z: float) -> float:
    """Swish(z) = z * sigma(z) in binary64."""
    return float(lib().orc_swish(float(z)))


def swiglu(g, u) -> np.ndarray:
    """h = Swish(g) * u elementwise in binary64 (g, u of the same shape)."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float64)
    lib().orc_swiglu_n(_ptr(g, ctypes.c_double), _ptr(u, ctypes.c_double),
                       _ptr(h, ctypes.c_double), g.size)
    return h


# ---- block-record interchange --------------------------------------------

def record_size(type_: int) -> int:
    return int(lib().orc_record_size(type_))


def rows_to_records(type_: int, rows, K: int) -> np.ndarray:
    """Packed rows (M, pitch) uint8 -> records, uint8 (M * K/32 * record_size,)."""
    rows = _c(rows, np.uint8)
    M, pitch = rows.shape
    out = np.zeros(M * (K // 32) * record_size(type_), np.uint8)
    rc = lib().orc_rows_to_records(type_, _ptr(rows, ctypes.c_uint8), pitch, K, M,
                                   _ptr(out, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("orc_rows_to_records rejected its arguments")
    return out


def records_to_rows(type_: int, records, K: int, M: int, pitch: int | None = None) -> np.ndarray:
    """Records -> packed rows (M, pitch) uint8, padding zero."""
    records = _c(records, np.uint8).ravel()
    pitch = row_size(type_, K) if pitch is None else pitch
    assert records.size == M * (K // 32) * record_size(type_)
    out = np.empty((M, pitch), np.uint8)
    rc = lib().orc_records_to_rows(type_, _ptr(records, ctypes.c_uint8), K, M,
                                   _ptr(out, ctypes.c_uint8), pitch)
    if rc != 0:
        raise ValueError("orc_records_to_rows rejected its arguments")
    return out


# ---- integer-activation MUL_MAT --------------------------------------------

def mul_mat_q8act(type_: int, packed, K: int, xq, rows: tuple[int, int] | None = None):
    """y[n][m] = sum_b Delta_w Delta_x sum_i q_i qx_i (integer block sums,
    binary64 over blocks) and a = sum_b |block term|; xq: (N, pitch) Q8_0 rows
    of the activations.  Returns (y, a), each (N, M) float64."""
    packed = _c(packed, np.uint8)
    xq = _c(xq, np.uint8)
    M, pitch = packed.shape
    N, x_pitch = xq.shape
    m0, m1 = (0, M) if rows is None else rows
    y = np.zeros((N, M), np.float64)
    a = np.zeros((N, M), np.float64)
    rc = lib().orc_mul_mat_q8act_rows(type_, _ptr(packed, ctypes.c_uint8), pitch, K, M,
                                      _ptr(xq, ctypes.c_uint8), x_pitch, N, m0, m1,
                                      _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_mul_mat_q8act_rows rejected its arguments")
    return y, a


# ---- timing (the CPU baseline) ---------------------------------------------

def online_cpus() -> int:
    return int(lib().orc_online_cpus())


def time_mul_mat(type_: int, packed, K: int, x, *, threads: int, reps: int = 3,
                 x_bf16_bits: bool = False) -> float:
    """Median wall seconds of `reps` runs of the oracle's MUL_MAT over all
    rows of packed, rows split over `threads` POSIX threads."""
    packed = _c(packed, np.uint8)
    M, pitch = packed.shape
    xa, xt = _x_args(x, x_bf16_bits)
    N = xa.shape[0]
    y = np.zeros((N, M), np.float64)
    a = np.zeros((N, M), np.float64)
    t = lib().orc_time_mul_mat(type_, _ptr(packed, ctypes.c_uint8), pitch, K, M,
                               xa.ctypes.data_as(ctypes.c_void_p), xt, N, threads, reps,
                               _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if t < 0:
        raise ValueError("orc_time_mul_mat rejected its arguments")
    return float(t)
