"""The C-ABI boundary on the CPU (no compute calls): libqmm.so loads, exports
every entry point include/qmm.h declares, sizes rows as the header states, and
rejects malformed descriptors before enqueueing anything.

Validation runs on the host before any HIP call, so the rejected calls below
never reach the GPU.  They use fake device addresses, so they only run where
no GPU is visible (the GPU tests exercise the accepted paths with real
memory)."""
import ctypes
import os
import re
import subprocess

import pytest

from quantized_matmul_ggml_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QMM_API\s+[^;(]*?\b(qmm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(qmm_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", qmm_lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qmm_\w+)", out))
    assert set(_declared()) <= exported
    assert exported == set(_declared()), "only the C ABI is exported"
    for name in _declared():
        assert getattr(qmm_lib.lib(), name) is not None


def test_row_size_closed_forms(qmm_lib):
    rs = qmm_lib.row_size
    for K in (256, 512, 2048, 5632, 32768):
        assert rs(B.Q8_0, K) == 17 * K // 16     # 34 bytes per 32 weights
        assert rs(B.Q4_0, K) == 9 * K // 16      # 18 bytes per 32 weights
    assert rs(B.Q4_0, 32) == 32 and rs(B.Q8_0, 32) == 48
    assert rs(B.Q4_0, 96) == 64 and rs(B.Q8_0, 96) == 112
    assert rs(B.F16, 7) == 14 and rs(B.F32, 7) == 28 and rs(B.BF16, 3) == 6
    assert rs(B.Q4_0, 33) == 0 and rs(B.Q8_0, -32) == 0 and rs(99, 32) == 0
    assert rs(B.Q4_0, 0) == 0


def test_row_size_matches_oracle(qmm_lib, orc):
    for K in (32, 64, 96, 160, 512, 2048, 5632, 4096 + 32):
        assert qmm_lib.row_size(B.Q8_0, K) == orc.row_size(orc.Q8_0, K)
        assert qmm_lib.row_size(B.Q4_0, K) == orc.row_size(orc.Q4_0, K)


def test_strerror_covers_every_status(qmm_lib):
    seen = set()
    for s in range(-8, 1):
        t = qmm_lib.strerror(s)
        assert t and t not in seen
        seen.add(t)
    assert "unknown" in qmm_lib.strerror(-99)


no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake device addresses: host-only validation checks run where no GPU is visible")

BASE = 0x7F0000000000        # fake, 4 KiB aligned device addresses
W_ADDR, X_ADDR, Y_ADDR = BASE, BASE + (1 << 32), BASE + (2 << 32)


def _w(type_=B.Q4_0, K=2048, M=64, addr=W_ADDR, pitch=None):
    return B.make_desc(type_, K, M, pitch if pitch is not None else B.row_size(type_, K), addr)


def _x(type_=B.F32, K=2048, N=1, addr=X_ADDR):
    es = 4 if type_ == B.F32 else 2
    return B.make_desc(type_, K, N, K * es, addr)


def _y(M=64, N=1, addr=Y_ADDR):
    return B.make_desc(B.F32, M, N, M * 4, addr)


@no_gpu
@pytest.mark.parametrize("case,expect", [
    ("null_w", B.ERR_NULL), ("null_data", B.ERR_NULL), ("w_f32", B.ERR_TYPE),
    ("x_bf16", B.ERR_TYPE), ("y_f16", B.ERR_TYPE), ("k_mismatch", B.ERR_SHAPE),
    ("k_not_32", B.ERR_SHAPE), ("n_over_8", B.ERR_SHAPE), ("y_rows", B.ERR_SHAPE),
    ("y_tokens", B.ERR_SHAPE), ("w_misaligned", B.ERR_LAYOUT), ("pitch_small", B.ERR_LAYOUT),
    ("pitch_unaligned", B.ERR_LAYOUT), ("nb0_quant", B.ERR_LAYOUT), ("nb0_dense", B.ERR_LAYOUT),
    ("x_misaligned", B.ERR_LAYOUT), ("three_dims", B.ERR_UNSUPPORTED),
    ("ne2", B.ERR_UNSUPPORTED), ("alias_y_w", B.ERR_ALIAS), ("alias_y_x", B.ERR_ALIAS),
    ("too_large", B.ERR_UNSUPPORTED), ("bad_type", B.ERR_TYPE), ("neg_ne", B.ERR_SHAPE),
])
def test_gemv_rejects(qmm_lib, case, expect):
    w, x, y = _w(), _x(), _y()
    if case == "null_w": w = None
    elif case == "null_data": x.data = None
    elif case == "w_f32": w = B.make_desc(B.F32, 2048, 64, 8192, W_ADDR)
    elif case == "x_bf16": x = _x(B.BF16)
    elif case == "y_f16": y = B.make_desc(B.F16, 64, 1, 128, Y_ADDR)
    elif case == "k_mismatch": x = _x(K=1024)
    elif case == "k_not_32": w = B.make_desc(B.Q4_0, 2040, 64, 1152, W_ADDR); x = _x(K=2040)
    elif case == "n_over_8": x = _x(N=9); y = _y(N=9)
    elif case == "y_rows": y = _y(M=63)
    elif case == "y_tokens": y = _y(N=2)
    elif case == "w_misaligned": w = _w(addr=W_ADDR + 8)
    elif case == "pitch_small": w = _w(pitch=1136)
    elif case == "pitch_unaligned": w = _w(pitch=1160)
    elif case == "nb0_quant": w.nb[0] = 18
    elif case == "nb0_dense": x.nb[0] = 8
    elif case == "x_misaligned": x.data = X_ADDR + 2
    elif case == "three_dims": w.n_dims = 3
    elif case == "ne2": w.ne[2] = 2
    elif case == "alias_y_w": y.data = W_ADDR + 1152 * 10
    elif case == "alias_y_x": y.data = X_ADDR + 4 * 100
    elif case == "too_large": w = _w(K=65536, M=4); x = _x(K=65536); y = _y(M=4)
    elif case == "bad_type": w.type = 9
    elif case == "neg_ne": w.ne[1] = -1
    assert B.call_raw("qmm_gemv", w, x, y) == expect


@no_gpu
@pytest.mark.parametrize("case,expect", [
    ("x_f32", B.ERR_TYPE), ("w_f32", B.ERR_TYPE), ("w_f16_k_not_32", B.ERR_UNSUPPORTED),
    ("x_unaligned_pitch", B.ERR_LAYOUT),
    ("x_misaligned", B.ERR_LAYOUT), ("alias", B.ERR_ALIAS), ("k_mismatch", B.ERR_SHAPE),
])
def test_gemm_rejects(qmm_lib, case, expect):
    w, x, y = _w(), _x(B.BF16, N=512), _y(N=512)
    if case == "x_f32": x = _x(B.F32, N=512)
    elif case == "w_f32": w = B.make_desc(B.F32, 2048, 64, 8192, W_ADDR)
    elif case == "w_f16_k_not_32":
        w = B.make_desc(B.F16, 2056, 64, 4112 + 16 - 4112 % 16, W_ADDR); x = _x(B.BF16, K=2056, N=512)
    elif case == "x_unaligned_pitch": x.nb[1] = 2048 * 2 + 2
    elif case == "x_misaligned": x.data = X_ADDR + 8
    elif case == "alias": y.data = X_ADDR
    elif case == "k_mismatch": x = _x(B.BF16, K=2080, N=512)
    assert B.call_raw("qmm_gemm", w, x, y) == expect


def _ws_call(w, x, y, ws, nbytes):
    import ctypes
    return B.lib().qmm_gemm_ws(*(ctypes.byref(d) if d is not None else None for d in (w, x, y)),
                               ctypes.c_void_p(ws), nbytes, ctypes.c_void_p(0))


def _gemm_pair(M, K, N):
    return _w(B.Q4_0, K=K, M=M), _x(B.BF16, K=K, N=N)


@no_gpu
def test_gemm_workspace_size(qmm_lib):
    """K is split only where the launch's cost estimate says it pays (few
    output tiles for 256 compute units, long K): into ranges that are
    multiples of 512 of K and at least that long, at most one workgroup per
    compute unit; the workspace is one M x N float slab per range (M rounded
    up to 4)."""
    import ctypes
    size = lambda M, K, N: B.lib().qmm_gemm_workspace_size(*(ctypes.byref(d) for d in _gemm_pair(M, K, N)))
    assert size(5632, 2048, 512) == 0             # 176 tiles: no split
    assert size(2048, 2048, 2048) == 0            # 256 tiles
    assert size(2048, 2048, 512) == 0             # 64 tiles, 32 steps: the partial sums cost more
    assert size(4096, 2048, 512) == 0             # 128 tiles
    assert size(100, 512, 5) == 0                 # 8 K-steps: too short to split
    assert size(2048, 5632, 512) == 4 * 512 * 2048 * 4     # 64 tiles, 88 steps: 24, 24, 24, 16
    assert size(1024, 4096, 512) == 4 * 512 * 1024 * 4     # 32 tiles, 64 steps: 4 x 16
    assert size(256, 2048, 512) == 4 * 512 * 256 * 4       # 8 tiles, 32 steps: 4 x 8
    assert size(300, 4160, 77) == 5 * 77 * 300 * 4         # 65 steps in ranges of 16
    assert size(1002, 2048, 3) == 4 * 3 * 1004 * 4         # rows rounded up to 4 floats
    assert B.lib().qmm_gemm_workspace_size(None, None) == 0
    # operands qmm_gemm_ws refuses get no size
    w, x = _gemm_pair(2048, 5632, 512)
    for bad_w, bad_x in ((B.make_desc(B.F32, 5632, 2048, 4 * 5632, W_ADDR), x),   # f32 weights
                         (w, _x(B.F32, K=5632, N=512)),                            # f32 tokens
                         (w, _x(B.BF16, K=2048, N=512))):                          # K mismatch
        assert B.lib().qmm_gemm_workspace_size(ctypes.byref(bad_w), ctypes.byref(bad_x)) == 0


@no_gpu
def test_gemm_ws_rejects(qmm_lib):
    w, x = _gemm_pair(64, 2048, 512)
    y = _y(M=64, N=512)
    ws_addr = BASE + (3 << 32)
    need = 4 * 512 * 64 * 4
    assert _ws_call(w, x, y, ws_addr + 8, need) == B.ERR_LAYOUT      # misaligned workspace
    assert _ws_call(w, x, y, Y_ADDR - 4096, need) == B.ERR_ALIAS     # runs into y
    assert _ws_call(w, x, y, W_ADDR, need) == B.ERR_ALIAS            # w's rows
    assert _ws_call(w, _x(B.F32, N=512), y, ws_addr, need) == B.ERR_TYPE   # operand checks first
    assert _ws_call(None, x, y, ws_addr, need) == B.ERR_NULL


def _gemm_batch_call(triples, count=None):
    import ctypes
    items = [B.QmmGemmItem(*(ctypes.pointer(d) if d is not None else None for d in t)) for t in triples]
    arr = (B.QmmGemmItem * max(1, len(items)))(*items)
    n = len(items) if count is None else count
    return B.lib().qmm_gemm_batch(arr, n, ctypes.c_void_p(0))


@no_gpu
def test_gemm_batch_rejects(qmm_lib):
    w0, w1 = _w(M=64), _w(M=32, addr=W_ADDR + (1 << 24))
    x = _x(B.BF16, N=512)
    y0, y1 = _y(M=64, N=512), _y(M=32, N=512, addr=Y_ADDR + (1 << 24))
    assert B.lib().qmm_gemm_batch(None, 1, None) == B.ERR_NULL
    assert _gemm_batch_call([(w0, x, y0)], count=0) == B.ERR_SHAPE
    assert _gemm_batch_call([(w0, x, y0)] * 9) == B.ERR_SHAPE
    assert _gemm_batch_call([(w0, x, y0), (_w(B.Q8_0, M=32, addr=W_ADDR + (1 << 24)), x, y1)]) == B.ERR_TYPE
    wk = _w(K=1024, M=32, addr=W_ADDR + (1 << 24))
    assert _gemm_batch_call([(w0, x, y0), (wk, _x(B.BF16, K=1024, N=512), y1)]) == B.ERR_SHAPE
    assert _gemm_batch_call([(w0, x, y0), (w1, _x(B.BF16, N=256), _y(M=32, N=256, addr=y1.data))]) == B.ERR_SHAPE
    assert _gemm_batch_call([(w0, x, y0), (w1, _x(B.F32, N=512), y1)]) == B.ERR_TYPE
    # an output overlapping another item's output or weights
    assert _gemm_batch_call([(w0, x, y0), (w1, x, _y(M=32, N=512, addr=Y_ADDR + 64))]) == B.ERR_ALIAS
    assert _gemm_batch_call([(w0, x, y0), (w1, x, _y(M=32, N=512, addr=W_ADDR))]) == B.ERR_ALIAS
    assert _gemm_batch_call([(w0, x, None)]) == B.ERR_NULL


@no_gpu
def test_gemm_swiglu_rejects(qmm_lib):
    U_ADDR = BASE + (3 << 32)
    g, u, x, h = _w(), _w(addr=U_ADDR), _x(B.BF16, N=512), _y(N=512)
    call = lambda *d: B.call_raw("qmm_gemm_swiglu", *d)
    assert call(None, u, x, h) == B.ERR_NULL
    assert call(g, B.make_desc(B.Q8_0, 2048, 64, 2176, U_ADDR), x, h) == B.ERR_TYPE   # mixed types
    assert call(g, _w(M=65, addr=U_ADDR), x, h) == B.ERR_SHAPE                       # mixed M
    assert call(g, u, _x(B.F32, N=512), h) == B.ERR_TYPE                             # f32 tokens
    assert call(g, u, _x(B.BF16, K=1024, N=512), h) == B.ERR_SHAPE                   # K mismatch
    assert call(g, u, x, _y(N=512, addr=U_ADDR + 64)) == B.ERR_ALIAS                 # h over w_up
    assert call(g, u, x, _y(N=512, addr=X_ADDR)) == B.ERR_ALIAS                      # h over x
    assert call(_w(M=0, addr=0), _w(M=0, addr=0), x, _y(M=0, N=512, addr=0)) == B.OK


@no_gpu
def test_quantize_and_dequantize_reject(qmm_lib):
    src = B.make_desc(B.F32, 2048, 64, 8192, X_ADDR)
    dst = _w()
    assert B.call_raw("qmm_quantize", None, dst) == B.ERR_NULL
    assert B.call_raw("qmm_quantize", src, B.make_desc(B.F16, 2048, 64, 4096, W_ADDR)) == B.ERR_TYPE
    assert B.call_raw("qmm_quantize", B.make_desc(B.F32, 2048, 63, 8192, X_ADDR), dst) == B.ERR_SHAPE
    assert B.call_raw("qmm_quantize", B.make_desc(B.F32, 2040, 64, 8192, X_ADDR),
                      B.make_desc(B.Q4_0, 2040, 64, 1152, W_ADDR)) == B.ERR_SHAPE
    assert B.call_raw("qmm_quantize", B.make_desc(B.F32, 2048, 64, 8192, W_ADDR + 64), dst) == B.ERR_ALIAS
    assert B.call_raw("qmm_dequantize", dst, B.make_desc(B.F16, 2048, 64, 4096, Y_ADDR)) == B.ERR_TYPE
    assert B.call_raw("qmm_dequantize", B.make_desc(B.F32, 2048, 64, 8192, X_ADDR),
                      B.make_desc(B.F32, 2048, 64, 8192, Y_ADDR)) == B.ERR_TYPE


@no_gpu
def test_quantize_rule_rejects(qmm_lib):
    src = B.make_desc(B.F32, 2048, 64, 8192, X_ADDR)
    call = lambda s, d, r: qmm_lib.lib().qmm_quantize_rule(
        ctypes.byref(s) if s is not None else None, ctypes.byref(d) if d is not None else None, r, None)
    assert call(src, _w(), 2) == B.ERR_UNSUPPORTED                       # unknown rule
    assert call(src, _w(), -1) == B.ERR_UNSUPPORTED
    assert call(src, _w(type_=B.Q8_0), 1) == B.ERR_TYPE                  # amax/7 is a Q4 rule
    assert call(None, _w(), 1) == B.ERR_NULL
    assert call(B.make_desc(B.F32, 2048, 0, 8192, 0), _w(M=0, addr=0), 1) == B.OK


@no_gpu
def test_gemv_batch_rejects(qmm_lib):
    item = lambda **kw: (_w(**{k: v for k, v in kw.items() if k in ("type_", "K", "M", "addr")}), _x(K=kw.get("K", 2048), addr=kw.get("xaddr", X_ADDR)), _y(M=kw.get("M", 64), addr=kw.get("yaddr", Y_ADDR)))
    a = item()
    b = item(addr=W_ADDR + (1 << 28), xaddr=X_ADDR + (1 << 28), yaddr=Y_ADDR + (1 << 28))
    assert B.call_batch_raw([a, b], count=0) == B.ERR_SHAPE
    assert B.call_batch_raw([a] * 9) == B.ERR_SHAPE
    assert B.call_batch_raw([a, (b[0], None, b[2])]) == B.ERR_NULL
    c = (B.make_desc(B.Q8_0, 2048, 64, 2176, W_ADDR + (1 << 28)), b[1], b[2])
    assert B.call_batch_raw([a, c]) == B.ERR_TYPE                     # mixed weight types
    d = (B.make_desc(B.Q4_0, 1024, 64, 576, W_ADDR + (1 << 28)), _x(K=1024, addr=b[1].data), b[2])
    assert B.call_batch_raw([a, d]) == B.ERR_SHAPE                    # mixed K
    e = (b[0], _x(N=2, addr=b[1].data), _y(N=2, addr=b[2].data))
    assert B.call_batch_raw([a, e]) == B.ERR_SHAPE                    # mixed N
    f = (b[0], b[1], _y(addr=a[1].data))                              # output over another item's x
    assert B.call_batch_raw([a, f]) == B.ERR_ALIAS
    g = (b[0], b[1], _y(addr=Y_ADDR + 16))                            # two outputs overlap
    assert B.call_batch_raw([a, g]) == B.ERR_ALIAS
    h = (b[0], _x(K=2048, addr=b[1].data), _y(M=63, addr=b[2].data))
    assert B.call_batch_raw([a, h]) == B.ERR_SHAPE
    # Q8_0 activations: all items or none, and quantized weights only
    xq = lambda addr: B.make_desc(B.Q8_0, 2048, 1, 2176, addr)
    qa = (a[0], xq(X_ADDR), a[2])
    qb = (b[0], xq(X_ADDR + (1 << 28)), b[2])
    assert B.call_batch_raw([qa, b]) == B.ERR_TYPE
    assert B.call_batch_raw([a, qb]) == B.ERR_TYPE
    assert B.call_batch_raw([(B.make_desc(B.F16, 2048, 64, 4096, W_ADDR), xq(X_ADDR), a[2])]) == B.ERR_TYPE
    assert B.call_batch_raw([qa, (b[0], B.make_desc(B.Q8_0, 2048, 1, 2176, X_ADDR + 8), b[2])]) == B.ERR_LAYOUT


@no_gpu
def test_gemv_swiglu_rejects(qmm_lib):
    U_ADDR = BASE + (3 << 32)
    g, u, x, h = _w(), _w(addr=U_ADDR), _x(), _y()
    call = lambda *d: B.call_raw("qmm_gemv_swiglu", *d)
    assert call(None, u, x, h) == B.ERR_NULL
    assert call(g, B.make_desc(B.Q8_0, 2048, 64, 2176, U_ADDR), x, h) == B.ERR_TYPE   # mixed types
    assert call(g, _w(M=65, addr=U_ADDR), x, h) == B.ERR_SHAPE                       # mixed M
    assert call(g, u, _x(N=9), _y(N=9)) == B.ERR_SHAPE                               # N > 8
    assert call(g, u, _x(K=1024), h) == B.ERR_SHAPE                                  # K mismatch
    assert call(g, u, x, _y(addr=U_ADDR + 64)) == B.ERR_ALIAS                        # h over w_up
    assert call(g, u, x, _y(addr=W_ADDR)) == B.ERR_ALIAS                             # h over w_gate
    assert call(g, u, x, _y(addr=X_ADDR)) == B.ERR_ALIAS                             # h over x
    assert call(B.make_desc(B.F32, 2048, 64, 8192, W_ADDR), u, x, h) == B.ERR_TYPE
    assert call(_w(M=0, addr=0), _w(M=0, addr=0), x, _y(M=0, addr=0)) == B.OK        # empty: no launch
    # Q8_0 activations: quantized weights only, same rules otherwise
    xq = B.make_desc(B.Q8_0, 2048, 1, 2176, X_ADDR)
    f16 = lambda addr: B.make_desc(B.F16, 2048, 64, 4096, addr)
    assert call(f16(W_ADDR), f16(U_ADDR), xq, h) == B.ERR_TYPE
    assert call(g, B.make_desc(B.Q8_0, 2048, 64, 2176, U_ADDR), xq, h) == B.ERR_TYPE
    assert call(g, u, B.make_desc(B.Q8_0, 2048, 9, 2176, X_ADDR), _y(N=9)) == B.ERR_SHAPE
    assert call(g, u, B.make_desc(B.Q8_0, 2048, 1, 2176, X_ADDR + 8), h) == B.ERR_LAYOUT
    assert call(g, u, xq, _y(addr=X_ADDR)) == B.ERR_ALIAS


def test_record_size_closed_forms(qmm_lib):
    # one fp16 scale (2 bytes) plus the codes of 32 weights
    assert qmm_lib.record_size(B.Q4_0) == 2 + 16
    assert qmm_lib.record_size(B.Q8_0) == 2 + 32
    for t in (B.F32, B.F16, B.BF16, 99, -1):
        assert qmm_lib.record_size(t) == 0


@no_gpu
def test_record_conversions_reject(qmm_lib):
    R_ADDR = BASE + (4 << 32)
    q = _w()                                             # Q4_0 2048 x 64
    for name, args in (("qmm_records_to_rows", lambda r, t: (r, t)),
                       ("qmm_rows_to_records", lambda r, t: (t, r))):
        call = lambda r, t: getattr(qmm_lib.lib(), name)(*[
            ctypes.c_void_p(r) if isinstance(r, int) else (ctypes.byref(r) if r is not None else None)
            for r in args(r, t)], None)
        assert call(R_ADDR, None) == B.ERR_NULL
        assert call(0, q) == B.ERR_NULL                  # NULL records, non-empty tensor
        assert call(R_ADDR + 8, q) == B.ERR_LAYOUT       # records not 16-byte aligned
        assert call(R_ADDR, B.make_desc(B.F16, 2048, 64, 4096, W_ADDR)) == B.ERR_TYPE
        assert call(R_ADDR, _w(pitch=1160)) == B.ERR_LAYOUT
        assert call(W_ADDR + 1152 * 63, q) == B.ERR_ALIAS   # records start inside the last row
        assert call(W_ADDR - 1024, q) == B.ERR_ALIAS        # records run into the first row
        assert call(R_ADDR, _w(M=0, addr=0)) == B.OK        # empty: nothing enqueued
        assert call(0, _w(M=0, addr=0)) == B.OK


@no_gpu
def test_gemv_q8_activations_reject(qmm_lib):
    xq = B.make_desc(B.Q8_0, 2048, 1, 2176, X_ADDR)
    assert B.call_raw("qmm_gemv", B.make_desc(B.F16, 2048, 64, 4096, W_ADDR), xq, _y()) == B.ERR_TYPE
    assert B.call_raw("qmm_gemv", _w(), B.make_desc(B.Q8_0, 2048, 9, 2176, X_ADDR), _y(N=9)) == B.ERR_SHAPE
    assert B.call_raw("qmm_gemv", _w(), B.make_desc(B.Q8_0, 2048, 2, 2184, X_ADDR), _y(N=2)) == B.ERR_LAYOUT
    assert B.call_raw("qmm_gemv", _w(), B.make_desc(B.Q8_0, 1024, 1, 1088, X_ADDR), _y()) == B.ERR_SHAPE
    assert B.call_raw("qmm_gemv", _w(), xq, _y(addr=X_ADDR + 64)) == B.ERR_ALIAS
    assert B.call_raw("qmm_gemv", _w(K=65536, M=4), B.make_desc(B.Q8_0, 65536, 1, 69632, X_ADDR),
                      _y(M=4)) == B.ERR_UNSUPPORTED


@no_gpu
def test_empty_operands_enqueue_nothing(qmm_lib):
    # zero rows / zero tokens are valid and launch no kernel (so they are safe
    # without a GPU); NULL data is allowed for empty tensors
    assert B.call_raw("qmm_gemv", _w(M=0, addr=0), _x(), _y(M=0, addr=0)) == B.OK
    assert B.call_raw("qmm_gemm", _w(), B.make_desc(B.BF16, 2048, 0, 4096, 0),
                      B.make_desc(B.F32, 64, 0, 256, 0)) == B.OK
    assert B.call_raw("qmm_quantize", B.make_desc(B.F32, 2048, 0, 8192, 0),
                      B.make_desc(B.Q4_0, 2048, 0, 1152, 0)) == B.OK


def test_row_size_64_blocks(qmm_lib, orc):
    rs = qmm_lib.row_size
    for K in (64, 128, 2048, 5632, 4096 + 64):
        assert rs(B.Q8_B64, K) == orc.row_size(orc.Q8_B64, K)
        assert rs(B.Q4_B64, K) == orc.row_size(orc.Q4_B64, K)
    for K in (512, 2048, 32768):                   # no padding when K % 512 == 0
        assert rs(B.Q8_B64, K) == K // 32 + K      # 66 bytes per 64 weights
        assert rs(B.Q4_B64, K) == K // 32 + K // 2   # 34 bytes per 64 weights
    assert rs(B.Q4_B64, 96) == 0 and rs(B.Q8_B64, 32) == 0   # K % 64 != 0
    assert qmm_lib.record_size(B.Q4_B64) == 0 and qmm_lib.record_size(B.Q8_B64) == 0


@no_gpu
def test_64_block_types_reject(qmm_lib):
    w = B.make_desc(B.Q4_B64, 2048, 64, 1088, W_ADDR)
    # K not a multiple of 64
    assert B.call_raw("qmm_gemv", B.make_desc(B.Q4_B64, 2080, 64, 1104, W_ADDR), _x(K=2080), _y()) == B.ERR_SHAPE
    assert B.call_raw("qmm_quantize", B.make_desc(B.F32, 2080, 64, 8320, X_ADDR),
                      B.make_desc(B.Q8_B64, 2080, 64, 2176, W_ADDR)) == B.ERR_SHAPE
    # the integer-activation path takes them too, but its activations stay Q8_0
    xq = B.make_desc(B.Q8_B64, 2048, 1, 2112, X_ADDR)
    assert B.call_raw("qmm_gemv", w, xq, _y()) == B.ERR_TYPE
    # no GGUF record for 64-blocks
    R_ADDR = BASE + (4 << 32)
    assert qmm_lib.lib().qmm_rows_to_records(ctypes.byref(w), ctypes.c_void_p(R_ADDR), None) == B.ERR_TYPE
    # the amax/7 rule is a Q4 rule: accepted for Q4_B64 (nothing enqueued for
    # an empty tensor), rejected for Q8_B64
    call = lambda s, d, r: qmm_lib.lib().qmm_quantize_rule(ctypes.byref(s), ctypes.byref(d), r, None)
    assert call(B.make_desc(B.F32, 2048, 0, 8192, 0), B.make_desc(B.Q4_B64, 2048, 0, 1088, 0), 1) == B.OK
    assert call(B.make_desc(B.F32, 2048, 64, 8192, X_ADDR), B.make_desc(B.Q8_B64, 2048, 64, 2112, W_ADDR), 1) == B.ERR_TYPE
    # a pitch below the 64-block row size
    assert B.call_raw("qmm_gemv", B.make_desc(B.Q4_B64, 2048, 64, 1072, W_ADDR), _x(), _y()) == B.ERR_LAYOUT


@no_gpu
def test_sizes_beyond_the_address_space_are_refused(qmm_lib):
    """Element counts above 2^48, spans that overflow 64 bits or wrap the
    address space: QMM_ERR_UNSUPPORTED before any arithmetic can overflow."""
    assert qmm_lib.row_size(B.Q4_0, 1 << 49) == 0 and qmm_lib.row_size(B.F32, 1 << 50) == 0
    x, y = _x(), _y()
    huge_rows = _w(M=1 << 50)
    assert B.call_raw("qmm_gemv", huge_rows, x, y) == B.ERR_UNSUPPORTED
    wide_pitch = _w(M=1 << 20, pitch=1 << 47)          # (M - 1) * nb[1] beyond 2^62
    assert B.call_raw("qmm_gemv", wide_pitch, x, y) == B.ERR_UNSUPPORTED
    wrapping = _w(addr=(1 << 64) - 4096)               # the span runs past the top of the address space
    assert B.call_raw("qmm_gemv", wrapping, x, y) == B.ERR_UNSUPPORTED
    # 2^31 blocks: the record count is refused, not overflowed
    rec = B.lib().qmm_rows_to_records(ctypes.byref(_w(K=1 << 20, M=1 << 16)),
                                      ctypes.c_void_p(BASE + (1 << 46)), None)
    assert rec == B.ERR_UNSUPPORTED
