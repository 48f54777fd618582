"""Pins for the oracle's block-record interchange (not GPU).

"Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §6.1:
a Q4_0 block is one FP16 scale (2 bytes) and 32 4-bit values (16 bytes),
18 bytes; §3.2: the tensor data of a GGUF file is an aligned array.  The
records are those blocks back to back in row-major order, scale first
(little endian), then the codes (Q4_0: byte j = nib_j | nib_{j+16} << 4;
Q8_0: 32 int8 bytes).

Pinned by: the hand-worked blocks of tests/golden (their fp16 scale bits and
packed bytes must appear verbatim, in that order, in each record), the
record sizes the pages print, an independent decode of the records (numpy
float16 scale times the codes) against the oracle's dequantized rows, and
round trips through padded pitches.
"""
import numpy as np

from golden_io import read_blocks


def test_record_sizes(orc):
    assert orc.record_size(orc.Q4_0) == 18
    assert orc.record_size(orc.Q8_0) == 34
    assert orc.record_size(orc.F16) == 0


def _golden_row(orc, type_, fixture):
    cases = read_blocks(fixture)
    w = np.concatenate([c["w"] for c in cases])[None, :]
    return cases, orc.quantize(type_, w), w.shape[1]


def test_q4_0_records_hold_the_hand_worked_blocks(orc):
    cases, rows, K = _golden_row(orc, orc.Q4_0, "q4_0_blocks.txt")
    rec = orc.rows_to_records(orc.Q4_0, rows, K).reshape(-1, 18)
    assert rec.shape[0] == len(cases)
    for i, c in enumerate(cases):
        assert int(rec[i, 0]) | int(rec[i, 1]) << 8 == c["scale"], c["name"]
        assert rec[i, 2:].tobytes() == c["bytes"], c["name"]


def test_q8_0_records_hold_the_hand_worked_blocks(orc):
    cases, rows, K = _golden_row(orc, orc.Q8_0, "q8_0_blocks.txt")
    rec = orc.rows_to_records(orc.Q8_0, rows, K).reshape(-1, 34)
    for i, c in enumerate(cases):
        assert int(rec[i, 0]) | int(rec[i, 1]) << 8 == c["scale"], c["name"]
        assert np.array_equal(rec[i, 2:].view(np.int8).astype(np.int64), c["codes"]), c["name"]


def _decode_records(type_q4, rec_bytes, M, K):
    """Values of the records straight from the block definition."""
    rs = 18 if type_q4 else 34
    rec = rec_bytes.reshape(M, K // 32, rs)
    scale = rec[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    if type_q4:
        b = rec[:, :, 2:].astype(np.int64)
        codes = np.concatenate([b & 15, b >> 4], axis=2) - 8          # elements j, then j + 16
    else:
        codes = rec[:, :, 2:].copy().view(np.int8).astype(np.int64)
    return (scale[:, :, None] * codes).reshape(M, K)


def test_records_decode_to_the_dequantized_rows(orc):
    rng = np.random.default_rng(11)
    for type_, q4 in ((orc.Q4_0, True), (orc.Q8_0, False)):
        for M, K in ((3, 32), (5, 96), (17, 2048), (2, 5632)):
            w = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
            rows = orc.quantize(type_, w)
            rec = orc.rows_to_records(type_, rows, K)
            assert rec.size == M * K // 32 * orc.record_size(type_)
            got = _decode_records(q4, rec, M, K)
            assert np.array_equal(got, orc.dequantize(type_, rows, K).astype(np.float64))


def test_round_trips_and_padding(orc):
    rng = np.random.default_rng(12)
    for type_ in (orc.Q4_0, orc.Q8_0):
        M, K = 9, 160
        rs = orc.row_size(type_, K)
        rows = orc.quantize(type_, (rng.standard_normal((M, K)) * 0.02).astype(np.float32), pitch=rs + 32)
        rec = orc.rows_to_records(type_, rows, K)
        back = orc.records_to_rows(type_, rec, K, M, pitch=rs + 32)
        assert np.array_equal(back, rows)            # quantize leaves the padding zero
        dirty = rows.copy()
        dirty[:, rs:] = 0xAB                         # pitch padding is not part of a record
        dirty[:, 2 * K // 32: 16] = 0xCD             # nor the gap before the codes
        assert np.array_equal(orc.rows_to_records(type_, dirty, K), rec)
        assert np.array_equal(orc.rows_to_records(type_, orc.records_to_rows(type_, rec, K, M), K), rec)
    # the config row sizes equal whole records: the same bytes per row either way
    for K in (512, 2048, 5632):
        assert orc.row_size(orc.Q4_0, K) == K // 32 * 18
        assert orc.row_size(orc.Q8_0, K) == K // 32 * 34
