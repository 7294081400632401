"""The tiled weight layout of the small-batch GEMV (q8_pack_tile16), on the CPU.

"Filling in the blanks: Inference using Phobos", section GPU Performance Heisenbugs, stores
the decode weights eight columns side by side, which makes a warp's loads span full
128-byte lines.
The pack is a pure permutation with zero padding, checked here element by element
against the layout built independently with numpy reshapes.
"""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_quantized_weight_q8_amd", "libq8gemv.so")
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARG, ERR_LAUNCH, ERR_OVERLAP = range(7)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libq8gemv.so not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    L.q8_pack_tile16.argtypes = [P, P, I64, I64, P, P]
    L.q8_tile16_sizes.argtypes = [I64, I64, ctypes.POINTER(I64), ctypes.POINTER(I64)]
    L.q8_gemv_batch_layout.argtypes = [ctypes.c_int, P, P, P, P, P, P, I64, I64, I64, P]
    L.q8g_batch_tiled_streams.argtypes = [I64, I64, ctypes.POINTER(ctypes.c_int)]
    return L


def sizes(lib, n, k):
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    assert lib.q8_tile16_sizes(n, k, ctypes.byref(cb), ctypes.byref(sb)) == OK
    return cb.value, sb.value


def expected_layout(qw, dw):
    """Codes: [tile][step][chunk c][row j][16 bytes]; scales: [tile][block][row j]."""
    n, k = qw.shape
    t = -(-n // 16)
    s = -(-k // 64)
    pq = np.zeros((16 * t, 64 * s), np.int8)
    pq[:n, :k] = qw
    codes = pq.reshape(t, 16, s, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    pd = np.zeros((16 * t, k // 32), np.uint16)
    pd[:n] = dw
    scales = pd.reshape(t, 16, k // 32).transpose(0, 2, 1).reshape(-1)
    return codes, scales


@pytest.mark.parametrize("n,k", [(1, 32), (16, 64), (17, 96), (37, 1024), (300, 2048 + 32), (33, 5120)])
def test_pack_matches_layout(lib, n, k):
    g = np.random.default_rng(n * 1000 + k)
    qw = g.integers(-127, 128, (n, k), dtype=np.int8)
    dw = g.integers(0, 1 << 16, (n, k // 32), dtype=np.uint16)
    cb, sb = sizes(lib, n, k)
    codes = np.full(cb, 99, np.int8)  # poison: every byte must be written
    scales = np.full(sb // 2, 0xABCD, np.uint16)
    assert lib.q8_pack_tile16(qw.ctypes.data, dw.ctypes.data, n, k, codes.ctypes.data, scales.ctypes.data) == OK
    ec, es = expected_layout(qw, dw)
    assert cb == ec.size and sb == 2 * es.size
    assert np.array_equal(codes, ec)
    assert np.array_equal(scales, es)
    # one KiB per 16-row step: lane l of a wave reads bytes [16 l, 16 l + 16), row l % 16
    # of the tile, columns 16 (l / 16) .. +15 of the step
    t, s, lane = 0, (k - 1) // 64, 37
    j, c = lane % 16, lane // 16
    chunk = codes[(t * (-(-k // 64)) + s) * 1024 + 16 * lane:][:16]
    cols = np.arange(64 * s + 16 * c, 64 * s + 16 * c + 16)
    want = np.where(cols < k, qw[min(j, n - 1), np.minimum(cols, k - 1)], 0) if j < n else np.zeros(16, np.int8)
    assert np.array_equal(chunk, want.astype(np.int8))


def test_pack_validation(lib):
    buf = np.zeros(64 * 1024, np.int8)
    sc = np.zeros(1024, np.uint16)
    p, d = buf.ctypes.data, sc.ctypes.data
    assert lib.q8_pack_tile16(p, d, 4, 48, p, d) == ERR_SHAPE  # K % 32
    assert lib.q8_pack_tile16(p, d, -1, 64, p, d) == ERR_SHAPE
    assert lib.q8_pack_tile16(None, None, 0, 64, None, None) == OK  # empty
    assert lib.q8_pack_tile16(None, d, 4, 64, p + 8192, d + 512) == ERR_NULL
    assert lib.q8_pack_tile16(p, d, 4, 64, p + 100, d + 512) == ERR_OVERLAP  # output over the codes
    assert lib.q8_pack_tile16(p, d, 4, 64, p + 8192, d) == ERR_OVERLAP  # scales over the scales
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    assert lib.q8_tile16_sizes(5, 33, ctypes.byref(cb), ctypes.byref(sb)) == ERR_SHAPE
    assert lib.q8_tile16_sizes(5, 96, None, None) == ERR_NULL
    assert sizes(lib, 5, 96) == (16 * 128, 16 * 3 * 2)


def test_layout_validation(lib):
    """Host-side rejects of the layout entry point (nothing is enqueued)."""
    A = 0x7F0000000000
    W, DW, QX, DX, Y = (A + i * 0x10000000 for i in range(5))
    g = lib.q8_gemv_batch_layout
    assert g(2, W, DW, QX, DX, None, Y, 8, 64, 2, None) == ERR_ARG
    assert g(-1, W, DW, QX, DX, None, Y, 8, 64, 2, None) == ERR_ARG
    assert g(1, W, DW, QX, DX, None, Y, 8, 48, 2, None) == ERR_SHAPE
    assert g(1, W, DW, QX, DX, None, Y, 8, 64, 17, None) == ERR_SHAPE
    assert g(1, W + 8, DW, QX, DX, None, Y, 8, 64, 2, None) == ERR_ALIGN
    # the tiled codes of 8 x 64 take 16 x 64 bytes: y just past the row layout's end still overlaps
    assert g(1, W, DW, QX, DX, None, W + 8 * 64, 8, 64, 2, None) == ERR_OVERLAP
    assert g(1, None, None, None, None, None, None, 0, 64, 2, None) == OK


def test_tiled_streams_query(lib):
    """The persistent streaming form: more than 2048 tiles and K of 8 or 16 64-column steps."""
    def q(n, k):
        v = ctypes.c_int(-1)
        assert lib.q8g_batch_tiled_streams(n, k, ctypes.byref(v)) == OK
        return v.value

    assert q(151936, 1024) == 1                         # the 0.8B output head
    assert q(2049 * 16, 1024) == 1 and q(2048 * 16, 1024) == 0 and q(2048 * 16 + 1, 1024) == 1
    assert q(40000, 992) == 1 and q(40000, 960) == 0    # 16 steps, 15 steps
    assert q(40000, 512) == 1 and q(40000, 480) == 1 and q(40000, 448) == 0
    assert q(40000, 2048) == 0 and q(40000, 5120) == 0 and q(0, 1024) == 0
    v = ctypes.c_int()
    assert lib.q8g_batch_tiled_streams(40000, 1000, ctypes.byref(v)) == ERR_SHAPE
    assert lib.q8g_batch_tiled_streams(-1, 1024, ctypes.byref(v)) == ERR_SHAPE
    assert lib.q8g_batch_tiled_streams(40000, 1024, None) == ERR_NULL
