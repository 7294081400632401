"""The C-ABI library without a GPU: exports and host-side validation.

Every call here fails validation on the host before anything is enqueued, so the
fake device addresses passed in are never dereferenced and no kernel is launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_quantized_weight_q8_amd", "libq8gemv.so")
INCLUDE = os.path.join(ROOT, "include")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARG, ERR_LAUNCH, ERR_OVERLAP = range(7)


def declared_functions():
    names = []
    for fn in sorted(os.listdir(INCLUDE)):
        if fn.endswith(".h"):
            text = open(os.path.join(INCLUDE, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libq8gemv.so not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64

    class Part(ctypes.Structure):
        _fields_ = [("w", P), ("dw", P), ("n", I64), ("y", P), ("residual", P)]

    L.Part = Part
    L.q8_quantize_act.argtypes = [P, P, P, I64, P]
    L.q8_gemv.argtypes = [P, P, P, P, P, P, I64, I64, P]
    L.bf16_gemv.argtypes = [P, P, P, P, I64, I64, P]
    L.f16_gemv.argtypes = [P, P, P, P, I64, I64, P]
    L.q8_gemv_batch.argtypes = [P, P, P, P, P, P, I64, I64, I64, P]
    L.gemv_stacked.argtypes = [ctypes.c_int, ctypes.POINTER(Part), ctypes.c_int, P, P, I64, P]
    L.q8_rmsnorm_quantize_act.argtypes = [P, P, ctypes.c_float, P, P, I64, P]
    L.q8_silu_mul_quantize_act.argtypes = [P, P, P, I64, P]
    L.gemv_stacked_rmsnorm.argtypes = [ctypes.POINTER(Part), ctypes.c_int, P, P, ctypes.c_float, I64, P]
    L.q8_gemv_silu_mul.argtypes = [P, P, P, P, P, I64, I64, P]
    L.q8_gateup_silu_quantize.argtypes = [P, P, P, P, I64, P, P, I64, P, P, P]
    L.q8_rmsnorm_quantize_act_batch.argtypes = [P, P, ctypes.c_float, P, P, I64, I64, P]
    L.q8_silu_mul_quantize_act_batch.argtypes = [P, P, P, I64, I64, P]
    L.q8_gateup_rmsnorm_silu_quantize.argtypes = [P, P, P, P, I64, P, P, ctypes.c_float, I64, P, P, P]
    L.q8_gateup_silu.argtypes = [P, P, P, P, I64, P, P, I64, P, P]
    L.q8_gateup_rmsnorm_silu.argtypes = [P, P, P, P, I64, P, P, ctypes.c_float, I64, P, P]
    L.q8g_status_str.argtypes = [ctypes.c_int]
    L.q8g_status_str.restype = ctypes.c_char_p
    L.q8g_probe_read.argtypes = [P, I64, P, P]
    L.q8g_flush.argtypes = [P, I64, ctypes.c_uint32, P]
    L.ptq1_rotate_quantize_act.argtypes = [P, P, P, P, I64, P]
    L.ptq1_gemv.argtypes = [P, P, P, P, P, I64, I64, P]
    L.q8g_gemv_config.argtypes = [ctypes.c_int, I64, I64, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    return L


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    for expected in ("q8_quantize_act", "q8_gemv", "q8_gemv_batch", "bf16_gemv", "f16_gemv", "gemv_stacked",
                     "q8g_status_str", "q8_rmsnorm_quantize_act", "q8_silu_mul_quantize_act",
                     "gemv_stacked_rmsnorm", "q8_gemv_silu_mul", "q8_gateup_silu_quantize",
                     "q8_gateup_rmsnorm_silu_quantize", "q8_gateup_silu", "q8_gateup_rmsnorm_silu",
                     "q8_rmsnorm_quantize_act_batch",
                     "q8_silu_mul_quantize_act_batch", "q8g_probe_read", "q8g_flush",
                     "ptq1_rotate_quantize_act", "ptq1_gemv"):
        assert expected in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings(lib):
    for s in range(7):
        assert lib.q8g_status_str(s)
    assert lib.q8g_status_str(99) == b"unknown status"


# fake, 256-byte aligned, non-overlapping device addresses (never dereferenced)
A = 0x7F0000000000
W, DW, QX, DX, Y, R, X = (A + i * 0x10000000 for i in range(7))


def test_quantize_validation(lib):
    q = lib.q8_quantize_act
    assert q(X, QX, DX, 33, None) == ERR_SHAPE
    assert q(X, QX, DX, -32, None) == ERR_SHAPE
    assert q(None, None, None, 0, None) == OK  # empty: nothing enqueued
    assert q(None, QX, DX, 64, None) == ERR_NULL
    assert q(X + 4, QX, DX, 64, None) == ERR_ALIGN
    assert q(X, QX + 1, DX, 64, None) == ERR_ALIGN
    assert q(X, QX, DX + 1, 64, None) == ERR_ALIGN
    assert q(X, X + 16, DX, 64, None) == ERR_OVERLAP  # codes inside x
    assert q(X, QX, QX + 32, 64, None) == ERR_OVERLAP  # scales inside codes


def test_q8_gemv_validation(lib):
    g = lib.q8_gemv
    assert g(W, DW, QX, DX, None, Y, 8, 48, None) == ERR_SHAPE  # K % 32
    assert g(W, DW, QX, DX, None, Y, -1, 64, None) == ERR_SHAPE
    assert g(W, DW, QX, DX, None, Y, 1 << 40, 1 << 30, None) == ERR_SHAPE  # N*K overflow guard
    assert g(None, None, None, None, None, None, 0, 64, None) == OK  # N == 0
    assert g(None, DW, QX, DX, None, Y, 8, 64, None) == ERR_NULL
    assert g(W, None, QX, DX, None, Y, 8, 64, None) == ERR_NULL
    assert g(W, DW, None, DX, None, Y, 8, 64, None) == ERR_NULL
    assert g(W, DW, QX, DX, None, None, 8, 64, None) == ERR_NULL
    assert g(W + 8, DW, QX, DX, None, Y, 8, 64, None) == ERR_ALIGN
    assert g(W, DW + 1, QX, DX, None, Y, 8, 64, None) == ERR_ALIGN
    assert g(W, DW, QX + 8, DX, None, Y, 8, 64, None) == ERR_ALIGN
    assert g(W, DW, QX, DX, R + 2, Y, 8, 64, None) == ERR_ALIGN
    assert g(W, DW, QX, DX, None, Y + 2, 8, 64, None) == ERR_ALIGN
    # outputs overlapping inputs
    assert g(W, DW, QX, DX, None, W + 64, 8, 64, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, None, DW, 8, 64, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, None, QX, 8, 64, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, None, DX, 8, 64, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, Y + 4, Y, 8, 64, None) == ERR_OVERLAP  # partial residual alias


def test_q8_gemv_batch_validation(lib):
    g = lib.q8_gemv_batch
    assert g(W, DW, QX, DX, None, Y, 8, 48, 2, None) == ERR_SHAPE  # K % 32
    assert g(W, DW, QX, DX, None, Y, 8, 64, 17, None) == ERR_SHAPE  # B > 16
    assert g(W, DW, QX, DX, None, Y, 8, 64, -1, None) == ERR_SHAPE
    assert g(W, DW, QX, DX, None, Y, -1, 64, 2, None) == ERR_SHAPE
    assert g(W, DW, QX, DX, None, Y, 1 << 40, 1 << 30, 2, None) == ERR_SHAPE  # N*K overflow guard
    assert g(None, None, None, None, None, None, 0, 64, 4, None) == OK  # N == 0
    assert g(None, None, None, None, None, None, 8, 64, 0, None) == OK  # B == 0
    assert g(None, DW, QX, DX, None, Y, 8, 64, 2, None) == ERR_NULL
    assert g(W, DW, QX, None, None, Y, 8, 64, 2, None) == ERR_NULL
    assert g(W, DW, QX, DX, None, None, 8, 64, 2, None) == ERR_NULL
    assert g(W + 8, DW, QX, DX, None, Y, 8, 64, 2, None) == ERR_ALIGN
    assert g(W, DW, QX + 8, DX, None, Y, 8, 64, 2, None) == ERR_ALIGN
    assert g(W, DW + 1, QX, DX, None, Y, 8, 64, 2, None) == ERR_ALIGN
    assert g(W, DW, QX, DX, R + 2, Y, 8, 64, 2, None) == ERR_ALIGN
    assert g(W, DW, QX, DX, None, Y + 2, 8, 64, 2, None) == ERR_ALIGN
    # y [B][N] against every input, and a residual that overlaps y without being y
    assert g(W, DW, QX, DX, None, W + 64, 8, 64, 2, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, None, QX + 64, 8, 64, 2, None) == ERR_OVERLAP  # inside vector 1's codes
    assert g(W, DW, QX, DX, None, DX, 8, 64, 2, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, None, DW, 8, 64, 2, None) == ERR_OVERLAP
    assert g(W, DW, QX, DX, Y + 4, Y, 8, 64, 2, None) == ERR_OVERLAP


@pytest.mark.parametrize("name", ["bf16_gemv", "f16_gemv"])
def test_16bit_gemv_validation(lib, name):
    g = getattr(lib, name)
    assert g(W, X, None, Y, 8, 12, None) == ERR_SHAPE  # K % 8
    assert g(W, X, None, Y, -3, 16, None) == ERR_SHAPE
    assert g(None, X, None, Y, 8, 16, None) == ERR_NULL
    assert g(W, None, None, Y, 8, 16, None) == ERR_NULL
    assert g(W + 2, X, None, Y, 8, 16, None) == ERR_ALIGN
    assert g(W, X + 2, None, Y, 8, 16, None) == ERR_ALIGN
    assert g(W, X, None, X, 8, 16, None) == ERR_OVERLAP
    assert g(W, X, R + 2, Y, 8, 16, None) == ERR_ALIGN
    assert g(W, X, None, Y + 2, 8, 16, None) == ERR_ALIGN
    assert g(W, X, None, W + 16, 8, 16, None) == ERR_OVERLAP
    assert g(None, None, None, None, 0, 16, None) == OK


def test_stacked_validation(lib):
    Part = lib.Part
    s = lib.gemv_stacked

    def parts(*ps):
        arr = (Part * max(1, len(ps)))()
        for i, p in enumerate(ps):
            arr[i] = Part(*p)
        return arr

    one = parts((W, DW, 8, Y, None))
    assert s(0, one, 0, QX, DX, 64, None) == ERR_ARG
    assert s(0, one, 5, QX, DX, 64, None) == ERR_ARG
    assert s(7, one, 1, QX, DX, 64, None) == ERR_ARG
    assert s(5, one, 1, QX, DX, 64, None) == ERR_ARG  # one past the last kind
    assert s(3, parts((W, None, 8, Y, None)), 1, X, None, 20, None) == ERR_SHAPE  # f16: K % 8
    assert s(3, parts((W + 2, None, 8, Y, None)), 1, X, None, 64, None) == ERR_ALIGN
    assert s(0, None, 1, QX, DX, 64, None) == ERR_NULL
    assert s(0, parts((W, DW, -1, Y, None)), 1, QX, DX, 64, None) == ERR_SHAPE
    assert s(0, one, 1, QX, None, 64, None) == ERR_NULL  # Q8_0 needs dx
    assert s(0, parts((W, None, 8, Y, None)), 1, QX, DX, 64, None) == ERR_NULL  # Q8_0 needs dw
    # two parts writing overlapping outputs
    two = parts((W, DW, 8, Y, None), (W + 0x100000, DW + 0x100000, 8, Y + 16, None))
    assert s(0, two, 2, QX, DX, 64, None) == ERR_OVERLAP
    # a part's output over another part's weights
    two = parts((W, DW, 8, Y, None), (W + 0x100000, DW + 0x100000, 8, W, None))
    assert s(0, two, 2, QX, DX, 64, None) == ERR_OVERLAP
    # residual of one part aliasing another part's output
    two = parts((W, DW, 8, Y, Y + 4096), (W + 0x100000, DW + 0x100000, 8, Y + 4096, None))
    assert s(0, two, 2, QX, DX, 64, None) == ERR_OVERLAP
    # all parts empty: nothing to do
    assert s(1, parts((None, None, 0, None, None), (None, None, 0, None, None)), 2, None, None, 16, None) == OK


def test_ptq1_rotate_validation(lib):
    q = lib.ptq1_rotate_quantize_act
    assert q(X, None, QX, DX, 96, None) == ERR_SHAPE  # K % 128
    assert q(X, None, QX, DX, -128, None) == ERR_SHAPE
    assert q(None, None, None, None, 0, None) == OK  # empty: nothing enqueued
    assert q(None, None, QX, DX, 128, None) == ERR_NULL
    assert q(X, None, None, DX, 128, None) == ERR_NULL
    assert q(X, None, QX, None, 128, None) == ERR_NULL
    assert q(X + 2, None, QX, DX, 128, None) == ERR_ALIGN
    assert q(X, R + 2, QX, DX, 128, None) == ERR_ALIGN
    assert q(X, None, QX, DX + 1, 128, None) == ERR_ALIGN
    assert q(X, None, X + 64, DX, 256, None) == ERR_OVERLAP  # codes inside x
    assert q(X, None, QX, QX + 32, 256, None) == ERR_OVERLAP  # scales inside codes
    assert q(X, X + 512, QX, DX, 256, None) == ERR_OVERLAP  # rotated values over x
    assert q(X, QX - 512, QX, DX, 256, None) == ERR_OVERLAP  # rotated values over the codes


def test_ptq1_gemv_validation(lib):
    g = lib.ptq1_gemv
    assert g(W, QX, DX, None, Y, 8, 96, None) == ERR_SHAPE  # K % 128
    assert g(W, QX, DX, None, Y, 8, 65536 + 128, None) == ERR_SHAPE  # K > Q8G_PTQ1_MAX_K
    assert g(W, QX, DX, None, Y, -1, 128, None) == ERR_SHAPE
    assert g(W, QX, DX, None, Y, (1 << 30) + 1, 128, None) == ERR_SHAPE  # N > Q8G_PTQ1_MAX_ROWS
    assert g(None, None, None, None, None, 0, 128, None) == OK  # N == 0
    assert g(None, QX, DX, None, Y, 8, 128, None) == ERR_NULL
    assert g(W, None, DX, None, Y, 8, 128, None) == ERR_NULL
    assert g(W, QX, None, None, Y, 8, 128, None) == ERR_NULL
    assert g(W, QX, DX, None, None, 8, 128, None) == ERR_NULL
    assert g(W + 2, QX, DX, None, Y, 8, 128, None) == ERR_ALIGN  # blocks are read as dwords
    assert g(W, QX + 8, DX, None, Y, 8, 128, None) == ERR_ALIGN
    assert g(W, QX, DX + 1, None, Y, 8, 128, None) == ERR_ALIGN
    assert g(W, QX, DX, R + 2, Y, 8, 128, None) == ERR_ALIGN
    assert g(W, QX, DX, None, Y + 2, 8, 128, None) == ERR_ALIGN
    assert g(W, QX, DX, None, W + 8 * 28 - 4, 8, 128, None) == ERR_OVERLAP  # y over the last block
    assert g(W, QX, DX, None, QX, 8, 128, None) == ERR_OVERLAP
    assert g(W, QX, DX, None, DX, 8, 128, None) == ERR_OVERLAP
    assert g(W, QX, DX, Y + 4, Y, 8, 128, None) == ERR_OVERLAP  # partial residual alias


def test_ptq1_stacked_validation(lib):
    Part = lib.Part
    s = lib.gemv_stacked
    arr = (Part * 2)()
    arr[0] = Part(W, None, 8, Y, None)
    arr[1] = Part(W + 0x100000, None, 8, Y + 16, None)
    assert s(4, arr, 2, QX, DX, 128, None) == ERR_OVERLAP  # outputs overlap
    arr[1] = Part(W + 0x100000, None, 8, W + 32, None)
    assert s(4, arr, 2, QX, DX, 128, None) == ERR_OVERLAP  # output over the other part's weights
    arr[1] = Part(W + 0x100000, None, 8, Y + 4096, None)
    assert s(4, arr, 2, QX, DX, 200, None) == ERR_SHAPE
    assert s(4, arr, 2, QX, None, 128, None) == ERR_NULL
    assert s(4, arr, 0, QX, DX, 128, None) == ERR_ARG
    rows, waves = ctypes.c_int(), ctypes.c_int()
    assert lib.q8g_gemv_config(4, 34816, 5120, ctypes.byref(rows), ctypes.byref(waves)) == OK
    assert (rows.value, waves.value) == (4, 5)  # 8 block columns x 4 rows per wave step, 5 waves per row
    assert lib.q8g_gemv_config(4, 100, 100, ctypes.byref(rows), ctypes.byref(waves)) == ERR_SHAPE


def test_rmsnorm_quantize_validation(lib):
    q = lib.q8_rmsnorm_quantize_act
    G = R  # gamma
    assert q(X, G, 1e-6, QX, DX, 48, None) == ERR_SHAPE  # K % 32
    assert q(X, G, 1e-6, QX, DX, 16384 + 32, None) == ERR_SHAPE  # one workgroup holds the row
    assert q(X, G, 1e-6, QX, DX, -32, None) == ERR_SHAPE
    assert q(X, G, -1e-6, QX, DX, 64, None) == ERR_ARG  # eps < 0
    assert q(X, G, float("nan"), QX, DX, 64, None) == ERR_ARG
    assert q(X, G, float("inf"), QX, DX, 64, None) == ERR_ARG
    assert q(None, None, 0.0, None, None, 0, None) == OK  # empty
    assert q(X, None, 1e-6, QX, DX, 64, None) == ERR_NULL
    assert q(None, G, 1e-6, QX, DX, 64, None) == ERR_NULL
    assert q(X, G, 1e-6, QX, None, 64, None) == ERR_NULL
    assert q(X, G + 4, 1e-6, QX, DX, 64, None) == ERR_ALIGN
    assert q(X + 4, G, 1e-6, QX, DX, 64, None) == ERR_ALIGN
    assert q(X, G, 1e-6, QX + 1, DX, 64, None) == ERR_ALIGN
    assert q(X, G, 1e-6, QX, DX + 1, 64, None) == ERR_ALIGN
    assert q(X, G, 1e-6, G + 16, DX, 64, None) == ERR_OVERLAP  # codes inside gamma
    assert q(X, G, 1e-6, QX, X + 64, 64, None) == ERR_OVERLAP  # scales inside x
    assert q(X, G, 1e-6, QX, QX + 32, 64, None) == ERR_OVERLAP


def test_silu_mul_quantize_validation(lib):
    q = lib.q8_silu_mul_quantize_act
    assert q(X, QX, DX, 48, None) == ERR_SHAPE
    assert q(X, QX, DX, -32, None) == ERR_SHAPE
    assert q(None, None, None, 0, None) == OK
    assert q(None, QX, DX, 64, None) == ERR_NULL
    assert q(X + 4, QX, DX, 64, None) == ERR_ALIGN
    assert q(X, QX, DX + 1, 64, None) == ERR_ALIGN
    assert q(X, X + 4 * 64, DX, 64, None) == ERR_OVERLAP  # codes inside the up half
    assert q(X, QX, QX + 32, 64, None) == ERR_OVERLAP


def test_batched_neighbour_quantize_validation(lib):
    n = lib.q8_rmsnorm_quantize_act_batch
    G = R
    assert n(X, G, 1e-6, QX, DX, 64, -1, None) == ERR_SHAPE
    assert n(X, G, 1e-6, QX, DX, 64, 65536, None) == ERR_SHAPE
    assert n(X, G, 1e-6, QX, DX, 48, 2, None) == ERR_SHAPE
    assert n(X, G, -1.0, QX, DX, 64, 2, None) == ERR_ARG
    assert n(None, None, 1e-6, None, None, 64, 0, None) == OK  # B == 0
    assert n(X, G, 1e-6, X + 4 * 64, DX, 64, 2, None) == ERR_OVERLAP  # codes inside vector 1 of x
    assert n(X, G, 1e-6, QX, QX + 64, 64, 2, None) == ERR_OVERLAP  # scales inside vector 1's codes
    s = lib.q8_silu_mul_quantize_act_batch
    assert s(X, QX, DX, 64, -1, None) == ERR_SHAPE
    assert s(X, QX, DX, 48, 2, None) == ERR_SHAPE
    assert s(None, None, None, 64, 0, None) == OK
    assert s(X, X + 8 * 64 + 16, DX, 64, 2, None) == ERR_OVERLAP  # codes inside vector 1's gate
    assert s(X + 4, QX, DX, 64, 2, None) == ERR_ALIGN


def test_fused_neighbour_gemv_validation(lib):
    Part = lib.Part
    s = lib.gemv_stacked_rmsnorm
    G = R
    one = (Part * 1)(Part(W, DW, 8, Y, None))
    assert s(one, 1, X, G, -1.0, 64, None) == ERR_ARG
    assert s(one, 0, X, G, 1e-6, 64, None) == ERR_ARG
    assert s(one, 1, X, G, 1e-6, 16384 + 32, None) == ERR_SHAPE
    assert s(one, 1, X, G, 1e-6, 48, None) == ERR_SHAPE
    assert s(one, 1, X, None, 1e-6, 64, None) == ERR_NULL  # gamma
    assert s(one, 1, X, G + 8, 1e-6, 64, None) == ERR_ALIGN
    assert s((Part * 1)(Part(W, DW, 8, G + 128, None)), 1, X, G, 1e-6, 64, None) == ERR_OVERLAP  # y in gamma
    assert s((Part * 1)(Part(W, None, 8, Y, None)), 1, X, G, 1e-6, 64, None) == ERR_NULL  # dw
    g = lib.q8_gemv_silu_mul
    assert g(W, DW, X, None, Y, 8, 48, None) == ERR_SHAPE
    assert g(W, DW, X, None, Y, -1, 64, None) == ERR_SHAPE
    assert g(W, DW, X, None, Y, 8, 16384 + 32, None) == ERR_SHAPE
    assert g(None, None, None, None, None, 0, 64, None) == OK
    assert g(W, DW, None, None, Y, 8, 64, None) == ERR_NULL
    assert g(W, DW, X + 4, None, Y, 8, 64, None) == ERR_ALIGN
    assert g(W, DW, X, None, X + 4 * 64, 8, 64, None) == ERR_OVERLAP  # y in the up half


def test_gateup_epilogue_validation(lib):
    g = lib.q8_gateup_silu_quantize
    WU, DU = W + 0x1000000, DW + 0x1000000
    QA, DA = Y, Y + 0x100000
    assert g(W, DW, WU, DU, 48, QX, DX, 64, QA, DA, None) == ERR_SHAPE  # F % 32
    assert g(W, DW, WU, DU, 64, QX, DX, 48, QA, DA, None) == ERR_SHAPE  # K % 32
    assert g(W, DW, WU, DU, -32, QX, DX, 64, QA, DA, None) == ERR_SHAPE
    assert g(None, None, None, None, 0, None, None, 64, None, None, None) == OK  # F == 0
    assert g(W, DW, WU, DU, 64, QX, DX, 64, None, DA, None) == ERR_NULL
    assert g(W, DW, None, DU, 64, QX, DX, 64, QA, DA, None) == ERR_NULL
    assert g(W, DW, WU, DU, 64, QX, None, 64, QA, DA, None) == ERR_NULL
    assert g(W, DW, WU, DU, 64, QX, DX, 64, QA + 4, DA, None) == ERR_ALIGN
    assert g(W, DW, WU + 8, DU, 64, QX, DX, 64, QA, DA, None) == ERR_ALIGN
    assert g(W, DW, WU, DU + 1, 64, QX, DX, 64, QA, DA, None) == ERR_ALIGN
    assert g(W, DW, WU, DU, 64, QX, DX, 64, WU + 64, DA, None) == ERR_OVERLAP  # codes in the up weights
    assert g(W, DW, WU, DU, 64, QX, DX, 64, QA, DX, None) == ERR_OVERLAP
    assert g(W, DW, WU, DU, 64, QX, DX, 64, QA, QA + 32, None) == ERR_OVERLAP
    n = lib.q8_gateup_rmsnorm_silu_quantize
    G = R
    assert n(W, DW, WU, DU, 64, X, G, 1e-6, 16384 + 32, QA, DA, None) == ERR_SHAPE
    assert n(W, DW, WU, DU, 64, X, G, -1.0, 64, QA, DA, None) == ERR_ARG
    assert n(W, DW, WU, DU, 64, X, None, 1e-6, 64, QA, DA, None) == ERR_NULL
    assert n(W, DW, WU, DU, 64, X, G + 4, 1e-6, 64, QA, DA, None) == ERR_ALIGN
    assert n(W, DW, WU, DU, 64, X, G, 1e-6, 64, G + 64, DA, None) == ERR_OVERLAP  # codes in gamma


def test_gateup_f32_epilogue_validation(lib):
    g = lib.q8_gateup_silu
    WU, DU = W + 0x1000000, DW + 0x1000000
    A = Y
    assert g(W, DW, WU, DU, 48, QX, DX, 64, A, None) == ERR_SHAPE  # F % 32
    assert g(W, DW, WU, DU, 64, QX, DX, 48, A, None) == ERR_SHAPE  # K % 32
    assert g(None, None, None, None, 0, None, None, 64, None, None) == OK  # F == 0
    assert g(W, DW, WU, DU, 64, QX, DX, 64, None, None) == ERR_NULL
    assert g(W, DW, WU, DU, 64, QX, None, 64, A, None) == ERR_NULL
    assert g(W, DW, WU, DU, 64, QX, DX, 64, A + 2, None) == ERR_ALIGN
    assert g(W, DW, WU, DU, 64, QX, DX, 64, WU + 64, None) == ERR_OVERLAP  # a in the up weights
    assert g(W, DW, WU, DU, 64, QX, DX, 64, DX, None) == ERR_OVERLAP
    n = lib.q8_gateup_rmsnorm_silu
    G = R
    assert n(W, DW, WU, DU, 64, X, G, 1e-6, 16384 + 32, A, None) == ERR_SHAPE
    assert n(W, DW, WU, DU, 64, X, G, -1.0, 64, A, None) == ERR_ARG
    assert n(W, DW, WU, DU, 64, X, None, 1e-6, 64, A, None) == ERR_NULL
    assert n(W, DW, WU, DU, 64, X, G + 4, 1e-6, 64, A, None) == ERR_ALIGN
    assert n(W, DW, WU, DU, 64, X, G, 1e-6, 64, G + 64, None) == ERR_OVERLAP  # a in gamma


def test_probe_validation(lib):
    assert lib.q8g_probe_read(X, 17, Y, None) == ERR_SHAPE
    assert lib.q8g_probe_read(None, 16, Y, None) == ERR_NULL
    assert lib.q8g_probe_read(X + 8, 16, Y, None) == ERR_ALIGN
    assert lib.q8g_flush(X, 15, 0, None) == ERR_SHAPE
    assert lib.q8g_flush(None, 0, 0, None) == OK
    assert lib.q8g_flush(X + 4, 16, 0, None) == ERR_ALIGN


def test_decode_stack_validation(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    Part = lib.Part

    class Op(ctypes.Structure):
        _fields_ = [("x", P), ("qx", P), ("dx", P), ("K", I64), ("nparts", ctypes.c_int32),
                    ("reserved", ctypes.c_int32), ("parts", Part * 4)]

    assert ctypes.sizeof(Op) == 200
    f = lib.q8_decode_stack
    f.argtypes = [ctypes.POINTER(Op), P, ctypes.c_int, P, P]
    f.restype = ctypes.c_int
    SYNC, DEV = A + 0x70000000, A + 0x78000000

    def ops(*specs):
        arr = (Op * max(1, len(specs)))()
        for i, (x, k, parts) in enumerate(specs):
            arr[i].x, arr[i].K, arr[i].nparts = x, k, len(parts)
            for j, p in enumerate(parts):
                arr[i].parts[j] = Part(*p)
        return arr

    good = ops((X, 64, [(W, DW, 8, Y, None)]))
    assert f(good, DEV, -1, SYNC, None) == ERR_ARG
    assert f(good, DEV, 0, SYNC, None) == OK
    assert f(good, None, 1, SYNC, None) == ERR_NULL
    assert f(good, DEV, 1, None, None) == ERR_NULL
    assert f(good, DEV, 1, SYNC + 4, None) == ERR_ALIGN
    assert f(ops((X, 48, [(W, DW, 8, Y, None)])), DEV, 1, SYNC, None) == ERR_SHAPE  # K % 32
    assert f(ops((X, 16384 + 32, [(W, DW, 8, Y, None)])), DEV, 1, SYNC, None) == ERR_SHAPE
    assert f(ops((X, 64, [])), DEV, 1, SYNC, None) == ERR_ARG  # no parts
    assert f(ops((X, 64, [(W, DW, 0, Y, None)])), DEV, 1, SYNC, None) == ERR_SHAPE  # no rows
    assert f(ops((None, 64, [(W, DW, 8, Y, None)])), DEV, 1, SYNC, None) == ERR_NULL
    assert f(ops((X + 4, 64, [(W, DW, 8, Y, None)])), DEV, 1, SYNC, None) == ERR_ALIGN
    assert f(ops((X, 64, [(W, DW, 8, X, None)])), DEV, 1, SYNC, None) == ERR_OVERLAP  # y over x
    # op 0 writes over op 1's weights
    assert f(ops((X, 64, [(W, DW, 8, W + 0x100000, None)]), (X, 64, [(W + 0x100000, DW, 8, Y, None)])),
             DEV, 2, SYNC, None) == ERR_OVERLAP
    # two ops writing one buffer
    assert f(ops((X, 64, [(W, DW, 8, Y, None)]), (X, 64, [(W, DW, 8, Y, None)])), DEV, 2, SYNC, None) == ERR_OVERLAP
    # op 1 writing op 0's input (read before op 1 runs): a race-free chain is the other way round
    assert f(ops((X, 64, [(W, DW, 8, Y, None)]), (X + 0x100000, 64, [(W, DW, 16, X, None)])), DEV, 2, SYNC,
             None) == ERR_OVERLAP

    # the same step over the library's static workspace: the same checks, plus the status word
    h = lib.q8_decode_stack_static
    h.argtypes = [ctypes.POINTER(Op), P, ctypes.c_int, P, P]
    h.restype = ctypes.c_int
    assert h(good, DEV, -1, None, None) == ERR_ARG
    assert h(good, DEV, 0, None, None) == OK
    assert h(good, None, 1, None, None) == ERR_NULL
    assert h(good, DEV + 4, 1, None, None) == ERR_ALIGN
    assert h(good, DEV, 1, SYNC + 2, None) == ERR_ALIGN  # status
    assert h(good, DEV, 1, Y + 4, None) == ERR_OVERLAP  # status over an output
    assert h(ops((X, 48, [(W, DW, 8, Y, None)])), DEV, 1, None, None) == ERR_SHAPE
    assert h(ops((X, 64, [(W, DW, 8, X, None)])), DEV, 1, None, None) == ERR_OVERLAP
