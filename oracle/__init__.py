"""Python front of the CPU oracle (oracle.c) for the decode-step GEMV.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does. It
shares no code with the HIP library. Arrays are numpy; results are f64.

What it computes is stated, with its sources, at the top of oracle.c:
the Q8_0 activation quantizer, the per-block int32 dot, the Q8_0 GEMV (single
vector and small batch), the bf16 and f16 GEMVs, the RMS-normalization and
gated-activation steps folded into a projection's prologue, and the PTQ1_0
ternary GEMV with its Hadamard-rotated activation, of "Filling in the blanks: Inference using Phobos" (section Fast
Decode) and "One level down: #002 the same compiler on a GPU" (sections
Emitting for a GPU and The numerical contract).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True, out: str | None = None, src: str | None = None) -> str:
    """Compile oracle.c with gcc into a shared object; returns its path."""
    out = out or _LIB
    src = src or _SRC
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def _bind(lib):
    lib.orc_f16_value.argtypes = [ctypes.c_uint16]
    lib.orc_f16_value.restype = ctypes.c_double
    lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_value.restype = ctypes.c_double
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_quantize_act.argtypes = [_P, _I64, _P, _P]
    lib.orc_quantize_act.restype = None
    lib.orc_block_isums.argtypes = [_P, _P, _I64, _I64, _P]
    lib.orc_block_isums.restype = None
    lib.orc_q8_gemv.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P, _P]
    lib.orc_q8_gemv.restype = None
    lib.orc_bf16_gemv.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
    lib.orc_bf16_gemv.restype = None
    lib.orc_q8_gemv_mt.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int]
    lib.orc_q8_gemv_mt.restype = ctypes.c_int
    lib.orc_bf16_gemv_mt.argtypes = [_P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int]
    lib.orc_bf16_gemv_mt.restype = ctypes.c_int
    lib.orc_f16_gemv.argtypes = [_P, _P, _P, _I64, _I64, _P, _P]
    lib.orc_f16_gemv.restype = None
    lib.orc_f16_gemv_mt.argtypes = [_P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int]
    lib.orc_f16_gemv_mt.restype = ctypes.c_int
    lib.orc_q8_gemv_batch.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
    lib.orc_q8_gemv_batch.restype = None
    lib.orc_rmsnorm.argtypes = [_P, _P, ctypes.c_float, _I64, _P]
    lib.orc_rmsnorm.restype = None
    lib.orc_silu_mul.argtypes = [_P, _I64, _P]
    lib.orc_silu_mul.restype = None
    lib.orc_quantize_blocks.argtypes = [_P, _I64, _I64, _P, _P]
    lib.orc_quantize_blocks.restype = None
    lib.orc_ptq1_decode.argtypes = [_P, _I64, _P, _P]
    lib.orc_ptq1_decode.restype = None
    lib.orc_hadamard128.argtypes = [_P, _I64, _P]
    lib.orc_hadamard128.restype = None
    lib.orc_ptq1_activation.argtypes = [_P, _I64, _P, _P, _P]
    lib.orc_ptq1_activation.restype = None
    lib.orc_ptq1_gemv.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P]
    lib.orc_ptq1_gemv.restype = None
    lib.orc_ptq1_gemv_mt.argtypes = [_P, _P, _P, _P, _I64, _I64, _P, _P, ctypes.c_int]
    lib.orc_ptq1_gemv_mt.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the built oracle (building it first if it is missing or stale)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


class Oracle:
    """The oracle's entry points over numpy arrays, bound to one loaded library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # number formats
    def f16_value(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([self.lib.orc_f16_value(int(b)) for b in bits], dtype=np.float64)

    def bf16_value(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16).ravel()
        return np.array([self.lib.orc_bf16_value(int(b)) for b in bits], dtype=np.float64)

    def f32_to_f16(self, values) -> np.ndarray:
        values = np.asarray(values, dtype=np.float32).ravel()
        return np.array([self.lib.orc_f32_to_f16(float(v)) for v in values], dtype=np.uint16)

    # neighbour steps folded into a projection's prologue
    def rmsnorm(self, x, gamma, eps):
        """f32 h = (x * r) * gamma with r = f32(1 / sqrt(mean(x^2) + eps)) from f64."""
        x, px = _c(x, np.float32)
        gamma, pg = _c(gamma, np.float32)
        assert x.ndim == 1 and gamma.shape == x.shape
        h = np.empty_like(x)
        self.lib.orc_rmsnorm(px, pg, float(eps), x.shape[0], h.ctypes.data)
        return h

    def silu_mul(self, gu):
        """f32 a = silu(gate) * up from gu = [gate (K) | up (K)], in f64 rounded once."""
        gu, pgu = _c(gu, np.float32)
        assert gu.ndim == 1 and gu.shape[0] % 2 == 0
        k = gu.shape[0] // 2
        a = np.empty(k, np.float32)
        self.lib.orc_silu_mul(pgu, k, a.ctypes.data)
        return a

    # the method
    def quantize_act(self, x):
        x, px = _c(x, np.float32)
        k = x.shape[0]
        if x.ndim != 1 or k % 32:
            raise ValueError("x must be 1-D with length a multiple of 32")
        qx = np.empty(k, np.int8)
        dx = np.empty(k // 32, np.uint16)
        self.lib.orc_quantize_act(px, k, qx.ctypes.data, dx.ctypes.data)
        return qx, dx

    def block_isums(self, qw, qx):
        qw, pw = _c(qw, np.int8)
        qx, pq = _c(qx, np.int8)
        n, k = qw.shape
        assert qx.shape == (k,) and k % 32 == 0
        out = np.empty((n, k // 32), np.int32)
        self.lib.orc_block_isums(pw, pq, n, k, out.ctypes.data)
        return out

    def q8_gemv(self, qw, dw, qx, dx, residual=None, nthreads: int = 0):
        """(y, S) in f64. nthreads 0: the single-threaded entry; otherwise row-partitioned threads."""
        qw, pw = _c(qw, np.int8)
        dw, pdw = _c(dw, np.uint16)
        qx, pq = _c(qx, np.int8)
        dx, pdx = _c(dx, np.uint16)
        n, k = qw.shape
        assert k % 32 == 0 and dw.shape == (n, k // 32) and qx.shape == (k,) and dx.shape == (k // 32,)
        pr = None
        if residual is not None:
            residual, pr = _c(residual, np.float32)
            assert residual.shape == (n,)
        y = np.empty(n, np.float64)
        s = np.empty(n, np.float64)
        if nthreads:
            rc = self.lib.orc_q8_gemv_mt(pw, pdw, pq, pdx, pr, n, k, y.ctypes.data, s.ctypes.data, nthreads)
            if rc < 0:
                raise MemoryError("oracle thread setup failed")
        else:
            self.lib.orc_q8_gemv(pw, pdw, pq, pdx, pr, n, k, y.ctypes.data, s.ctypes.data)
        return y, s

    def q8_gemv_batch(self, qw, dw, qx, dx, residual=None, nthreads: int = 0):
        """(y, S) as [B, N] f64 for B activation vectors qx [B, K], dx [B, K/32].
        nthreads 0: the oracle's batch entry; otherwise the threaded GEMV once per vector."""
        qw, pw = _c(qw, np.int8)
        dw, pdw = _c(dw, np.uint16)
        qx, pq = _c(qx, np.int8)
        dx, pdx = _c(dx, np.uint16)
        n, k = qw.shape
        b = qx.shape[0]
        assert k % 32 == 0 and dw.shape == (n, k // 32) and qx.shape == (b, k) and dx.shape == (b, k // 32)
        pr = None
        if residual is not None:
            residual, pr = _c(residual, np.float32)
            assert residual.shape == (b, n)
        y = np.empty((b, n), np.float64)
        s = np.empty((b, n), np.float64)
        if nthreads:
            for i in range(b):
                yi, si = self.q8_gemv(qw, dw, qx[i], dx[i], None if residual is None else residual[i], nthreads)
                y[i], s[i] = yi, si
        else:
            self.lib.orc_q8_gemv_batch(pw, pdw, pq, pdx, pr, n, k, b, y.ctypes.data, s.ctypes.data)
        return y, s

    # PTQ1_0: ternary weights, 128 per 28-byte block, Hadamard-rotated activation
    PTQ1_BLOCK = 128
    PTQ1_BYTES = 28

    def quantize_blocks(self, x, block):
        """The activation quantizer over blocks of `block` values: (codes int8, scale bits)."""
        x, px = _c(x, np.float32)
        k = x.shape[0]
        if x.ndim != 1 or k % block:
            raise ValueError("x must be 1-D with length a multiple of the block")
        qx = np.empty(k, np.int8)
        dx = np.empty(k // block, np.uint16)
        self.lib.orc_quantize_blocks(px, k, block, qx.ctypes.data, dx.ctypes.data)
        return qx, dx

    def ptq1_decode(self, w):
        """Trits int8 [N, K] and scale bits uint16 [N, K/128] of PTQ1_0 rows w uint8 [N, 28 K/128]."""
        w, pw = _c(w, np.uint8)
        n, nbytes = w.shape
        assert nbytes % self.PTQ1_BYTES == 0
        nb = nbytes // self.PTQ1_BYTES
        t = np.empty((n, nb * self.PTQ1_BLOCK), np.int8)
        sc = np.empty((n, nb), np.uint16)
        self.lib.orc_ptq1_decode(pw, n * nb, t.ctypes.data, sc.ctypes.data)
        return t, sc

    def hadamard128(self, x):
        """f32 H x / sqrt(128) per 128-value block (Sylvester order), from f64 sums."""
        x, px = _c(x, np.float32)
        k = x.shape[0]
        assert x.ndim == 1 and k % self.PTQ1_BLOCK == 0
        out = np.empty(k, np.float32)
        self.lib.orc_hadamard128(px, k, out.ctypes.data)
        return out

    def ptq1_activation(self, x):
        """(rotated f32, codes int8 [K], scale bits [K/128]) of an activation x f32 [K]."""
        x, px = _c(x, np.float32)
        k = x.shape[0]
        assert x.ndim == 1 and k % self.PTQ1_BLOCK == 0
        rot = np.empty(k, np.float32)
        qx = np.empty(k, np.int8)
        dx = np.empty(k // self.PTQ1_BLOCK, np.uint16)
        self.lib.orc_ptq1_activation(px, k, rot.ctypes.data, qx.ctypes.data, dx.ctypes.data)
        return rot, qx, dx

    def ptq1_gemv(self, w, qx, dx, residual=None, nthreads: int = 0):
        """(y, S) in f64 for PTQ1_0 rows w uint8 [N, 28 K/128] and the rotated, quantized
        activation qx int8 [K], dx [K/128]."""
        w, pw = _c(w, np.uint8)
        qx, pq = _c(qx, np.int8)
        dx, pdx = _c(dx, np.uint16)
        n = w.shape[0]
        k = qx.shape[0]
        assert k % self.PTQ1_BLOCK == 0 and w.shape == (n, k // self.PTQ1_BLOCK * self.PTQ1_BYTES)
        assert dx.shape == (k // self.PTQ1_BLOCK,)
        pr = None
        if residual is not None:
            residual, pr = _c(residual, np.float32)
            assert residual.shape == (n,)
        y = np.empty(n, np.float64)
        s = np.empty(n, np.float64)
        if nthreads:
            rc = self.lib.orc_ptq1_gemv_mt(pw, pq, pdx, pr, n, k, y.ctypes.data, s.ctypes.data, nthreads)
            if rc < 0:
                raise MemoryError("oracle thread setup failed")
        else:
            self.lib.orc_ptq1_gemv(pw, pq, pdx, pr, n, k, y.ctypes.data, s.ctypes.data)
        return y, s

    def f16_gemv(self, w, x, residual=None, nthreads: int = 0):
        return self._16bit_gemv("f16", w, x, residual, nthreads)

    def bf16_gemv(self, w, x, residual=None, nthreads: int = 0):
        return self._16bit_gemv("bf16", w, x, residual, nthreads)

    def _16bit_gemv(self, kind, w, x, residual, nthreads):
        w, pw = _c(w, np.uint16)
        x, px = _c(x, np.uint16)
        n, k = w.shape
        assert x.shape == (k,)
        pr = None
        if residual is not None:
            residual, pr = _c(residual, np.float32)
            assert residual.shape == (n,)
        y = np.empty(n, np.float64)
        s = np.empty(n, np.float64)
        st = getattr(self.lib, f"orc_{kind}_gemv")
        mt = getattr(self.lib, f"orc_{kind}_gemv_mt")
        if nthreads:
            rc = mt(pw, px, pr, n, k, y.ctypes.data, s.ctypes.data, nthreads)
            if rc < 0:
                raise MemoryError("oracle thread setup failed")
        else:
            st(pw, px, pr, n, k, y.ctypes.data, s.ctypes.data)
        return y, s


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def quantize_act(x):
    return get().quantize_act(x)


def block_isums(qw, qx):
    return get().block_isums(qw, qx)


def q8_gemv(qw, dw, qx, dx, residual=None, nthreads: int = 0):
    return get().q8_gemv(qw, dw, qx, dx, residual, nthreads)


def bf16_gemv(w, x, residual=None, nthreads: int = 0):
    return get().bf16_gemv(w, x, residual, nthreads)


def f16_gemv(w, x, residual=None, nthreads: int = 0):
    return get().f16_gemv(w, x, residual, nthreads)


def q8_gemv_batch(qw, dw, qx, dx, residual=None, nthreads: int = 0):
    return get().q8_gemv_batch(qw, dw, qx, dx, residual, nthreads)


def rmsnorm(x, gamma, eps):
    return get().rmsnorm(x, gamma, eps)


def silu_mul(gu):
    return get().silu_mul(gu)


def ptq1_activation(x):
    return get().ptq1_activation(x)


def ptq1_gemv(w, qx, dx, residual=None, nthreads: int = 0):
    return get().ptq1_gemv(w, qx, dx, residual, nthreads)
