"""Python binding of libq8gemv: decode-step GEMV for Q8_0 and bf16 weights on MI355X.

The entry points mirror the C ABI of include/q8gemv.h one for one. This module only
checks and marshals arguments (torch tensors in device memory, the current torch
stream); every step of the computation runs in the HIP kernels of the library.
There is no fallback: if the library is missing, every call raises.

Storage conventions (as in the C header):
  * Q8_0 weights: codes int8 [N, K], scales as binary16 bits [N, K/32] (torch.float16,
    torch.int16 or torch.uint16 tensors are all accepted as 16-bit storage);
  * quantized activation: codes int8 [K], scales binary16 bits [K/32];
  * bf16 weights / activation: torch.bfloat16 (or 16-bit integer storage of the bits);
  * PTQ1_0 weights: uint8 [N, K/128 * 28] (28-byte blocks of 128 ternary weights); their
    activation is the rotated codes int8 [K] with binary16 scales [K/128] of
    ptq1_rotate_quantize_act;
  * outputs and residuals: torch.float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8gemv.so")

Q8G_Q8_0 = 0
Q8G_BF16 = 1
Q8G_Q8_0_F32 = 2
Q8G_F16 = 3
Q8G_PTQ1_0 = 4
Q8G_LAYOUT_ROWS = 0
Q8G_LAYOUT_TILE16 = 1
PTQ1_BLOCK = 128
PTQ1_BYTES = 28
PTQ1_MAX_K = 65536
FUSED_MAX_K = 16384
MAX_PARTS = 4
BATCH_MAX = 16
PROBE_SINK_WORDS = 16384

_STATUS = {
    0: "Q8G_OK",
    1: "Q8G_ERR_NULL",
    2: "Q8G_ERR_SHAPE",
    3: "Q8G_ERR_ALIGN",
    4: "Q8G_ERR_ARG",
    5: "Q8G_ERR_LAUNCH",
    6: "Q8G_ERR_OVERLAP",
}


class Q8GemvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({msg})")
        self.status = status


class _Part(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("dw", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("y", ctypes.c_void_p),
        ("residual", ctypes.c_void_p),
    ]


class _StackOp(ctypes.Structure):
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("qx", ctypes.c_void_p),
        ("dx", ctypes.c_void_p),
        ("K", ctypes.c_int64),
        ("nparts", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("parts", _Part * 4),
    ]


STACK_SYNC_WORDS = 20480
STACK_MAX_OPS = 256
STACK_ERR_WORD = 16
STACK_MAX_K = 16384

_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load_library(path: str = LIB_PATH):
    """Load libq8gemv.so (built by __graft_entry__.build()). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.q8_quantize_act.argtypes = [_P, _P, _P, _I64, _P]
    lib.q8_gemv.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _P]
    lib.bf16_gemv.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
    lib.f16_gemv.argtypes = [_P, _P, _P, _P, _I64, _I64, _P]
    lib.q8_gemv_batch.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
    lib.q8g_batch_config.argtypes = [_I64, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.q8g_batch_tiled_streams.argtypes = [_I64, _I64, ctypes.POINTER(ctypes.c_int)]
    lib.q8_gemv_batch_layout.argtypes = [ctypes.c_int, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P]
    lib.q8_tile16_sizes.argtypes = [_I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
    lib.q8_pack_tile16.argtypes = [_P, _P, _I64, _I64, _P, _P]
    lib.gemv_stacked.argtypes = [ctypes.c_int, ctypes.POINTER(_Part), ctypes.c_int, _P, _P, _I64, _P]
    lib.q8_rmsnorm_quantize_act.argtypes = [_P, _P, ctypes.c_float, _P, _P, _I64, _P]
    lib.q8_silu_mul_quantize_act.argtypes = [_P, _P, _P, _I64, _P]
    lib.q8_rmsnorm_quantize_act_batch.argtypes = [_P, _P, ctypes.c_float, _P, _P, _I64, _I64, _P]
    lib.q8_silu_mul_quantize_act_batch.argtypes = [_P, _P, _P, _I64, _I64, _P]
    lib.gemv_stacked_rmsnorm.argtypes = [ctypes.POINTER(_Part), ctypes.c_int, _P, _P, ctypes.c_float, _I64, _P]
    lib.q8_gemv_silu_mul.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P]
    lib.q8_gateup_silu_quantize.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _P, _P]
    lib.q8_gateup_rmsnorm_silu_quantize.argtypes = [_P, _P, _P, _P, _I64, _P, _P, ctypes.c_float, _I64, _P, _P, _P]
    lib.q8_gateup_silu.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _I64, _P, _P]
    lib.q8_gateup_rmsnorm_silu.argtypes = [_P, _P, _P, _P, _I64, _P, _P, ctypes.c_float, _I64, _P, _P]
    lib.ptq1_rotate_quantize_act.argtypes = [_P, _P, _P, _P, _I64, _P]
    lib.ptq1_gemv.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _P]
    lib.q8g_status_str.argtypes = [ctypes.c_int]
    lib.q8g_status_str.restype = ctypes.c_char_p
    lib.q8g_probe_read.argtypes = [_P, _I64, _P, _P]
    lib.q8g_probe_read_cached.argtypes = [_P, _I64, _P, _P]
    lib.q8g_flush.argtypes = [_P, _I64, ctypes.c_uint32, _P]
    lib.q8_decode_stack.argtypes = [ctypes.POINTER(_StackOp), _P, ctypes.c_int, _P, _P]
    lib.q8_decode_stack_static.argtypes = [ctypes.POINTER(_StackOp), _P, ctypes.c_int, _P, _P]
    lib.q8g_gemv_config.argtypes = [ctypes.c_int, _I64, _I64, ctypes.POINTER(ctypes.c_int),
                                    ctypes.POINTER(ctypes.c_int)]
    for fn in ("q8_quantize_act", "q8_gemv", "q8_gemv_batch", "bf16_gemv", "f16_gemv", "gemv_stacked",
               "q8g_probe_read", "q8g_probe_read_cached", "q8g_flush", "q8g_gemv_config", "q8g_batch_config",
               "q8g_batch_tiled_streams", "q8_decode_stack",
               "q8_decode_stack_static",
               "q8_rmsnorm_quantize_act", "q8_silu_mul_quantize_act", "gemv_stacked_rmsnorm",
               "q8_gemv_silu_mul", "q8_gateup_silu_quantize", "q8_gateup_rmsnorm_silu_quantize",
               "q8_gateup_silu", "q8_gateup_rmsnorm_silu",
               "q8_rmsnorm_quantize_act_batch", "q8_silu_mul_quantize_act_batch",
               "ptq1_rotate_quantize_act", "ptq1_gemv", "q8_gemv_batch_layout", "q8_tile16_sizes",
               "q8_pack_tile16"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def unload_library():
    """Unload libq8gemv.so (its code object is unregistered from the HIP runtime at once).
    Only for process teardown: nothing of the library may be in flight or referenced by a
    graph, and every later call loads it again."""
    global _lib
    if _lib is None:
        return
    import _ctypes

    handle = _lib._handle
    _lib = None
    _ctypes.dlclose(handle)


def _check(fn: str, status: int):
    if status != 0:
        raise Q8GemvError(fn, status, load_library().q8g_status_str(status).decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t, name, dtypes, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t.data_ptr() if t.numel() else None


_I8 = (torch.int8,)
_H16 = (torch.float16, torch.int16, torch.uint16)
_B16 = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def q8_quantize_act(x, qx=None, dx=None, stream=None):
    """Quantize f32 x [K] into Q8_0 codes qx int8 [K] and binary16 scales dx [K/32]."""
    k = x.shape[0] if x.dim() == 1 else -1
    if k < 0 or k % 32:
        raise ValueError("x must be 1-D with a length that is a multiple of 32")
    if qx is None:
        qx = torch.empty(k, dtype=torch.int8, device=x.device)
    if dx is None:
        dx = torch.empty(k // 32, dtype=torch.float16, device=x.device)
    st = load_library().q8_quantize_act(_ptr(x, "x", _F32), _ptr(qx, "qx", _I8, (k,)),
                                        _ptr(dx, "dx", _H16, (k // 32,)), k, _stream(stream))
    _check("q8_quantize_act", st)
    return qx, dx


def q8_rmsnorm_quantize_act(x, gamma, eps, qx=None, dx=None, stream=None):
    """Quantize (x * r) * gamma, r = 1/sqrt(mean(x^2) + eps), into Q8_0 codes qx int8 [K] and
    binary16 scales dx [K/32]. x, gamma f32 [K], K <= 16384. With x [B, K], each row is
    normalized and quantized on its own (one launch): qx [B, K], dx [B, K/32]."""
    if x.dim() not in (1, 2) or x.shape[-1] % 32:
        raise ValueError("x must be [K] or [B, K] with K a multiple of 32")
    k = x.shape[-1]
    lead = tuple(x.shape[:-1])
    if qx is None:
        qx = torch.empty(lead + (k,), dtype=torch.int8, device=x.device)
    if dx is None:
        dx = torch.empty(lead + (k // 32,), dtype=torch.float16, device=x.device)
    lib = load_library()
    args = (_ptr(x, "x", _F32), _ptr(gamma, "gamma", _F32, (k,)), float(eps), _ptr(qx, "qx", _I8, lead + (k,)),
            _ptr(dx, "dx", _H16, lead + (k // 32,)), k)
    if lead:
        st = lib.q8_rmsnorm_quantize_act_batch(*args, lead[0], _stream(stream))
        _check("q8_rmsnorm_quantize_act_batch", st)
    else:
        st = lib.q8_rmsnorm_quantize_act(*args, _stream(stream))
        _check("q8_rmsnorm_quantize_act", st)
    return qx, dx


def q8_silu_mul_quantize_act(gu, qx=None, dx=None, stream=None):
    """Quantize silu(gate) * up, gu = [gate | up] f32 [2K], into qx int8 [K] and dx [K/32].
    With gu [B, 2K], each row on its own (one launch): qx [B, K], dx [B, K/32]."""
    if gu.dim() not in (1, 2) or gu.shape[-1] % 64:
        raise ValueError("gu must be [2K] or [B, 2K] with K a multiple of 32")
    k = gu.shape[-1] // 2
    lead = tuple(gu.shape[:-1])
    if qx is None:
        qx = torch.empty(lead + (k,), dtype=torch.int8, device=gu.device)
    if dx is None:
        dx = torch.empty(lead + (k // 32,), dtype=torch.float16, device=gu.device)
    lib = load_library()
    args = (_ptr(gu, "gu", _F32), _ptr(qx, "qx", _I8, lead + (k,)), _ptr(dx, "dx", _H16, lead + (k // 32,)), k)
    if lead:
        st = lib.q8_silu_mul_quantize_act_batch(*args, lead[0], _stream(stream))
        _check("q8_silu_mul_quantize_act_batch", st)
    else:
        st = lib.q8_silu_mul_quantize_act(*args, _stream(stream))
        _check("q8_silu_mul_quantize_act", st)
    return qx, dx


def q8_gemv(qw, dw, qx, dx, y=None, residual=None, stream=None):
    """y = Q8_0(qw, dw) · (qx, dx) (+ residual). Returns y (f32 [N])."""
    if qw.dim() != 2:
        raise ValueError("qw must be [N, K]")
    n, k = qw.shape
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=qw.device)
    st = load_library().q8_gemv(
        _ptr(qw, "qw", _I8), _ptr(dw, "dw", _H16, (n, k // 32)), _ptr(qx, "qx", _I8, (k,)),
        _ptr(dx, "dx", _H16, (k // 32,)), _ptr(residual, "residual", _F32, (n,), optional=True),
        _ptr(y, "y", _F32, (n,)), n, k, _stream(stream))
    _check("q8_gemv", st)
    return y


def q8_gemv_batch(qw, dw, qx, dx, y=None, residual=None, stream=None):
    """Small batch: y[b] = Q8_0(qw, dw) · (qx[b], dx[b]) (+ residual[b]) for B <= 16 activation
    vectors sharing one pass over the weights. qw int8 [N, K] and dw [N, K/32], or a Tile16
    (from pack_tile16); qx int8 [B, K], dx [B, K/32]; returns y (f32 [B, N])."""
    if qx.dim() != 2:
        raise ValueError("qx must be [B, K]")
    if isinstance(qw, Tile16):
        n, k, layout = qw.n, qw.k, Q8G_LAYOUT_TILE16
        pw, pdw = _ptr(qw.codes, "codes", _I8), _ptr(qw.scales, "scales", _H16)
    else:
        if qw.dim() != 2:
            raise ValueError("qw must be [N, K]")
        n, k = qw.shape
        layout = Q8G_LAYOUT_ROWS
        pw, pdw = _ptr(qw, "qw", _I8), _ptr(dw, "dw", _H16, (n, k // 32))
    b = qx.shape[0]
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=qx.device)
    st = load_library().q8_gemv_batch_layout(
        layout, pw, pdw, _ptr(qx, "qx", _I8, (b, k)), _ptr(dx, "dx", _H16, (b, k // 32)),
        _ptr(residual, "residual", _F32, (b, n), optional=True), _ptr(y, "y", _F32, (b, n)), n, k, b,
        _stream(stream))
    _check("q8_gemv_batch_layout", st)
    return y


class Tile16:
    """Q8_0 weights in the 16-row tiled layout of q8_gemv_batch (Q8G_LAYOUT_TILE16):
    codes int8 and scales (16-bit) as 1-D device tensors of the sizes q8_tile16_sizes gives."""

    def __init__(self, codes, scales, n, k):
        self.codes, self.scales, self.n, self.k = codes, scales, int(n), int(k)


def tile16_sizes(n, k):
    """(code bytes, scale bytes) of the tiled layout of an n x k matrix."""
    cb, sb = _I64(), _I64()
    _check("q8_tile16_sizes", load_library().q8_tile16_sizes(n, k, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def pack_tile16_host(qw, dw):
    """Host-side pack (numpy in, numpy out): qw int8 [N, K], dw uint16 [N, K/32] ->
    (codes int8 [code bytes], scales uint16 [scale bytes / 2]) in the tiled layout."""
    import numpy as np

    qw = np.ascontiguousarray(qw, dtype=np.int8)
    dw = np.ascontiguousarray(dw).view(np.uint16)
    n, k = qw.shape
    if dw.shape != (n, k // 32):
        raise ValueError("dw must be [N, K/32]")
    cb, sb = tile16_sizes(n, k)
    codes = np.empty(cb, np.int8)
    scales = np.empty(sb // 2, np.uint16)
    st = load_library().q8_pack_tile16(qw.ctypes.data if qw.size else None, dw.ctypes.data if dw.size else None,
                                       n, k, codes.ctypes.data if codes.size else None,
                                       scales.ctypes.data if scales.size else None)
    _check("q8_pack_tile16", st)
    return codes, scales


def pack_tile16(qw, dw, device="cuda"):
    """Pack host weights (numpy int8 [N, K] and uint16 [N, K/32]) into a device Tile16."""
    import numpy as np

    codes, scales = pack_tile16_host(qw, dw)
    n, k = np.asarray(qw).shape
    return Tile16(torch.from_numpy(codes).to(device), torch.from_numpy(scales.view(np.int16)).to(device), n, k)


def batch_config(n):
    """(k_split, steps_in_flight) that q8_gemv_batch uses for n rows."""
    ks, sf = ctypes.c_int(), ctypes.c_int()
    _check("q8g_batch_config", load_library().q8g_batch_config(n, ctypes.byref(ks), ctypes.byref(sf)))
    return ks.value, sf.value


def batch_tiled_streams(n, k):
    """True when q8_gemv_batch on an n x k Tile16 (16-byte aligned scales) streams whole
    tiles per wave (the persistent form), False when it takes batch_config(n)'s shape."""
    st = ctypes.c_int()
    _check("q8g_batch_tiled_streams", load_library().q8g_batch_tiled_streams(n, k, ctypes.byref(st)))
    return bool(st.value)


def q8_gemv_f32(qw, dw, x, y=None, residual=None, stream=None):
    """y = Q8_0(qw, dw) · quantize(x) (+ residual) with x f32 [K], quantized inside the
    launch exactly as q8_quantize_act would (one launch instead of two)."""
    if qw.dim() != 2:
        raise ValueError("qw must be [N, K]")
    return gemv_stacked([{"w": qw, "dw": dw, "y": y, "residual": residual}], x, stream=stream)[0]


def bf16_gemv(w, x, y=None, residual=None, stream=None):
    """y = w · x with bf16 inputs and f32 accumulation (+ residual). Returns y (f32 [N])."""
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    st = load_library().bf16_gemv(
        _ptr(w, "w", _B16), _ptr(x, "x", _B16, (k,)),
        _ptr(residual, "residual", _F32, (n,), optional=True), _ptr(y, "y", _F32, (n,)), n, k,
        _stream(stream))
    _check("bf16_gemv", st)
    return y


def f16_gemv(w, x, y=None, residual=None, stream=None):
    """y = w · x with IEEE binary16 inputs and f32 accumulation (+ residual). Returns y (f32 [N])."""
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    st = load_library().f16_gemv(
        _ptr(w, "w", _H16), _ptr(x, "x", _H16, (k,)),
        _ptr(residual, "residual", _F32, (n,), optional=True), _ptr(y, "y", _F32, (n,)), n, k,
        _stream(stream))
    _check("f16_gemv", st)
    return y


def ptq1_rotate_quantize_act(x, qx=None, dx=None, rot=None, stream=None):
    """Rotate f32 x [K] per 128-value block by the normalized Hadamard matrix and quantize
    the result per 128 values: returns (qx int8 [K], dx binary16 [K/128]). rot (f32 [K]),
    if given, receives the rotated values."""
    k = x.shape[0] if x.dim() == 1 else -1
    if k < 0 or k % PTQ1_BLOCK:
        raise ValueError("x must be 1-D with a length that is a multiple of 128")
    if qx is None:
        qx = torch.empty(k, dtype=torch.int8, device=x.device)
    if dx is None:
        dx = torch.empty(k // PTQ1_BLOCK, dtype=torch.float16, device=x.device)
    st = load_library().ptq1_rotate_quantize_act(
        _ptr(x, "x", _F32), _ptr(rot, "rot", _F32, (k,), optional=True), _ptr(qx, "qx", _I8, (k,)),
        _ptr(dx, "dx", _H16, (k // PTQ1_BLOCK,)), k, _stream(stream))
    _check("ptq1_rotate_quantize_act", st)
    return qx, dx


def ptq1_gemv(w, qx, dx, y=None, residual=None, stream=None):
    """y = PTQ1_0(w) · (qx, dx) (+ residual). w uint8 [N, K/128 * 28]; qx int8 [K] and dx
    binary16 [K/128] from ptq1_rotate_quantize_act. Returns y (f32 [N])."""
    if w.dim() != 2 or w.shape[1] % PTQ1_BYTES:
        raise ValueError("w must be [N, K/128 * 28]")
    n = w.shape[0]
    k = w.shape[1] // PTQ1_BYTES * PTQ1_BLOCK
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=w.device)
    st = load_library().ptq1_gemv(
        _ptr(w, "w", _U8), _ptr(qx, "qx", _I8, (k,)), _ptr(dx, "dx", _H16, (k // PTQ1_BLOCK,)),
        _ptr(residual, "residual", _F32, (n,), optional=True), _ptr(y, "y", _F32, (n,)), n, k, _stream(stream))
    _check("ptq1_gemv", st)
    return y


def gemv_stacked(parts, x, dx=None, stream=None):
    """One launch over 1..4 matrices sharing the input.

    parts: sequence of dicts with keys w (int8 [n, K] for Q8_0, bf16 [n, K], uint8
    [n, K/128 * 28] for PTQ1_0), dw (Q8_0 scales, omitted otherwise), y (f32 [n], allocated
    if absent), residual (optional).
    x: int8 codes [K] with dx binary16 scales [K/32] (Q8_0); or f32 [K] for Q8_0 weights
    (quantized inside the launch, dx None); or bf16 [K] / float16 [K] for bf16 / float16
    weights (dx None); or the rotated codes int8 [K] with dx binary16 [K/128] (PTQ1_0).
    The weight dtype selects the kind.
    Returns the list of outputs.
    """
    if not 1 <= len(parts) <= MAX_PARTS:
        raise ValueError("1 to 4 parts")
    if parts[0]["w"].dtype == torch.uint8:
        return _ptq1_stacked(parts, x, dx, stream)
    q8 = parts[0]["w"].dtype == torch.int8
    f16 = parts[0]["w"].dtype == torch.float16
    fused = q8 and x.dtype == torch.float32
    k = x.shape[0]
    arr = (_Part * len(parts))()
    outs = []
    for i, p in enumerate(parts):
        w = p["w"]
        if w.dim() != 2 or w.shape[1] != k:
            raise ValueError(f"part {i}: w must be [n, {k}]")
        n = w.shape[0]
        y = p.get("y")
        if y is None:
            y = torch.empty(n, dtype=torch.float32, device=w.device)
        outs.append(y)
        arr[i].w = _ptr(w, f"parts[{i}].w", _I8 if q8 else ((torch.float16,) if f16 else _B16))
        arr[i].dw = _ptr(p.get("dw"), f"parts[{i}].dw", _H16, (n, k // 32), optional=not q8) if q8 else None
        arr[i].n = n
        arr[i].y = _ptr(y, f"parts[{i}].y", _F32, (n,))
        arr[i].residual = _ptr(p.get("residual"), f"parts[{i}].residual", _F32, (n,), optional=True)
    px = _ptr(x, "x", _F32 if fused else (_I8 if q8 else ((torch.float16,) if f16 else _B16)), (k,))
    pdx = _ptr(dx, "dx", _H16, (k // 32,)) if (q8 and not fused) else None
    dt = Q8G_Q8_0_F32 if fused else (Q8G_Q8_0 if q8 else (Q8G_F16 if f16 else Q8G_BF16))
    st = load_library().gemv_stacked(dt, arr, len(parts), px, pdx, k, _stream(stream))
    _check("gemv_stacked", st)
    return outs


def _ptq1_stacked(parts, qx, dx, stream):
    k = qx.shape[0]
    if k % PTQ1_BLOCK:
        raise ValueError("K must be a multiple of 128")
    row = k // PTQ1_BLOCK * PTQ1_BYTES
    arr = (_Part * len(parts))()
    outs = []
    for i, p in enumerate(parts):
        w = p["w"]
        if w.dim() != 2 or w.shape[1] != row:
            raise ValueError(f"part {i}: w must be [n, {row}]")
        n = w.shape[0]
        y = p.get("y")
        if y is None:
            y = torch.empty(n, dtype=torch.float32, device=w.device)
        outs.append(y)
        arr[i].w = _ptr(w, f"parts[{i}].w", _U8)
        arr[i].dw = None
        arr[i].n = n
        arr[i].y = _ptr(y, f"parts[{i}].y", _F32, (n,))
        arr[i].residual = _ptr(p.get("residual"), f"parts[{i}].residual", _F32, (n,), optional=True)
    st = load_library().gemv_stacked(Q8G_PTQ1_0, arr, len(parts), _ptr(qx, "x", _I8, (k,)),
                                     _ptr(dx, "dx", _H16, (k // PTQ1_BLOCK,)), k, _stream(stream))
    _check("gemv_stacked", st)
    return outs


def gemv_stacked_rmsnorm(parts, x, gamma, eps, stream=None):
    """One launch over 1..4 Q8_0 matrices (parts as for gemv_stacked) of RMSnorm(x) * gamma:
    x, gamma f32 [K], K <= 16384, normalized and quantized inside the launch."""
    if not 1 <= len(parts) <= MAX_PARTS:
        raise ValueError("1 to 4 parts")
    k = x.shape[0]
    arr, outs = _q8_parts(parts, k)
    st = load_library().gemv_stacked_rmsnorm(arr, len(parts), _ptr(x, "x", _F32, (k,)),
                                             _ptr(gamma, "gamma", _F32, (k,)), float(eps), k, _stream(stream))
    _check("gemv_stacked_rmsnorm", st)
    return outs


def q8_gemv_silu_mul(qw, dw, gu, y=None, residual=None, stream=None):
    """y = Q8_0(qw, dw) · quantize(silu(gate) * up) (+ residual), gu = [gate | up] f32 [2K],
    the activation formed and quantized inside the launch. Returns y (f32 [N])."""
    if qw.dim() != 2:
        raise ValueError("qw must be [N, K]")
    n, k = qw.shape
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=qw.device)
    st = load_library().q8_gemv_silu_mul(
        _ptr(qw, "qw", _I8), _ptr(dw, "dw", _H16, (n, k // 32)), _ptr(gu, "gu", _F32, (2 * k,)),
        _ptr(residual, "residual", _F32, (n,), optional=True), _ptr(y, "y", _F32, (n,)), n, k, _stream(stream))
    _check("q8_gemv_silu_mul", st)
    return y


def q8_gateup_silu_quantize(w_gate, dw_gate, w_up, dw_up, x, dx=None, gamma=None, eps=None, qa=None, da=None,
                            stream=None):
    """Gate+up projection (Q8_0, F rows each) with a = silu(gate) * up quantized in the epilogue:
    returns (qa int8 [F], da binary16 [F/32]), the down projection's quantized input. x is either
    int8 codes [K] with dx binary16 scales [K/32], or f32 [K] with gamma f32 [K] and eps (RMS
    normalization in the prologue)."""
    if w_gate.dim() != 2 or w_up.shape != w_gate.shape:
        raise ValueError("w_gate and w_up must both be [F, K]")
    f, k = w_gate.shape
    if qa is None:
        qa = torch.empty(f, dtype=torch.int8, device=w_gate.device)
    if da is None:
        da = torch.empty(f // 32, dtype=torch.float16, device=w_gate.device)
    lib = load_library()
    common = (_ptr(w_gate, "w_gate", _I8), _ptr(dw_gate, "dw_gate", _H16, (f, k // 32)), _ptr(w_up, "w_up", _I8),
              _ptr(dw_up, "dw_up", _H16, (f, k // 32)), f)
    outs = (_ptr(qa, "qa", _I8, (f,)), _ptr(da, "da", _H16, (f // 32,)))
    if gamma is None:
        st = lib.q8_gateup_silu_quantize(*common, _ptr(x, "x", _I8, (k,)), _ptr(dx, "dx", _H16, (k // 32,)), k,
                                         *outs, _stream(stream))
        fn = "q8_gateup_silu_quantize"
    else:
        if eps is None:
            raise ValueError("eps is required with gamma")
        st = lib.q8_gateup_rmsnorm_silu_quantize(*common, _ptr(x, "x", _F32, (k,)), _ptr(gamma, "gamma", _F32, (k,)),
                                                 float(eps), k, *outs, _stream(stream))
        fn = "q8_gateup_rmsnorm_silu_quantize"
    _check(fn, st)
    return qa, da


def q8_gateup_silu(w_gate, dw_gate, w_up, dw_up, x, dx=None, gamma=None, eps=None, a=None, stream=None):
    """Gate+up projection (Q8_0, F rows each) with a = silu(gate) * up formed in the epilogue and
    returned in f32 [F] (the input of an f32-input down projection, which quantizes it). x as for
    q8_gateup_silu_quantize: int8 codes [K] with dx, or f32 [K] with gamma and eps."""
    if w_gate.dim() != 2 or w_up.shape != w_gate.shape:
        raise ValueError("w_gate and w_up must both be [F, K]")
    f, k = w_gate.shape
    if a is None:
        a = torch.empty(f, dtype=torch.float32, device=w_gate.device)
    lib = load_library()
    common = (_ptr(w_gate, "w_gate", _I8), _ptr(dw_gate, "dw_gate", _H16, (f, k // 32)), _ptr(w_up, "w_up", _I8),
              _ptr(dw_up, "dw_up", _H16, (f, k // 32)), f)
    if gamma is None:
        st = lib.q8_gateup_silu(*common, _ptr(x, "x", _I8, (k,)), _ptr(dx, "dx", _H16, (k // 32,)), k,
                                _ptr(a, "a", _F32, (f,)), _stream(stream))
        fn = "q8_gateup_silu"
    else:
        if eps is None:
            raise ValueError("eps is required with gamma")
        st = lib.q8_gateup_rmsnorm_silu(*common, _ptr(x, "x", _F32, (k,)), _ptr(gamma, "gamma", _F32, (k,)),
                                        float(eps), k, _ptr(a, "a", _F32, (f,)), _stream(stream))
        fn = "q8_gateup_rmsnorm_silu"
    _check(fn, st)
    return a


def _q8_parts(parts, k):
    arr = (_Part * len(parts))()
    outs = []
    for i, p in enumerate(parts):
        w = p["w"]
        if w.dim() != 2 or w.shape[1] != k:
            raise ValueError(f"part {i}: w must be [n, {k}]")
        n = w.shape[0]
        y = p.get("y")
        if y is None:
            y = torch.empty(n, dtype=torch.float32, device=w.device)
        outs.append(y)
        arr[i].w = _ptr(w, f"parts[{i}].w", _I8)
        arr[i].dw = _ptr(p.get("dw"), f"parts[{i}].dw", _H16, (n, k // 32))
        arr[i].n = n
        arr[i].y = _ptr(y, f"parts[{i}].y", _F32, (n,))
        arr[i].residual = _ptr(p.get("residual"), f"parts[{i}].residual", _F32, (n,), optional=True)
    return arr, outs


def probe_read(buf, sink, stream=None):
    """Stream-read every byte of `buf` once (the measured read ceiling)."""
    st = load_library().q8g_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                       _stream(stream))
    _check("q8g_probe_read", st)


def probe_read_cached(buf, sink, stream=None):
    """Read every byte of `buf` once with plain (cached) loads (counter calibration)."""
    st = load_library().q8g_probe_read_cached(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                              _stream(stream))
    _check("q8g_probe_read_cached", st)


def flush(buf, value: int = 0, stream=None):
    """Overwrite `buf` (evicts the caches before a cold-cache timing)."""
    st = load_library().q8g_flush(buf.data_ptr(), buf.numel() * buf.element_size(), value & 0xFFFFFFFF,
                                  _stream(stream))
    _check("q8g_flush", st)


def gemv_config(dtype: int, n_total: int, k: int):
    """(rows per wave, waves per workgroup) the library launches a GEMV of n_total rows with."""
    r, w = ctypes.c_int(), ctypes.c_int()
    _check("q8g_gemv_config", load_library().q8g_gemv_config(dtype, n_total, k, ctypes.byref(r), ctypes.byref(w)))
    return r.value, w.value


class DecodeStackPlan:
    """Descriptors of a sequence of stacked Q8_0 projections for q8_decode_stack.

    ops: sequence of dicts with keys x (f32 [K]), parts (list of dicts with w, dw, y and
    optional residual, as for gemv_stacked), and optional qx / dx (outputs for the codes
    and scales). The host descriptor array, its device copy and the synchronization
    workspace (zero-filled here) are kept by the plan; tensors must stay alive with it.
    """

    def __init__(self, ops, device="cuda"):
        n = len(ops)
        arr = (_StackOp * max(1, n))()
        self._keep = []
        for i, op in enumerate(ops):
            x = op["x"]
            k = x.shape[0]
            arr[i].x = _ptr(x, f"ops[{i}].x", _F32, (k,))
            arr[i].qx = _ptr(op.get("qx"), f"ops[{i}].qx", _I8, (k,), optional=True)
            arr[i].dx = _ptr(op.get("dx"), f"ops[{i}].dx", _H16, (k // 32,), optional=True)
            arr[i].K = k
            parts = op["parts"]
            if not 1 <= len(parts) <= MAX_PARTS:
                raise ValueError("1 to 4 parts per op")
            arr[i].nparts = len(parts)
            arr[i].reserved = 0
            for j, p in enumerate(parts):
                w = p["w"]
                nrow = w.shape[0]
                arr[i].parts[j].w = _ptr(w, f"ops[{i}].parts[{j}].w", _I8, (nrow, k))
                arr[i].parts[j].dw = _ptr(p["dw"], f"ops[{i}].parts[{j}].dw", _H16, (nrow, k // 32))
                arr[i].parts[j].n = nrow
                arr[i].parts[j].y = _ptr(p["y"], f"ops[{i}].parts[{j}].y", _F32, (nrow,))
                arr[i].parts[j].residual = _ptr(p.get("residual"), f"ops[{i}].parts[{j}].residual", _F32, (nrow,),
                                                optional=True)
            self._keep.append(op)
        self.nops = n
        self.host = arr
        raw = bytes(memoryview(arr))[: n * ctypes.sizeof(_StackOp)] if n else b"\0"
        self.dev = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device)
        self.sync = torch.zeros(STACK_SYNC_WORDS, dtype=torch.int32, device=device)

    def run(self, stream=None):
        """Enqueue one launch of all projections."""
        st = load_library().q8_decode_stack(self.host, self.dev.data_ptr(), self.nops, self.sync.data_ptr(),
                                            _stream(stream))
        _check("q8_decode_stack", st)

    def run_static(self, stream=None, status=None):
        """Enqueue one launch through q8_decode_stack_static: the library's own static
        workspace instead of self.sync (cleared by the call itself). status: None or an
        int32 device tensor of one element that a launch which gave up waiting sets to 1."""
        sp = _ptr(status, "status", (torch.int32,), (1,), optional=True)
        st = load_library().q8_decode_stack_static(self.host, self.dev.data_ptr(), self.nops, sp, _stream(stream))
        _check("q8_decode_stack_static", st)

    def error_flag(self) -> int:
        """Nonzero if a launch gave up waiting at a barrier (synchronizes)."""
        return int(self.sync[STACK_ERR_WORD].item())
