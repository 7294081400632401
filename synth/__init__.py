"""Seeded synthetic inputs for the decode-step GEMV, shared by the oracle and the HIP path.

This module draws random numbers and encodes them into the storage formats the
two sides consume (int8 codes, IEEE binary16 bits, bf16 bits, f32). It holds
none of the method's arithmetic: no quantization of activations, no dot
products, no scaling. The stored bits it returns are the truth for both sides.

Value distributions follow the decode workloads of "Filling in the blanks:
Inference using Phobos" (§Fast Decode: Q8_0 weights, one scale per 32-element
block, activation quantized once) and "One level down: #002 the same compiler
on a GPU" (§Emitting for a GPU: the bf16 gate+up projection, 1024->7168 on the
0.8B model, 2560->18432 on the 4B model):

* Q8_0 weight codes: uniform integers in [-127, 127].
* Q8_0 weight scales: |N(0, 1)| * 0.02 / 127 in f32, then rounded to binary16.
* Q8_0 activation: N(0, 1) in f32 (quantized later by the method itself).
* bf16 weights: N(0, 1) * 0.02 in f32, rounded to bf16 (nearest, ties to even).
* bf16 activation: N(0, 1) in f32, rounded to bf16.
* f16 weights / activation: as bf16, rounded to IEEE binary16 instead.
* residual: N(0, 1) in f32.
* normalization input: N(0, 1) in f32; its weights gamma: 1 + 0.1 N(0, 1).
* gated activation input [gate | up]: gate 2 N(0, 1), up N(0, 1), in f32.
* PTQ1_0 ternary weights ("Filling in the blanks", §PrismML Ternary-Bonsai: weights -1, 0
  or +1, 128 of them in 28 bytes): trits uniform over {-1, 0, +1}; one scale per 128
  weights, |N(0, 1)| * 0.02 in f32 rounded to binary16; packed as 26 bytes of base-3 digits
  (digit = trit + 1, five per byte, least significant first) followed by the scale bits,
  little-endian (the layout reading is stated in the design notes).

Every matrix j of workload `tag` draws from
``np.random.default_rng(np.random.SeedSequence([tag, j]))`` in the order
weights, scales, activation, residual.
"""
from __future__ import annotations

import dataclasses

import numpy as np

QBLOCK = 32  # elements per Q8_0 block

# Workload tags (first SeedSequence word).
TAG_Q8_GATEUP = 0
TAG_BF16_GATEUP = 1
TAG_Q8_STACK = 2
TAG_BF16_4B_GATEUP = 3
TAG_Q8_HEAD = 4
TAG_F16_GATEUP = 5
TAG_Q8_BATCH = 6
TAG_NEIGHBOUR = 7
TAG_LAYERS = 8
TAG_PTQ1 = 9
TAG_TEST = 100

PTQ1_BLOCK = 128  # weights per PTQ1_0 block
PTQ1_BYTES = 28   # bytes per PTQ1_0 block: 26 of base-3 digits, 2 of binary16 scale


def rng_for(tag: int, j: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(tag), int(j)]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to bf16 storage bits, nearest with ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round f32 values to IEEE binary16 storage bits (numpy's nearest-even cast)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def q8_weights(rng: np.random.Generator, n: int, k: int):
    """(codes int8 [n, k], scale bits uint16 [n, k/32])."""
    if k % QBLOCK:
        raise ValueError("k must be a multiple of 32")
    qw = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    s = np.abs(rng.standard_normal((n, k // QBLOCK), dtype=np.float32))
    s *= np.float32(0.02 / 127.0)
    return qw, f32_to_f16_bits(s)


def ptq1_pack(trits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Encode ternary weights trits int8 [n, k] (-1, 0, +1) with scale bits uint16
    [n, k/128] into PTQ1_0 rows uint8 [n, 28 k/128]."""
    n, k = trits.shape
    if k % PTQ1_BLOCK:
        raise ValueError("k must be a multiple of 128")
    nb = k // PTQ1_BLOCK
    digits = np.zeros((n, nb, 130), np.int32)  # 26 bytes of five digit slots
    digits[..., :PTQ1_BLOCK] = trits.reshape(n, nb, PTQ1_BLOCK).astype(np.int32) + 1
    place = np.array([1, 3, 9, 27, 81], np.int32)
    packed = (digits.reshape(n, nb, 26, 5) * place).sum(axis=-1)
    out = np.empty((n, nb, PTQ1_BYTES), np.uint8)
    out[..., :26] = packed.astype(np.uint8)
    sb = np.asarray(scale_bits, dtype=np.uint16).reshape(n, nb)
    out[..., 26] = (sb & 0xFF).astype(np.uint8)
    out[..., 27] = (sb >> 8).astype(np.uint8)
    return out.reshape(n, nb * PTQ1_BYTES)


def ptq1_weights(rng: np.random.Generator, n: int, k: int):
    """(PTQ1_0 rows uint8 [n, 28 k/128], trits int8 [n, k], scale bits uint16 [n, k/128])."""
    if k % PTQ1_BLOCK:
        raise ValueError("k must be a multiple of 128")
    t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    s = np.abs(rng.standard_normal((n, k // PTQ1_BLOCK), dtype=np.float32))
    s *= np.float32(0.02)
    sb = f32_to_f16_bits(s)
    return ptq1_pack(t, sb), t, sb


def activation_f32(rng: np.random.Generator, k: int) -> np.ndarray:
    return rng.standard_normal(k, dtype=np.float32)


def bf16_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(0.02)
    return f32_to_bf16_bits(w)


def bf16_activation(rng: np.random.Generator, k: int) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(k, dtype=np.float32))


def f16_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(0.02)
    return f32_to_f16_bits(w)


def f16_activation(rng: np.random.Generator, k: int) -> np.ndarray:
    return f32_to_f16_bits(rng.standard_normal(k, dtype=np.float32))


def residual_f32(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.standard_normal(n, dtype=np.float32)


def norm_gamma(rng: np.random.Generator, k: int) -> np.ndarray:
    """Per-channel RMS-normalization weights: 1 + 0.1 N(0, 1)."""
    g = rng.standard_normal(k, dtype=np.float32)
    g *= np.float32(0.1)
    g += np.float32(1.0)
    return g


def gate_up_f32(rng: np.random.Generator, k: int) -> np.ndarray:
    """[gate | up] f32 [2k]: gate 2 N(0, 1) (both arms of silu), up N(0, 1)."""
    gate = rng.standard_normal(k, dtype=np.float32)
    gate *= np.float32(2.0)
    return np.concatenate([gate, rng.standard_normal(k, dtype=np.float32)])


# ---------------------------------------------------------------------------
# Workload shapes


@dataclasses.dataclass(frozen=True)
class Gemv:
    """One projection of a decode step: ``parts`` output-row counts sharing one input of length k."""

    name: str
    parts: tuple
    k: int
    residual: bool = False

    @property
    def n(self) -> int:
        return int(sum(self.parts))


def q8_stack_08b(layers: int = 24, hidden: int = 1024, vocab: int = 151936):
    """The 0.8B-shaped Q8_0 decode stack: per layer QKV 1024->4096 (stacked 2048/1024/1024),
    out 2048->1024, gate+up 1024->7168 (stacked 3584/3584), down 3584->1024 with the residual
    folded in; then the output head 1024->151936."""
    ops = []
    for l in range(layers):
        ops.append(Gemv(f"L{l}.qkv", (2048, 1024, 1024), hidden))
        ops.append(Gemv(f"L{l}.out", (hidden,), 2048))
        ops.append(Gemv(f"L{l}.gateup", (3584, 3584), hidden))
        ops.append(Gemv(f"L{l}.down", (hidden,), 3584, residual=True))
    ops.append(Gemv("head", (vocab,), hidden))
    return ops


def layer_chain_inputs(layers: int = 24, hidden: int = 1024, attn_width: int = 2048, tag: int = TAG_LAYERS):
    """Seeded inputs of the decode-layer chain: the residual stream entering layer 0, per layer
    the two normalization weight vectors and the attention output (a stand-in: attention is not
    part of this path), and the final normalization's weights."""
    g = rng_for(tag, 0)
    out = {"h": activation_f32(g, hidden), "gamma_attn": [], "gamma_mlp": [], "attn": []}
    for _ in range(layers):
        out["gamma_attn"].append(norm_gamma(g, hidden))
        out["gamma_mlp"].append(norm_gamma(g, hidden))
        out["attn"].append(activation_f32(g, attn_width))
    out["gamma_final"] = norm_gamma(g, hidden)
    return out


def layer_chain_batch_inputs(nb: int, layers: int = 24, hidden: int = 1024, attn_width: int = 2048,
                             tag: int = TAG_LAYERS):
    """Per-stream inputs of the batched decode-layer chain: the residual streams entering
    layer 0, f32 [nb, hidden], and per layer the attention stand-ins, f32 [nb, attn_width]."""
    g = rng_for(tag, 1)
    h = np.stack([activation_f32(g, hidden) for _ in range(nb)])
    attn = [np.stack([activation_f32(g, attn_width) for _ in range(nb)]) for _ in range(layers)]
    return {"h": h, "attn": attn}


def q8_gemv_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic HBM bytes of one Q8_0 GEMV: codes + scales + quantized activation + f32 out (+ residual)."""
    b = n * k + n * (k // QBLOCK) * 2 + k + (k // QBLOCK) * 2 + n * 4
    return b + (n * 4 if residual else 0)


def q8_gemv_f32x_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic HBM bytes of one Q8_0 GEMV that reads its activation as f32 and
    quantizes it in the same launch: codes + scales + f32 activation + f32 out (+ residual)."""
    b = n * k + n * (k // QBLOCK) * 2 + 4 * k + n * 4
    return b + (n * 4 if residual else 0)


def q8_batch_gemv_bytes(n: int, k: int, nb: int, residual: bool = False) -> int:
    """Algorithmic HBM bytes of one small-batch Q8_0 GEMV over nb vectors: the weights
    once, each vector's quantized activation, f32 outputs (and residuals)."""
    b = n * k + n * (k // QBLOCK) * 2 + nb * (k + (k // QBLOCK) * 2) + nb * n * 4
    return b + (nb * n * 4 if residual else 0)


def q8_rmsnorm_gemv_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic bytes of a Q8_0 GEMV that normalizes its f32 input in the same
    launch: q8_gemv_f32x_bytes plus the f32 normalization weights."""
    return q8_gemv_f32x_bytes(n, k, residual) + 4 * k


def q8_silu_gemv_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic bytes of a Q8_0 GEMV that forms silu(gate) * up from f32 [2k] in the
    same launch: q8_gemv_f32x_bytes plus the second f32 half."""
    return q8_gemv_f32x_bytes(n, k, residual) + 4 * k


def q8_gateup_epilogue_bytes(f: int, k: int) -> int:
    """Algorithmic bytes of the gate+up launch with the normalization in its prologue and
    silu(gate) * up quantized in its epilogue: both weight planes of 2f rows, x and gamma
    f32 [k], codes [f] and binary16 scales [f/32] out."""
    return 2 * f * k + 2 * (2 * f) * (k // QBLOCK) + 8 * k + f + 2 * (f // QBLOCK)


def q8_gateup_silu_f32_bytes(f: int, k: int) -> int:
    """Algorithmic bytes of the gate+up launch with the normalization in its prologue and
    a = silu(gate) * up written in f32 in its epilogue: both weight planes of 2f rows, x and
    gamma f32 [k], a f32 [f] out."""
    return 2 * f * k + 2 * (2 * f) * (k // QBLOCK) + 8 * k + 4 * f


def q8_layers_08b_bytes(layers: int = 24, hidden: int = 1024, ffn: int = 3584, vocab: int = 151936) -> int:
    """Algorithmic bytes of one token of the fused decode-layer chain: per layer the QKV launch
    with its normalization, the out projection (f32 input, residual), the gate+up launch with
    its f32 epilogue (a = silu(gate) * up written in f32) and the down projection (f32 input,
    residual); then the head with the final normalization in its prologue."""
    per_layer = (q8_rmsnorm_gemv_bytes(4096, hidden) + q8_gemv_f32x_bytes(hidden, 2048, residual=True)
                 + q8_gateup_silu_f32_bytes(ffn, hidden) + q8_gemv_f32x_bytes(hidden, ffn, residual=True))
    return layers * per_layer + q8_rmsnorm_gemv_bytes(vocab, hidden)


def q8_quantize_bytes(k: int) -> int:
    """Algorithmic bytes of one activation quantize: f32 in, int8 codes + binary16 scales out."""
    return 4 * k + k + (k // QBLOCK) * 2


def bf16_gemv_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic bytes of one 16-bit (bf16 or f16) GEMV."""
    b = 2 * n * k + 2 * k + 4 * n
    return b + (n * 4 if residual else 0)


def ptq1_rotate_bytes(k: int) -> int:
    """Algorithmic bytes of one rotate + quantize of a PTQ1_0 input: f32 in, codes + scales out."""
    return 4 * k + k + (k // PTQ1_BLOCK) * 2


def ptq1_gemv_bytes(n: int, k: int, residual: bool = False) -> int:
    """Algorithmic bytes of one PTQ1_0 GEMV: 28-byte blocks + rotated codes and scales + f32 out (+ residual)."""
    b = n * (k // PTQ1_BLOCK) * PTQ1_BYTES + k + (k // PTQ1_BLOCK) * 2 + n * 4
    return b + (n * 4 if residual else 0)


def q8_stack_inputs(ops, tag: int = TAG_Q8_STACK):
    """Seeded host inputs for each projection j of a stack: codes, scale bits, f32 input,
    and a residual where the projection folds one in."""
    host = []
    for j, op in enumerate(ops):
        g = rng_for(tag, j)
        qw, dw = q8_weights(g, op.n, op.k)
        x = activation_f32(g, op.k)
        r = residual_f32(g, op.n) if op.residual else None
        host.append({"qw": qw, "dw": dw, "x": x, "r": r})
    return host


def q8_batch_inputs(ops, nb: int, tag: int = TAG_Q8_BATCH):
    """Seeded activation vectors [nb, k] (and residuals [nb, n] where the projection folds
    one in) for each projection j of a stack, for nb decode streams at once."""
    out = []
    for j, op in enumerate(ops):
        g = rng_for(tag, j)
        x = np.stack([activation_f32(g, op.k) for _ in range(nb)])
        r = np.stack([residual_f32(g, op.n) for _ in range(nb)]) if op.residual else None
        out.append({"x": x, "r": r})
    return out
