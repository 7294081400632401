"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch. They are
run against the real oracle (test_oracle.py) and against deliberately broken copies
of it (test_oracle_mutants.py), which must each fail at least one pin.

Independent references used here (none calls into the oracle; the PTQ1_0 packing of
synth.ptq1_pack is the encoder the oracle's decoder is checked against):
  * numpy's own binary16 cast and f32 bit reinterpretation for bf16;
  * a numpy float32 quantizer (IEEE f32 division, np.rint ties-to-even);
  * Python integers and fractions.Fraction for exact block sums and dot products;
  * numpy f64 matmul of the dequantized operands;
  * closed forms that follow from the definitions ("Filling in the blanks: Inference
    using Phobos", section Fast Decode: 32 int8 values with their own scale, the
    block math in int8; "One level down: #002 the same compiler on a GPU", section
    The numerical contract: bf16 in, f32 accumulate);
  * for PTQ1_0 ("Filling in the blanks", section PrismML Ternary-Bonsai: ternary
    weights, 128 in 28 bytes, a Hadamard-rotated activation): scipy's Sylvester
    Hadamard matrix with exactly rounded sums (math.fsum), the rotation's closed forms
    (one-hot and constant blocks, the rotation being its own inverse, norm kept), and
    its stated purpose (an outlier spread over the block quantizes with less error).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import synth

QB = 32


# ----------------------------------------------------------------------------- helpers


def np_f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def np_bf16(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_quantize(x, block=QB):
    """Independent quantizer: numpy f32 division and np.rint (round half to even)."""
    xb = np.asarray(x, dtype=np.float32).reshape(-1, block)
    amax = np.abs(xb).max(axis=1)
    d = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xb / d[:, None]).astype(np.float32)
    q = np.clip(np.rint(t), -127, 127)
    q = np.where(d[:, None] == 0, 0, q).astype(np.int8)
    dx = d.astype(np.float16).view(np.uint16)
    return q.ravel(), dx


def dequant_rows(qw, dw):
    n, k = qw.shape
    return qw.astype(np.float64) * np.repeat(np_f16(dw).reshape(n, k // QB), QB, axis=1)


def rng(j):
    return synth.rng_for(synth.TAG_TEST, j)


def close_to(y, ref, S, rel):
    err = np.abs(np.asarray(y) - np.asarray(ref))
    bad = err > rel * np.asarray(S) + 1e-300
    assert not bad.any(), f"max err {err.max()} vs bound {rel} * S (first bad row {np.argmax(bad)})"


# ----------------------------------------------------------------------------- number formats


def pin_f16_decoder_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = o.f16_value(bits)
    ref = np_f16(bits)
    assert np.array_equal(ours, ref, equal_nan=True)


def pin_bf16_decoder_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = o.bf16_value(bits)
    ref = np_bf16(bits)
    assert np.array_equal(ours, ref, equal_nan=True)


def pin_f16_encoder_vs_numpy(o):
    g = rng(1)
    vals = [
        g.standard_normal(2000).astype(np.float32),
        (g.standard_normal(2000) * 1e-6).astype(np.float32),  # subnormal binary16 range
        (g.standard_normal(2000) * 3e4).astype(np.float32),  # near overflow
        np.float32([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e6, 2.0**-24, 2.0**-25,
                    3 * 2.0**-26, 2.0**-14, 2.0**-14 - 2.0**-25]),
    ]
    # exact half-way points between adjacent binary16 values (representable in f32)
    h = g.integers(1, 0x7BFF, 2000).astype(np.uint16)
    lo = np_f16(h)
    hi = np_f16(h + 1)
    vals.append(((lo + hi) / 2).astype(np.float32))
    vals.append((-(lo + hi) / 2).astype(np.float32))
    x = np.concatenate(vals)
    ours = o.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref), f"{np.count_nonzero(ours != ref)} mismatches, e.g. x={x[ours != ref][:4]}"


# ----------------------------------------------------------------------------- quantizer


def _quant_inputs():
    g = rng(2)
    blocks = [
        g.standard_normal(4096).astype(np.float32),
        # log-uniform magnitudes over a wide range, random signs
        (np.exp(g.uniform(-30, 30, 4096)) * g.choice([-1, 1], 4096)).astype(np.float32),
        # small blocks: activation scales in the binary16 subnormal range
        (g.standard_normal(1024) * 1e-4).astype(np.float32),
        (g.standard_normal(1024) * 1e-7).astype(np.float32),
        # sparse blocks with zeros
        (g.standard_normal(1024) * (g.random(1024) < 0.2)).astype(np.float32),
    ]
    return np.concatenate(blocks)


def pin_quantizer_vs_numpy_f32(o):
    x = _quant_inputs()
    qx, dx = o.quantize_act(x)
    rq, rd = np_quantize(x)
    assert np.array_equal(qx, rq), f"{np.count_nonzero(qx != rq)} code mismatches"
    assert np.array_equal(dx, rd), f"{np.count_nonzero(dx != rd)} scale mismatches"


def pin_quantizer_near_ties(o):
    """Values that sit next to a rounding boundary of x/d, chosen where the plausible
    alternative x*(1/d) rounds differently; the division form decides."""
    g = rng(3)
    found = []
    for _ in range(200):
        amax = np.float32(np.exp(g.uniform(-5, 5)))
        d = np.float32(amax / np.float32(127))
        inv = np.float32(np.float32(1) / d)
        ks = g.integers(-126, 126, 4000)
        cand = ((ks + 0.5) * d.astype(np.float64)).astype(np.float32)
        cand = np.concatenate([cand, np.nextafter(cand, np.float32(np.inf)), np.nextafter(cand, np.float32(-np.inf))])
        a = np.rint(cand / d)
        b = np.rint(cand * inv)
        sel = cand[(a != b) & (np.abs(cand) < amax)]
        for v in sel[:3]:
            found.append((amax, v))
        if len(found) >= 32:
            break
    assert len(found) >= 8, "could not build near-tie cases"
    x = np.zeros(32 * len(found), np.float32)
    for i, (amax, v) in enumerate(found):
        x[32 * i] = amax
        x[32 * i + 1] = v
    qx, dx = o.quantize_act(x)
    rq, rd = np_quantize(x)
    assert np.array_equal(qx, rq) and np.array_equal(dx, rd)


def pin_quantizer_closed_forms(o):
    # constant block c != 0: every code is +-127, scale binary16(|c|/127)
    for c in (1.0, -3.25, 1e-3, 7e4, -2.0**-20):
        x = np.full(32, c, np.float32)
        qx, dx = o.quantize_act(x)
        assert np.all(qx == (127 if c > 0 else -127))
        assert dx[0] == np.float16(np.float32(abs(np.float32(c))) / np.float32(127)).view(np.uint16)
    # one-hot block: +-127 at the hot index, zero elsewhere
    for i, v in ((0, 2.5), (17, -0.001), (31, 9.0)):
        x = np.zeros(32, np.float32)
        x[i] = v
        qx, _ = o.quantize_act(x)
        expect = np.zeros(32, np.int8)
        expect[i] = 127 if v > 0 else -127
        assert np.array_equal(qx, expect)
    # all-zero block: zero codes and a zero scale
    qx, dx = o.quantize_act(np.zeros(64, np.float32))
    assert not qx.any() and not dx.any()
    # ties: with 127 in the block d = 1 exactly, so x/d = x; halves round to even
    vals = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 125.5, 126.5, -126.5, 0.49999997, 63.5]
    expect = [0, 2, 2, 0, -2, -2, 4, 126, 126, -126, 0, 64]
    x = np.zeros(32, np.float32)
    x[0] = 127.0
    x[1:1 + len(vals)] = vals
    qx, dx = o.quantize_act(x)
    assert dx[0] == 0x3C00
    assert qx[0] == 127 and list(qx[1:1 + len(vals)]) == expect, list(qx[1:1 + len(vals)])


def pin_quantizer_properties(o):
    x = _quant_inputs()[:4096]
    qx, dx = o.quantize_act(x)
    # sign symmetry
    qn, dn = o.quantize_act(-x)
    assert np.array_equal(qn, -qx) and np.array_equal(dn, dx)
    # round trip: |x - q*d| <= d/2 with the f32 scale (plus one rounding of x/d)
    d = (np.abs(x.reshape(-1, QB)).max(axis=1) / np.float32(127)).astype(np.float64)
    err = np.abs(x.reshape(-1, QB).astype(np.float64) - qx.reshape(-1, QB) * d[:, None])
    assert np.all(err <= d[:, None] * (0.5 + 2.0**-20) + 1e-300)
    # codes are within [-127, 127] and the block maximum hits +-127
    assert qx.min() >= -127 and qx.max() <= 127
    nz = d > 0
    assert np.all(np.abs(qx.reshape(-1, QB)).max(axis=1)[nz] == 127)


# ----------------------------------------------------------------------------- block integer dot


def pin_block_isums_brute_force(o):
    g = rng(4)
    n, k = 5, 96
    qw = g.integers(-128, 128, (n, k), dtype=np.int8)
    qx = g.integers(-128, 128, k, dtype=np.int8)
    got = o.block_isums(qw, qx)
    for r in range(n):
        for b in range(k // QB):
            s = sum(int(qw[r, QB * b + i]) * int(qx[QB * b + i]) for i in range(QB))
            assert got[r, b] == s


def pin_block_isums_closed_forms(o):
    ones = np.ones((1, 32), np.int8)
    assert o.block_isums(ones, ones[0])[0, 0] == 32
    p = np.full((1, 32), 127, np.int8)
    assert o.block_isums(p, p[0])[0, 0] == 516128
    assert o.block_isums(p, -p[0])[0, 0] == -516128
    m = np.full((1, 32), -128, np.int8)
    assert o.block_isums(m, m[0])[0, 0] == 524288
    alt = np.array([[1, -1] * 16], np.int8)
    assert o.block_isums(alt, np.ones(32, np.int8))[0, 0] == 0
    # a block sees only its own 32 elements
    w = np.zeros((1, 64), np.int8)
    w[0, 32:] = 1
    x = np.arange(64, dtype=np.int8)
    assert list(o.block_isums(w, x)[0]) == [0, sum(range(32, 64))]


# ----------------------------------------------------------------------------- Q8_0 GEMV


def _q8_case(j, n, k, resid=True):
    g = rng(j)
    qw, dw = synth.q8_weights(g, n, k)
    x = synth.activation_f32(g, k)
    r = synth.residual_f32(g, n) if resid else None
    return qw, dw, x, r


def pin_q8_exact_rational(o):
    qw, dw, x, r = _q8_case(5, 4, 96)
    qx, dx = o.quantize_act(x)
    y, S = o.q8_gemv(qw, dw, qx, dx, r)
    for row in range(4):
        ex = Fraction(0)
        for b in range(3):
            isum = sum(int(qw[row, QB * b + i]) * int(qx[QB * b + i]) for i in range(QB))
            ex += isum * Fraction(float(np_f16(dw[row, b]))) * Fraction(float(np_f16(dx[b])))
        ex += Fraction(float(r[row]))
        assert abs(Fraction(y[row]) - ex) <= Fraction(4 * 2.0**-53) * Fraction(S[row])


def pin_q8_vs_dense_dequant(o):
    for j, (n, k) in enumerate(((64, 1024), (33, 3584), (7, 5120))):
        qw, dw, x, r = _q8_case(10 + j, n, k, resid=(j == 1))
        qx, dx = o.quantize_act(x)
        y, S = o.q8_gemv(qw, dw, qx, dx, r)
        ref = dequant_rows(qw, dw) @ (qx.astype(np.float64) * np.repeat(np_f16(dx), QB))
        if r is not None:
            ref = ref + r.astype(np.float64)
        close_to(y, ref, S, k * 2.0**-52)
        absref = np.abs(dequant_rows(qw, dw)) @ np.abs(qx.astype(np.float64) * np.repeat(np_f16(dx), QB))
        if r is not None:
            absref = absref + np.abs(r.astype(np.float64))
        close_to(S, absref, absref, k * 2.0**-52)


def pin_q8_closed_forms(o):
    g = rng(6)
    n, k = 6, 256
    nb = k // QB
    # all-ones blocks: each block contributes 32 * dw * dx
    qw = np.ones((n, k), np.int8)
    qx = np.ones(k, np.int8)
    dw = synth.f32_to_f16_bits(np.abs(g.standard_normal((n, nb))).astype(np.float32) * np.float32(0.01))
    dx = synth.f32_to_f16_bits(np.abs(g.standard_normal(nb)).astype(np.float32))
    y, S = o.q8_gemv(qw, dw, qx, dx)
    ref = 32.0 * (np_f16(dw).reshape(n, nb) * np_f16(dx)[None, :]).sum(axis=1)
    close_to(y, ref, S, 8 * 2.0**-53)
    assert np.allclose(S, y, rtol=1e-15)
    # power-of-two scales: the sum is exact, so equality is bit-for-bit
    dw2 = np.full((n, nb), 0x3800, np.uint16)  # 0.5
    dx2 = np.full(nb, 0x4400, np.uint16)  # 4.0
    y2, _ = o.q8_gemv(qw, dw2, qx, dx2)
    assert np.all(y2 == 32 * nb * 2.0)
    # single-block isolation: only block b has a nonzero weight scale
    qw3, _, x3, _ = _q8_case(7, n, k, resid=False)
    qx3, dx3 = o.quantize_act(x3)
    isum = np.array([[sum(int(qw3[r_, QB * b + i]) * int(qx3[QB * b + i]) for i in range(QB))
                      for b in range(nb)] for r_ in range(n)])
    for b in (0, 3, nb - 1):
        dwb = np.zeros((n, nb), np.uint16)
        dwb[:, b] = 0x3C00 + np.arange(n, dtype=np.uint16)
        yb, _ = o.q8_gemv(qw3, dwb, qx3, dx3)
        assert np.array_equal(yb, isum[:, b] * np_f16(dwb[:, b]) * np_f16(dx3[b]))


def pin_q8_invariants(o):
    qw, dw, x, r = _q8_case(8, 40, 512)
    qx, dx = o.quantize_act(x)
    y, S = o.q8_gemv(qw, dw, qx, dx)
    # y(-W) = -y(W), bit-exact
    yn, Sn = o.q8_gemv(-qw, dw, qx, dx)
    assert np.array_equal(yn, -y) and np.array_equal(Sn, S)
    # doubling every weight scale doubles y exactly: a normal binary16 gains one in
    # its exponent field; a subnormal's bits double (carrying into the exponent)
    assert np.all((dw & 0x7C00) < 0x7800)
    dw2 = np.where((dw & 0x7C00) != 0, dw + 0x0400, dw * 2).astype(np.uint16)
    y2, _ = o.q8_gemv(qw, dw2, qx, dx)
    assert np.array_equal(y2, 2 * y)
    # a row permutation permutes y
    p = rng(9).permutation(40)
    yp, _ = o.q8_gemv(qw[p], dw[p], qx, dx)
    assert np.array_equal(yp, y[p])
    # -128 weights are exact
    qm = qw.copy()
    qm[:, ::7] = -128
    ym, Sm = o.q8_gemv(qm, dw, qx, dx)
    ref = dequant_rows(qm, dw) @ (qx.astype(np.float64) * np.repeat(np_f16(dx), QB))
    close_to(ym, ref, Sm, 512 * 2.0**-52)


def pin_q8_residual(o):
    qw, dw, x, r = _q8_case(11, 24, 256)
    qx, dx = o.quantize_act(x)
    y0, S0 = o.q8_gemv(np.zeros_like(qw), dw, qx, dx, r)
    assert np.array_equal(y0, r.astype(np.float64))
    assert np.array_equal(S0, np.abs(r.astype(np.float64)))
    y1, S1 = o.q8_gemv(qw, dw, qx, dx, r)
    y2, S2 = o.q8_gemv(qw, dw, qx, dx)
    close_to(y1, y2 + r, S1, 4 * 2.0**-53)
    assert np.allclose(S1, S2 + np.abs(r), rtol=1e-15)


# ----------------------------------------------------------------------------- bf16 GEMV


def pin_bf16_integer_valued(o):
    g = rng(12)
    n, k = 37, 1024
    wi = g.integers(-8, 9, (n, k))
    xi = g.integers(-8, 9, k)
    w = synth.f32_to_bf16_bits(wi.astype(np.float32))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    y, S = o.bf16_gemv(w, x)
    assert np.array_equal(y, (wi @ xi).astype(np.float64))
    assert np.array_equal(S, (np.abs(wi) @ np.abs(xi)).astype(np.float64))


def pin_bf16_vs_dense(o):
    for j, (n, k) in enumerate(((48, 1024), (19, 2560), (5, 8))):
        g = rng(13 + j)
        w = synth.bf16_weights(g, n, k)
        x = synth.bf16_activation(g, k)
        r = synth.residual_f32(g, n)
        y, S = o.bf16_gemv(w, x, r)
        W = np_bf16(w).reshape(n, k)
        X = np_bf16(x)
        close_to(y, W @ X + r, S, k * 2.0**-52)
        close_to(S, np.abs(W) @ np.abs(X) + np.abs(r), S, k * 2.0**-52)


def pin_bf16_exact_rational(o):
    g = rng(16)
    n, k = 3, 24
    w = synth.bf16_weights(g, n, k)
    x = synth.bf16_activation(g, k)
    y, S = o.bf16_gemv(w, x)
    W = np_bf16(w).reshape(n, k)
    X = np_bf16(x)
    for row in range(n):
        ex = sum(Fraction(float(W[row, i])) * Fraction(float(X[i])) for i in range(k))
        assert abs(Fraction(y[row]) - ex) <= Fraction(k * 2.0**-53) * Fraction(S[row])


def pin_bf16_residual(o):
    g = rng(17)
    w = np.zeros((9, 64), np.uint16)
    x = synth.bf16_activation(g, 64)
    r = synth.residual_f32(g, 9)
    y, S = o.bf16_gemv(w, x, r)
    assert np.array_equal(y, r.astype(np.float64))


# ----------------------------------------------------------------------------- small-batch Q8_0 GEMV


def _q8_batch_case(j, n, k, nb, resid=True):
    g = rng(j)
    qw, dw = synth.q8_weights(g, n, k)
    x = np.stack([synth.activation_f32(g, k) for _ in range(nb)])
    r = np.stack([synth.residual_f32(g, n) for _ in range(nb)]) if resid else None
    return qw, dw, x, r


def pin_q8_batch_unit_scales_exact(o):
    """All scales 1.0: y[b] = qx[b] . qw^T in integers, an exact int64 matmul."""
    g = rng(30)
    n, k, nb = 23, 160, 6
    qw = g.integers(-128, 128, (n, k)).astype(np.int8)
    qx = g.integers(-127, 128, (nb, k)).astype(np.int8)
    one = np.uint16(0x3C00)
    dw = np.full((n, k // QB), one, np.uint16)
    dx = np.full((nb, k // QB), one, np.uint16)
    y, S = o.q8_gemv_batch(qw, dw, qx, dx)
    W, X = qw.astype(np.int64), qx.astype(np.int64)
    assert np.array_equal(y, (X @ W.T).astype(np.float64))
    assert np.array_equal(S, (np.abs(X) @ np.abs(W).T).astype(np.float64))


def pin_q8_batch_vs_dense_dequant(o):
    for j, (n, k, nb) in enumerate(((40, 1024, 16), (9, 96, 3), (17, 2048, 5))):
        qw, dw, x, r = _q8_batch_case(31 + j, n, k, nb, resid=(j != 1))
        q = [np_quantize(v) for v in x]
        qx = np.stack([a for a, _ in q])
        dx = np.stack([d for _, d in q])
        y, S = o.q8_gemv_batch(qw, dw, qx, dx, r)
        W = dequant_rows(qw, dw)
        X = np.stack([dequant_rows(qx[i][None, :], dx[i][None, :])[0] for i in range(nb)])
        R = 0.0 if r is None else r.astype(np.float64)
        close_to(y, X @ W.T + R, S, (k // QB) * 2.0**-52)
        close_to(S, np.abs(X) @ np.abs(W).T + np.abs(R), S, (k // QB) * 2.0**-52)


def pin_q8_batch_rows_are_single_gemvs(o):
    """Vector b of a batch gives what the single-vector GEMV gives for qx[b]
    (both pinned independently above), with vectors kept apart."""
    qw, dw, x, r = _q8_batch_case(35, 21, 128, 4)
    q = [np_quantize(v) for v in x]
    qx = np.stack([a for a, _ in q])
    dx = np.stack([d for _, d in q])
    dx[2] = np.uint16(0x4000)  # a distinct scale plane per vector
    y, S = o.q8_gemv_batch(qw, dw, qx, dx, r)
    for b in range(4):
        yb, Sb = o.q8_gemv(qw, dw, qx[b], dx[b], r[b])
        assert np.array_equal(y[b], yb) and np.array_equal(S[b], Sb)
    for t in (2, 5):
        yt, St = o.q8_gemv_batch(qw, dw, qx, dx, r, nthreads=t)
        assert np.array_equal(yt, y) and np.array_equal(St, S)


# ----------------------------------------------------------------------------- neighbour steps


def np_rmsnorm(x, gamma, eps):
    """Independent RMS normalization: math.fsum of the squares (correctly rounded), numpy
    f32 multiplies in the same order (x * r, then * gamma)."""
    import math

    x = np.asarray(x, np.float32)
    ss = math.fsum(float(v) * float(v) for v in x)
    r = np.float32(1.0 / math.sqrt(ss / x.shape[0] + float(eps)))
    return (x * r).astype(np.float32) * np.asarray(gamma, np.float32)


def pin_rmsnorm_vs_independent(o):
    for j, k in enumerate((32, 1024, 3584, 5120)):
        g = rng(40 + j)
        x = g.standard_normal(k, dtype=np.float32) * np.float32(3.0)
        gamma = (1.0 + 0.1 * g.standard_normal(k)).astype(np.float32)
        for eps in (1e-6, 1e-2):
            h = o.rmsnorm(x, gamma, eps)
            ref = np_rmsnorm(x, gamma, eps)
            assert np.array_equal(h.view(np.uint32), ref.view(np.uint32)), (k, eps, np.count_nonzero(h != ref))


def pin_rmsnorm_closed_forms(o):
    k = 64
    ones = np.ones(k, np.float32)
    # a constant vector c = +-2^e with eps = 0 normalizes to exactly +-1
    for c in (1.0, -4.0, 2.0**-20, 2.0**30):
        h = o.rmsnorm(np.full(k, c, np.float32), ones, 0.0)
        assert np.all(h == np.float32(np.sign(c))), (c, h[:3])
    # with eps = 0, scaling x by 2^e changes nothing, bit for bit
    g = rng(45)
    x = g.standard_normal(k, dtype=np.float32)
    gamma = g.standard_normal(k, dtype=np.float32)
    h = o.rmsnorm(x, gamma, 0.0)
    for e in (-40, -3, 5, 60):
        assert np.array_equal(o.rmsnorm(x * np.float32(2.0**e), gamma, 0.0), h)
    # gamma enters linearly: doubling it doubles h exactly
    assert np.array_equal(o.rmsnorm(x, gamma * np.float32(2), 0.0), h * np.float32(2))
    # eps dominating a tiny input: r rounds to 1 in f32, h = x * gamma exactly
    tiny = (x * np.float32(1e-20)).astype(np.float32)
    assert np.array_equal(o.rmsnorm(tiny, gamma, 1.0), tiny * gamma)


def np_silu_mul(gu):
    gu = np.asarray(gu, np.float32)
    k = gu.shape[0] // 2
    gt, up = gu[:k].astype(np.float64), gu[k:].astype(np.float64)
    with np.errstate(over="ignore"):
        return ((gt * up) / (1.0 + np.exp(-gt))).astype(np.float32)


def pin_silu_mul_vs_independent(o):
    g = rng(46)
    for k in (32, 3584):
        gu = (g.standard_normal(2 * k) * 3.0).astype(np.float32)
        a = o.silu_mul(gu)
        ref = np_silu_mul(gu)
        assert np.array_equal(a.view(np.uint32), ref.view(np.uint32)), np.count_nonzero(a != ref)


def pin_silu_mul_closed_forms(o):
    k = 8
    up = np.float32([1.5, -2.0, 3.0, 0.25, 7.0, -1.0, 100.0, 0.5])
    # gate 0 gives 0; up 0 gives 0
    assert np.all(o.silu_mul(np.concatenate([np.zeros(k, np.float32), up])) == 0)
    gate = np.float32([0.5, -3.0, 2.0, 9.0, -0.1, 4.0, 1.0, -7.0])
    assert np.all(o.silu_mul(np.concatenate([gate, np.zeros(k, np.float32)])) == 0)
    # large gate: exp(-g) vanishes against 1 in f64, so a = f32(g * u) exactly
    big = np.float32([100.0, 250.0, 90.0, 1000.0, 120.0, 800.0, 64.0, 3e4])
    assert np.array_equal(o.silu_mul(np.concatenate([big, up])),
                          (big.astype(np.float64) * up.astype(np.float64)).astype(np.float32))
    # very negative gate: exp(-g) overflows, a is a signed zero
    assert np.all(o.silu_mul(np.concatenate([-big * np.float32(10), up])) == 0)
    # silu(g) - silu(-g) = g, so a(g, u) - a(-g, u) = g * u up to rounding
    d = o.silu_mul(np.concatenate([gate, up])).astype(np.float64) - \
        o.silu_mul(np.concatenate([-gate, up])).astype(np.float64)
    assert np.allclose(d, gate.astype(np.float64) * up, rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------------------- f16 GEMV


def pin_f16_integer_valued(o):
    g = rng(20)
    n, k = 29, 1024
    wi = g.integers(-8, 9, (n, k))
    xi = g.integers(-8, 9, k)
    w = synth.f32_to_f16_bits(wi.astype(np.float32))
    x = synth.f32_to_f16_bits(xi.astype(np.float32))
    y, S = o.f16_gemv(w, x)
    assert np.array_equal(y, (wi @ xi).astype(np.float64))
    assert np.array_equal(S, (np.abs(wi) @ np.abs(xi)).astype(np.float64))


def pin_f16_vs_dense(o):
    for j, (n, k) in enumerate(((48, 1024), (19, 2560), (5, 8))):
        g = rng(21 + j)
        w = synth.f16_weights(g, n, k)
        x = synth.f16_activation(g, k)
        r = synth.residual_f32(g, n)
        y, S = o.f16_gemv(w, x, r)
        W = np_f16(w).reshape(n, k)
        X = np_f16(x)
        close_to(y, W @ X + r, S, k * 2.0**-52)
        close_to(S, np.abs(W) @ np.abs(X) + np.abs(r), S, k * 2.0**-52)


def pin_f16_exact_rational_subnormal(o):
    """Tiny shape with binary16 subnormal weights: exact rational sum."""
    g = rng(24)
    n, k = 3, 16
    w = g.integers(1, 0x400, (n, k)).astype(np.uint16) | (g.integers(0, 2, (n, k)).astype(np.uint16) << 15)
    x = synth.f16_activation(g, k)
    y, S = o.f16_gemv(w, x)
    W = np_f16(w).reshape(n, k)
    X = np_f16(x)
    for row in range(n):
        ex = sum(Fraction(float(W[row, i])) * Fraction(float(X[i])) for i in range(k))
        assert abs(Fraction(y[row]) - ex) <= Fraction(k * 2.0**-53) * Fraction(S[row])
    assert np.all(S > 0)


# ----------------------------------------------------------------------------- threading


def pin_threads_match_single(o):
    qw, dw, x, r = _q8_case(18, 101, 1024)
    qx, dx = o.quantize_act(x)
    y, S = o.q8_gemv(qw, dw, qx, dx, r)
    for t in (1, 3, 8, 200):
        yt, St = o.q8_gemv(qw, dw, qx, dx, r, nthreads=t)
        assert np.array_equal(yt, y) and np.array_equal(St, S)
    g = rng(19)
    w = synth.bf16_weights(g, 77, 512)
    xb = synth.bf16_activation(g, 512)
    y, S = o.bf16_gemv(w, xb)
    for t in (2, 7, 100):
        yt, St = o.bf16_gemv(w, xb, nthreads=t)
        assert np.array_equal(yt, y) and np.array_equal(St, S)
    wf = synth.f16_weights(g, 53, 256)
    xf = synth.f16_activation(g, 256)
    y, S = o.f16_gemv(wf, xf)
    for t in (3, 64):
        yt, St = o.f16_gemv(wf, xf, nthreads=t)
        assert np.array_equal(yt, y) and np.array_equal(St, S)


# ----------------------------------------------------------------------------- PTQ1_0

PB = 128  # weights per PTQ1_0 block


def np_hadamard_rotate(x):
    """H x / sqrt(128) per block with scipy's Sylvester matrix and exactly rounded sums."""
    import math

    from scipy.linalg import hadamard

    H = hadamard(PB)
    xb = np.asarray(x, dtype=np.float32).reshape(-1, PB).astype(np.float64)
    out = np.empty(xb.shape, np.float32)
    for b in range(xb.shape[0]):
        for i in range(PB):
            out[b, i] = np.float32(math.fsum(H[i] * xb[b]) / math.sqrt(PB))
    return out.ravel()


def _ptq1_case(j, n, k, resid=True):
    g = rng(j)
    w, t, sb = synth.ptq1_weights(g, n, k)
    x = synth.activation_f32(g, k)
    r = synth.residual_f32(g, n) if resid else None
    return w, t, sb, x, r


def pin_ptq1_decode_vs_encoder(o):
    w, t, sb, _, _ = _ptq1_case(40, 9, 512)
    tt, ss = o.ptq1_decode(w)
    assert np.array_equal(tt, t) and np.array_equal(ss, sb)
    # single bytes: base-3 digits, least significant first, digit = trit + 1
    blk = np.zeros((1, 28), np.uint8)
    for byte, want in ((0, [-1] * 5), (242, [1] * 5), (121, [0] * 5), (1, [0, -1, -1, -1, -1]),
                       (3, [-1, 0, -1, -1, -1]), (81 * 2, [-1, -1, -1, -1, 1])):
        blk[0, 7] = byte
        tt, _ = o.ptq1_decode(blk)
        assert list(tt[0, 35:40]) == want, (byte, list(tt[0, 35:40]))
    # the last byte holds weights 125..127; scale bits little-endian after the trits
    blk[0, 25], blk[0, 26], blk[0, 27] = 2 + 0 * 3 + 1 * 9, 0x34, 0x12
    tt, ss = o.ptq1_decode(blk)
    assert list(tt[0, 125:128]) == [1, -1, 0] and ss[0, 0] == 0x1234


def pin_hadamard_closed_forms(o):
    inv = np.float32(1.0 / np.sqrt(np.float64(PB)))
    for k in (0, 1, 37, 127):
        e = np.zeros(PB, np.float32)
        e[k] = 1.0
        h = o.hadamard128(e)
        signs = np.array([(-1) ** bin(i & k).count("1") for i in range(PB)], np.float32)
        assert np.array_equal(h, signs * inv), f"one-hot {k}"
    c = np.full(PB, 0.75, np.float32)
    h = o.hadamard128(c)
    assert h[0] == np.float32(128 * 0.75 / np.sqrt(128.0)) and np.all(h[1:] == 0)
    g = rng(41)
    x = g.standard_normal(4 * PB).astype(np.float32)
    y = o.hadamard128(x)
    # a rotation: norms kept; H / sqrt(128) is symmetric and orthogonal, so applying it twice
    # returns the input (up to the f32 roundings)
    for b in range(4):
        xb, yb = x[b * PB:(b + 1) * PB].astype(np.float64), y[b * PB:(b + 1) * PB].astype(np.float64)
        assert abs(np.linalg.norm(yb) - np.linalg.norm(xb)) <= 1e-6 * np.linalg.norm(xb)
    back = o.hadamard128(y)
    assert np.max(np.abs(back.astype(np.float64) - x)) <= 1e-5 * np.max(np.abs(x))
    # blocks are rotated independently
    z = x.copy()
    z[PB:] = 0
    assert np.array_equal(o.hadamard128(z)[:PB], y[:PB])


def pin_hadamard_vs_scipy(o):
    g = rng(42)
    x = np.concatenate([g.standard_normal(6 * PB), g.standard_normal(2 * PB) * 1e-3]).astype(np.float32)
    ours = o.hadamard128(x)
    ref = np_hadamard_rotate(x)
    assert np.array_equal(ours, ref), f"{np.count_nonzero(ours != ref)} mismatches"


def pin_ptq1_activation_quantizer(o):
    g = rng(43)
    x = np.concatenate([g.standard_normal(8 * PB), g.standard_normal(PB) * 1e-6, np.zeros(PB)]).astype(np.float32)
    rot, q, d = o.ptq1_activation(x)
    assert np.array_equal(rot, o.hadamard128(x))
    rq, rd = np_quantize(rot, PB)
    assert np.array_equal(q, rq) and np.array_equal(d, rd)
    assert np.all(q[-PB:] == 0) and d[-1] == 0


def pin_ptq1_rotation_spreads_outlier(o):
    """[P] §PrismML Ternary-Bonsai: the rotation evens out a large value across its block,
    which makes quantization less lossy. One 128-value block with a single large value: quantized
    directly, the small values fall below one code step; rotated, quantized, dequantized and
    rotated back, they survive."""
    g = rng(44)
    x = g.standard_normal(PB).astype(np.float32)
    x[17] = 100.0
    q, d = o.quantize_blocks(x, PB)
    direct = q.astype(np.float64) * np_f16(d)[0]
    rot, qr, dr = o.ptq1_activation(x)
    back = o.hadamard128((qr.astype(np.float64) * np_f16(dr)[0]).astype(np.float32)).astype(np.float64)
    keep = np.arange(PB) != 17
    err_direct = np.sqrt(np.mean((direct[keep] - x[keep]) ** 2))
    err_rot = np.sqrt(np.mean((back[keep] - x[keep]) ** 2))
    assert err_rot < err_direct / 4, (err_rot, err_direct)


def pin_ptq1_exact_rational(o):
    w, t, sb, x, r = _ptq1_case(45, 3, 256)
    _, qx, dx = o.ptq1_activation(x)
    y, S = o.ptq1_gemv(w, qx, dx, r)
    for row in range(3):
        ex = Fraction(0)
        for b in range(2):
            isum = sum(int(t[row, PB * b + i]) * int(qx[PB * b + i]) for i in range(PB))
            ex += isum * Fraction(float(np_f16(sb[row, b]))) * Fraction(float(np_f16(dx[b])))
        ex += Fraction(float(r[row]))
        assert abs(Fraction(y[row]) - ex) <= Fraction(4 * 2.0**-53) * Fraction(S[row])


def pin_ptq1_vs_dense_dequant(o):
    for j, (n, k) in enumerate(((40, 1024), (9, 3584), (5, 5120))):
        w, t, sb, x, r = _ptq1_case(46 + j, n, k)
        _, qx, dx = o.ptq1_activation(x)
        y, S = o.ptq1_gemv(w, qx, dx, r)
        W = t.astype(np.float64) * np.repeat(np_f16(sb), PB, axis=1)
        xd = qx.astype(np.float64) * np.repeat(np_f16(dx), PB)
        close_to(y, W @ xd + r.astype(np.float64), S, 1e-13)


def pin_ptq1_closed_forms(o):
    n, k = 4, 512
    g = rng(49)
    qx = g.integers(-127, 128, k).astype(np.int8)
    one = np.full(k // PB, 0x3C00, np.uint16)  # binary16 1.0
    r = synth.residual_f32(g, n)
    zero = synth.ptq1_pack(np.zeros((n, k), np.int8), np.tile(one, (n, 1)))
    y, S = o.ptq1_gemv(zero, qx, one, r)
    assert np.array_equal(y, r.astype(np.float64))  # zero trits give the residual
    ones = synth.ptq1_pack(np.ones((n, k), np.int8), np.tile(one, (n, 1)))
    y, _ = o.ptq1_gemv(ones, qx, one)
    assert np.all(y == float(qx.astype(np.int64).sum()))  # all +1 at unit scales: the sum of the codes
    w, t, sb, x, _ = _ptq1_case(50, n, k, resid=False)
    _, qx, dx = o.ptq1_activation(x)
    y, _ = o.ptq1_gemv(w, qx, dx)
    yn, _ = o.ptq1_gemv(synth.ptq1_pack(-t, sb), qx, dx)
    assert np.array_equal(yn, -y)  # negated trits negate the output exactly
    y2, _ = o.ptq1_gemv(w, qx, (np_f16(dx) * 2).astype(np.float16).view(np.uint16))
    assert np.array_equal(y2, 2 * y)  # doubling every activation scale doubles the output


def pin_ptq1_threads_match_single(o):
    w, _, _, x, r = _ptq1_case(51, 333, 1024)
    _, qx, dx = o.ptq1_activation(x)
    y1, s1 = o.ptq1_gemv(w, qx, dx, r)
    y4, s4 = o.ptq1_gemv(w, qx, dx, r, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4)


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
