"""Neighbour steps folded into the projection, HIP path vs the oracle (needs an MI355X).

RMS normalization before a stacked projection and the gated activation before the
down projection ("One level down: #002 the same compiler on a GPU", section
Emitting for a GPU; "Filling in the blanks: Inference using Phobos", section
Q4_K_M). Bars: the quantized codes and scale bits bit-exact against the oracle's
normalization or activation followed by its quantization (both sides form the
same f32 values, the one f64 sum of squares aside: its order is a rounding order,
and r = f32(1/sqrt(ss/K + eps)) agrees unless the f64 sums straddle an f32
rounding boundary); the fused launch bit-identical to the two-launch path; f32
outputs within 1e-5 * sum|w*x| of the oracle.
"""
import numpy as np
import pytest

import synth
from tests.test_gpu_parity import bits, dev, h16, host, print_case, within

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

EPS = 1e-6
KS = [32, 64, 1024, 2048, 3584, 5120, 16384]


@pytest.fixture(scope="module")
def q8():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_q8_amd as m

    m.load_library()
    return m


def norm_case(k, j):
    g = synth.rng_for(synth.TAG_NEIGHBOUR, j)
    return synth.activation_f32(g, k), synth.norm_gamma(g, k)


def silu_case(k, j):
    return synth.gate_up_f32(synth.rng_for(synth.TAG_NEIGHBOUR, 500 + j), k)


# --------------------------------------------------------------------------- quantize only


def check_norm_codes(q8, orc, x, gamma, eps, what):
    qx, dx = q8.q8_rmsnorm_quantize_act(dev(x), dev(gamma), eps)
    rq, rd = orc.quantize_act(orc.rmsnorm(x, gamma, eps))
    gq, gd = host(qx), bits(dx)
    assert np.array_equal(gq, rq), f"{what}: {np.count_nonzero(gq != rq)} codes differ"
    assert np.array_equal(gd, rd), f"{what}: {np.count_nonzero(gd != rd)} scales differ"


@pytest.mark.parametrize("k", KS)
def test_rmsnorm_quantize_bit_exact(q8, orc, k):
    print_case("rmsnorm quantize", k)
    x, gamma = norm_case(k, k)
    check_norm_codes(q8, orc, x, gamma, EPS, f"rmsnorm {k}")


def test_rmsnorm_quantize_special(q8, orc):
    """eps = 0 (pure scale invariance), eps dominating a tiny input, an all-zero input,
    a constant input, one outlier channel, huge and f32-subnormal magnitudes."""
    print_case("rmsnorm quantize special")
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 90)
    k = 1024
    gamma = synth.norm_gamma(g, k)
    x = synth.activation_f32(g, k)
    check_norm_codes(q8, orc, x, gamma, 0.0, "eps 0")
    check_norm_codes(q8, orc, (x * np.float32(1e-6)).astype(np.float32), gamma, 1e-2, "eps dominates")
    check_norm_codes(q8, orc, np.zeros(k, np.float32), gamma, 1e-5, "zero input")
    check_norm_codes(q8, orc, np.full(k, -2.5, np.float32), gamma, 0.0, "constant")
    xo = x.copy()
    xo[77] = 3000.0
    check_norm_codes(q8, orc, xo, gamma, EPS, "outlier channel")
    check_norm_codes(q8, orc, (x * np.float32(1e18)).astype(np.float32), gamma, 0.0, "huge")
    check_norm_codes(q8, orc, (x * np.float32(1e-38)).astype(np.float32), gamma, 0.0, "subnormal")


@pytest.mark.parametrize("k", KS + [32 * 3001])
def test_silu_mul_quantize_bit_exact(q8, orc, k):
    print_case("silu*up quantize", k)
    gu = silu_case(k, k)
    qx, dx = q8.q8_silu_mul_quantize_act(dev(gu))
    rq, rd = orc.quantize_act(orc.silu_mul(gu))
    assert np.array_equal(host(qx), rq), f"{np.count_nonzero(host(qx) != rq)} codes differ"
    assert np.array_equal(bits(dx), rd)


def test_silu_mul_quantize_special(q8, orc):
    """Gates far into both tails (exp overflows to inf in f64 at -gate > 709.8), zeros,
    the silu(0) = 0 point, tiny gates."""
    print_case("silu*up quantize special")
    k = 256
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 91)
    gate = np.concatenate([np.float32([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 88.0, -88.0, 700.0, -700.0,
                                       -710.0, -1000.0, 3e38, -3e38]),
                           g.standard_normal(k - 14).astype(np.float32) * np.float32(8.0)])
    up = g.standard_normal(k).astype(np.float32)
    up[:14] = 0.5
    up[20:40] = 0.0
    gu = np.concatenate([gate, up]).astype(np.float32)
    qx, dx = q8.q8_silu_mul_quantize_act(dev(gu))
    rq, rd = orc.quantize_act(orc.silu_mul(gu))
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(bits(dx), rd)


# --------------------------------------------------------------------------- fused into the GEMV


# (300, 7) x 2560 and x 3584: 8 waves per workgroup with two activation passes (2048 < K <= 4096)
NORM_SHAPES = [((1,), 32), ((2048, 1024, 1024), 1024), ((3584, 3584), 1024), ((300, 7), 2048),
               ((9,), 16384), ((8200,), 1024), ((40000,), 2080), ((200003,), 64), ((5, 6, 7, 8), 96),
               ((300, 7), 2560), ((300, 7), 3584)]


@pytest.mark.parametrize("sizes,k", NORM_SHAPES)
def test_rmsnorm_gemv_fused_equals_two_launches(q8, orc, sizes, k):
    """gemv_stacked_rmsnorm is bit-identical to q8_rmsnorm_quantize_act + q8_gemv on each part,
    and within 1e-5 * S of the oracle."""
    print_case("rmsnorm fused gemv", sizes, k)
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 1000 + sum(sizes) + k)
    x, gamma = synth.activation_f32(g, k), synth.norm_gamma(g, k)
    ws = [synth.q8_weights(g, n, k) for n in sizes]
    rs = [synth.residual_f32(g, n) if i % 2 else None for i, n in enumerate(sizes)]
    X, G = dev(x), dev(gamma)
    parts = [{"w": dev(qw), "dw": h16(dw), "residual": dev(r) if r is not None else None}
             for (qw, dw), r in zip(ws, rs)]
    fused = [host(y) for y in q8.gemv_stacked_rmsnorm(parts, X, G, EPS)]
    qx, dx = q8.q8_rmsnorm_quantize_act(X, G, EPS)
    rq, rd = orc.quantize_act(orc.rmsnorm(x, gamma, EPS))
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    for i, p in enumerate(parts):
        two = host(q8.q8_gemv(p["w"], p["dw"], qx, dx, residual=p["residual"]))
        assert np.array_equal(fused[i], two), f"part {i}: fused and two-launch results differ"
        yr, S = orc.q8_gemv(ws[i][0], ws[i][1], rq, rd, rs[i])
        within(fused[i], yr, S, f"rmsnorm part {i} {sizes[i]}x{k}")


# 40000 x 1056: 4 waves per workgroup with two activation passes
SILU_SHAPES = [(1, 32), (7, 96), (1024, 3584), (4096, 2048), (8200, 1024), (40000, 2080), (5, 16384), (40000, 1056)]


@pytest.mark.parametrize("n,k", SILU_SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_silu_gemv_fused_equals_two_launches(q8, orc, n, k, resid):
    print_case("silu fused gemv", n, k, resid)
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 2000 + n + k)
    qw, dw = synth.q8_weights(g, n, k)
    gu = synth.gate_up_f32(g, k)
    r = synth.residual_f32(g, n) if resid else None
    W, DW, GU = dev(qw), h16(dw), dev(gu)
    R = dev(r) if resid else None
    fused = host(q8.q8_gemv_silu_mul(W, DW, GU, residual=R))
    qx, dx = q8.q8_silu_mul_quantize_act(GU)
    two = host(q8.q8_gemv(W, DW, qx, dx, residual=R))
    assert np.array_equal(fused, two)
    rq, rd = orc.quantize_act(orc.silu_mul(gu))
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    yr, S = orc.q8_gemv(qw, dw, rq, rd, r)
    within(fused, yr, S, f"silu {n}x{k}")


def test_silu_gemv_residual_in_place(q8, orc):
    """The down projection adds the residual stream in place: y == residual."""
    print_case("silu fused gemv in place")
    n, k = 1024, 3584
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 3000)
    qw, dw = synth.q8_weights(g, n, k)
    gu = synth.gate_up_f32(g, k)
    r = synth.residual_f32(g, n)
    Y = dev(r)
    q8.q8_gemv_silu_mul(dev(qw), h16(dw), dev(gu), y=Y, residual=Y)
    yr, S = orc.q8_gemv(qw, dw, *orc.quantize_act(orc.silu_mul(gu)), r)
    within(host(Y), yr, S, "silu in place")


def test_outputs_not_written_past_end(q8):
    import torch

    print_case("neighbour guards")
    n, k = 1000, 1024
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 3001)
    qw, dw = synth.q8_weights(g, n, k)
    x, gamma = synth.activation_f32(g, k), synth.norm_gamma(g, k)
    gu = synth.gate_up_f32(g, k)
    buf = torch.full((n + 64,), 7.0, dtype=torch.float32, device="cuda")
    q8.gemv_stacked_rmsnorm([{"w": dev(qw), "dw": h16(dw), "y": buf[:n]}], dev(x), dev(gamma), EPS)
    assert (host(buf[n:]) == 7.0).all()
    buf2 = torch.full((n + 64,), 7.0, dtype=torch.float32, device="cuda")
    q8.q8_gemv_silu_mul(dev(qw), h16(dw), dev(gu), y=buf2[:n])
    assert (host(buf2[n:]) == 7.0).all()
    q = torch.full((k + 64,), 5, dtype=torch.int8, device="cuda")
    d = torch.full((k // 32 + 8,), 1.0, dtype=torch.float16, device="cuda")
    q8.q8_rmsnorm_quantize_act(dev(x), dev(gamma), EPS, qx=q[:k], dx=d[:k // 32])
    assert (host(q[k:]) == 5).all() and (host(d[k // 32:]) == 1.0).all()
    q8.q8_silu_mul_quantize_act(dev(gu), qx=q[:k], dx=d[:k // 32])
    assert (host(q[k:]) == 5).all() and (host(d[k // 32:]) == 1.0).all()


def test_rejections(q8):
    import torch

    k = 16384 + 32
    w = torch.zeros((2, k), dtype=torch.int8, device="cuda")
    dw = torch.zeros((2, k // 32), dtype=torch.float16, device="cuda")
    x = torch.zeros(k, dtype=torch.float32, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.gemv_stacked_rmsnorm([{"w": w, "dw": dw}], x, x.clone(), EPS)
    assert e.value.status == 2
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_rmsnorm_quantize_act(x, x.clone(), EPS)
    assert e.value.status == 2
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_gemv_silu_mul(w, dw, torch.zeros(2 * k, dtype=torch.float32, device="cuda"))
    assert e.value.status == 2
    xs = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_rmsnorm_quantize_act(xs, xs.clone(), -1.0)
    assert e.value.status == 4


# --------------------------------------------------------------------------- gate+up with the activation in its epilogue


EPI_SHAPES = [(32, 32), (64, 96), (3584, 1024), (9216, 2560), (4096 + 32, 1024 + 32), (96, 16384), (32, 40960)]


def gateup_case(f, k, j):
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 4000 + j)
    qw, dw = synth.q8_weights(g, 2 * f, k)  # one stacked [2F][K] matrix: gate rows, then up rows
    return g, qw, dw


def check_epilogue(q8, orc, qa, da, W, DW, qw, dw, rq, rd, f, what):
    """qa/da == the two-launch path (gemv_stacked over gate and up, then silu*up quantize), and
    == the oracle's silu*up + quantizer applied to those f32 gate/up results; gate/up within
    1e-5 * S of the oracle."""
    yg, yu = q8.gemv_stacked([{"w": W[:f], "dw": DW[:f]}, {"w": W[f:], "dw": DW[f:]}], dev(rq), h16(rd))
    gu = np.concatenate([host(yg), host(yu)])
    q2, d2 = q8.q8_silu_mul_quantize_act(dev(gu))
    gq, gd = host(qa), bits(da)
    assert np.array_equal(gq, host(q2)), f"{what}: {np.count_nonzero(gq != host(q2))} codes differ from two launches"
    assert np.array_equal(gd, bits(d2)), f"{what}: scales differ from two launches"
    oq, od = orc.quantize_act(orc.silu_mul(gu))
    assert np.array_equal(gq, oq) and np.array_equal(gd, od), f"{what}: differs from the oracle's silu*up + quantize"
    yr, S = orc.q8_gemv(qw, dw, rq, rd)
    within(gu, yr, S, f"{what} gate/up")


@pytest.mark.parametrize("f,k", EPI_SHAPES)
def test_gateup_epilogue_codes_input(q8, orc, f, k):
    print_case("gate+up silu epilogue, codes in", f, k)
    g, qw, dw = gateup_case(f, k, f + k)
    x = synth.activation_f32(g, k)
    W, DW = dev(qw), h16(dw)
    qx, dx = q8.q8_quantize_act(dev(x))
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq)
    qa, da = q8.q8_gateup_silu_quantize(W[:f], DW[:f], W[f:], DW[f:], qx, dx)
    check_epilogue(q8, orc, qa, da, W, DW, qw, dw, rq, rd, f, f"codes {f}x{k}")


@pytest.mark.parametrize("f,k", [s for s in EPI_SHAPES if s[1] <= 16384])
def test_gateup_epilogue_rmsnorm_input(q8, orc, f, k):
    """The whole MLP front in one launch: normalize, gate and up, silu*up, quantize."""
    print_case("gate+up silu epilogue, rmsnorm in", f, k)
    g, qw, dw = gateup_case(f, k, 7 * f + k)
    x, gamma = synth.activation_f32(g, k), synth.norm_gamma(g, k)
    W, DW = dev(qw), h16(dw)
    qa, da = q8.q8_gateup_silu_quantize(W[:f], DW[:f], W[f:], DW[f:], dev(x), gamma=dev(gamma), eps=EPS)
    qx, dx = q8.q8_rmsnorm_quantize_act(dev(x), dev(gamma), EPS)
    rq, rd = orc.quantize_act(orc.rmsnorm(x, gamma, EPS))
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    check_epilogue(q8, orc, qa, da, W, DW, qw, dw, rq, rd, f, f"rmsnorm {f}x{k}")


def test_gateup_epilogue_separate_matrices_and_mlp_chain(q8, orc):
    """Gate and up as two allocations; the chain epilogue -> down projection with the residual
    equals the prologue-fused chain and the four-launch chain bit for bit."""
    print_case("mlp chains")
    f, k = 3584, 1024
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 4999)
    qg, dg = synth.q8_weights(g, f, k)
    qu, du = synth.q8_weights(g, f, k)
    qd, dd = synth.q8_weights(g, k, f)
    x, gamma, r = synth.activation_f32(g, k), synth.norm_gamma(g, k), synth.residual_f32(g, k)
    Wg, Dg, Wu, Du, Wd, Dd = dev(qg), h16(dg), dev(qu), h16(du), dev(qd), h16(dd)
    X, G, Rr = dev(x), dev(gamma), dev(r)
    qa, da = q8.q8_gateup_silu_quantize(Wg, Dg, Wu, Du, X, gamma=G, eps=EPS)
    y_epi = host(q8.q8_gemv(Wd, Dd, qa, da, residual=Rr))
    yg, yu = q8.gemv_stacked_rmsnorm([{"w": Wg, "dw": Dg}, {"w": Wu, "dw": Du}], X, G, EPS)
    import torch

    gu = torch.cat([yg, yu])
    y_pro = host(q8.q8_gemv_silu_mul(Wd, Dd, gu, residual=Rr))
    qx, dx = q8.q8_rmsnorm_quantize_act(X, G, EPS)
    yg2, yu2 = q8.gemv_stacked([{"w": Wg, "dw": Dg}, {"w": Wu, "dw": Du}], qx, dx)
    qa2, da2 = q8.q8_silu_mul_quantize_act(torch.cat([yg2, yu2]))
    y_four = host(q8.q8_gemv(Wd, Dd, qa2, da2, residual=Rr))
    assert np.array_equal(y_epi, y_pro) and np.array_equal(y_epi, y_four)
    rq, rd = orc.quantize_act(orc.silu_mul(host(gu)))
    yr, S = orc.q8_gemv(qd, dd, rq, rd, r)
    within(y_epi, yr, S, "mlp chain")


@pytest.mark.parametrize("f,k,norm", [(f, k, n) for f, k in EPI_SHAPES for n in (False, True) if not (n and k > 16384)])
def test_gateup_f32_epilogue(q8, orc, f, k, norm):
    """a = silu(gate) * up written in f32 by the gate+up launch: bit for bit the oracle's silu*up of
    the same rows as gemv_stacked computes them, and quantized (q8_quantize_act) into exactly the
    codes and scales the quantizing epilogue writes (the normalizing prologue takes K <= 16384)."""
    print_case("gate+up f32 silu epilogue", f, k, "rmsnorm in" if norm else "codes in")
    g, qw, dw = gateup_case(f, k, 3 * f + k + (1 if norm else 0))
    x, gamma = synth.activation_f32(g, k), synth.norm_gamma(g, k)
    W, DW, X, G = dev(qw), h16(dw), dev(x), dev(gamma)
    if norm:
        a = q8.q8_gateup_silu(W[:f], DW[:f], W[f:], DW[f:], X, gamma=G, eps=EPS)
        qa, da = q8.q8_gateup_silu_quantize(W[:f], DW[:f], W[f:], DW[f:], X, gamma=G, eps=EPS)
        qx, dx = q8.q8_rmsnorm_quantize_act(X, G, EPS)
    else:
        qx, dx = q8.q8_quantize_act(X)
        a = q8.q8_gateup_silu(W[:f], DW[:f], W[f:], DW[f:], qx, dx)
        qa, da = q8.q8_gateup_silu_quantize(W[:f], DW[:f], W[f:], DW[f:], qx, dx)
    yg, yu = q8.gemv_stacked([{"w": W[:f], "dw": DW[:f]}, {"w": W[f:], "dw": DW[f:]}], qx, dx)
    gu = np.concatenate([host(yg), host(yu)])
    ah = host(a)
    assert np.array_equal(ah, orc.silu_mul(gu)), f"{np.count_nonzero(ah != orc.silu_mul(gu))} values differ"
    q2, d2 = q8.q8_quantize_act(a)
    assert np.array_equal(host(q2), host(qa)) and np.array_equal(bits(d2), bits(da))


def test_gateup_f32_epilogue_mlp_chain(q8, orc):
    """The MLP block as the f32 epilogue then the f32-input down projection (residual in place)
    equals the quantizing-epilogue chain bit for bit."""
    print_case("mlp chain, f32 epilogue")
    f, k = 3584, 1024
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 5111)
    qg, dg = synth.q8_weights(g, f, k)
    qu, du = synth.q8_weights(g, f, k)
    qd, dd = synth.q8_weights(g, k, f)
    x, gamma, r = synth.activation_f32(g, k), synth.norm_gamma(g, k), synth.residual_f32(g, k)
    Wg, Dg, Wu, Du, Wd, Dd = dev(qg), h16(dg), dev(qu), h16(du), dev(qd), h16(dd)
    X, G = dev(x), dev(gamma)
    qa, da = q8.q8_gateup_silu_quantize(Wg, Dg, Wu, Du, X, gamma=G, eps=EPS)
    y_epi = host(q8.q8_gemv(Wd, Dd, qa, da, residual=dev(r)))
    a = q8.q8_gateup_silu(Wg, Dg, Wu, Du, X, gamma=G, eps=EPS)
    h = dev(r)
    q8.gemv_stacked([{"w": Wd, "dw": Dd, "y": h, "residual": h}], a)
    assert np.array_equal(host(h), y_epi)
    rq, rd = orc.quantize_act(host(a))
    yr, S = orc.q8_gemv(qd, dd, rq, rd, r)
    within(y_epi, yr, S, "mlp chain, f32 epilogue")


def test_gateup_f32_epilogue_k0_and_guards(q8):
    import torch

    print_case("gate+up f32 epilogue K=0 and guards")
    f = 64
    w = torch.empty((f, 0), dtype=torch.int8, device="cuda")
    dw = torch.empty((f, 0), dtype=torch.float16, device="cuda")
    buf = torch.full((f + 64,), 7.0, dtype=torch.float32, device="cuda")
    q8.q8_gateup_silu(w, dw, w, dw, torch.empty(0, dtype=torch.int8, device="cuda"),
                      torch.empty(0, dtype=torch.float16, device="cuda"), a=buf[:f])
    assert (host(buf[:f]) == 0).all() and (host(buf[f:]) == 7.0).all()
    k = 1024
    g, qw, dwn = gateup_case(f, k, 78)
    W, DW = dev(qw), h16(dwn)
    x = dev(synth.activation_f32(g, k))
    buf = torch.full((f + 64,), float("nan"), dtype=torch.float32, device="cuda")
    buf[f:] = 7.0
    q8.q8_gateup_silu(W[:f], DW[:f], W[f:], DW[f:], x, gamma=dev(synth.norm_gamma(g, k)), eps=EPS, a=buf[:f])
    hb = host(buf)
    assert not np.isnan(hb[:f]).any() and (hb[f:] == 7.0).all()
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_gateup_silu(W[:48], DW[:48], W[f:f + 48], DW[f:f + 48], x, gamma=x.clone(), eps=EPS)
    assert e.value.status == 2


def test_gateup_epilogue_k0_and_guards(q8):
    import torch

    print_case("gate+up epilogue K=0 and guards")
    f = 64
    w = torch.empty((f, 0), dtype=torch.int8, device="cuda")
    dw = torch.empty((f, 0), dtype=torch.float16, device="cuda")
    qa = torch.full((f + 64,), 5, dtype=torch.int8, device="cuda")
    da = torch.full((f // 32 + 8,), 1.0, dtype=torch.float16, device="cuda")
    q8.q8_gateup_silu_quantize(w, dw, w, dw, torch.empty(0, dtype=torch.int8, device="cuda"),
                               torch.empty(0, dtype=torch.float16, device="cuda"), qa=qa[:f], da=da[:f // 32])
    assert (host(qa[:f]) == 0).all() and (bits(da[:f // 32]) == 0).all()
    assert (host(qa[f:]) == 5).all() and (host(da[f // 32:]) == 1.0).all()
    k = 1024
    g, qw, dwn = gateup_case(f, k, 77)
    W, DW = dev(qw), h16(dwn)
    x = dev(synth.activation_f32(g, k))
    qa = torch.full((f + 64,), 5, dtype=torch.int8, device="cuda")
    da = torch.full((f // 32 + 8,), 1.0, dtype=torch.float16, device="cuda")
    q8.q8_gateup_silu_quantize(W[:f], DW[:f], W[f:], DW[f:], x, gamma=dev(synth.norm_gamma(g, k)), eps=EPS,
                               qa=qa[:f], da=da[:f // 32])
    assert (host(qa[f:]) == 5).all() and (host(da[f // 32:]) == 1.0).all()
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_gateup_silu_quantize(W[:48], DW[:48], W[f:f + 48], DW[f:f + 48], x, gamma=x.clone(), eps=EPS)
    assert e.value.status == 2
