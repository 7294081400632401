"""HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

Bars: quantized codes, scale bits and every integer result bit-exact; f32 outputs
within 1e-5 * sum|w*x| per row (the magnitude the oracle reports as S); stacked
launches bit-identical to single-matrix launches; outputs never written past their end.
"""
import numpy as np
import pytest

import synth
from tests import oracle_pins

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL = 1e-5


@pytest.fixture(scope="module")
def q8():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_q8_amd as m

    m.load_library()
    return m


@pytest.fixture(scope="module")
def torch_mod():
    import torch

    return torch


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def h16(a):
    import torch

    return dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.float16)


def b16(a):
    import torch

    return dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits(t):
    import torch

    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def within(y_gpu, y_ref, S, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * S
    assert not bad.any(), (f"{what}: {bad.sum()} rows beyond 1e-5*S; worst row {np.argmax(err / np.maximum(S, 1e-300))}"
                           f" err {err.max():.3e}")


def print_case(*a):
    print("case:", *a, flush=True)


# --------------------------------------------------------------------------- quantize


QUANT_KS = [32, 64, 1024, 2048, 3584, 5120, 32 * 1001]


@pytest.mark.parametrize("k", QUANT_KS)
def test_quantize_bit_exact_normal(q8, orc, k):
    print_case("quantize N(0,1)", k)
    x = synth.activation_f32(synth.rng_for(synth.TAG_TEST, 200 + k), k)
    qx, dx = q8.q8_quantize_act(dev(x))
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(bits(dx), rd)


def test_quantize_bit_exact_special(q8, orc):
    """Wide ranges, binary16-subnormal scales, f32-subnormal inputs, zero blocks, ties, near-ties."""
    print_case("quantize special blocks")
    g = synth.rng_for(synth.TAG_TEST, 201)
    parts = [oracle_pins._quant_inputs()]
    # f32 subnormal magnitudes (the scale itself is an f32 subnormal)
    parts.append((g.standard_normal(256) * 1e-39).astype(np.float32))
    # huge magnitudes (scale overflows binary16: outside the contract for the dot, but the codes are defined)
    parts.append((g.standard_normal(64) * 1e30).astype(np.float32))
    # ties with d = 1 exactly
    t = np.zeros(32, np.float32)
    t[0] = 127.0
    t[1:13] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 125.5, 126.5, -126.5, 0.49999997, 63.5]
    parts.append(t)
    parts.append(np.zeros(64, np.float32))
    parts.append(np.full(32, -3.25, np.float32))
    x = np.concatenate(parts)
    x = np.concatenate([x, np.zeros((-len(x)) % 32, np.float32)])
    qx, dx = q8.q8_quantize_act(dev(x))
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq), f"{np.count_nonzero(host(qx) != rq)} codes differ"
    assert np.array_equal(bits(dx), rd), f"{np.count_nonzero(bits(dx) != rd)} scales differ"


def test_quantize_near_ties(q8, orc):
    """Values next to a rounding boundary of x/d, where x*(1/d) would round the other way."""
    print_case("quantize near ties")
    g = synth.rng_for(synth.TAG_TEST, 202)
    xs = []
    for _ in range(400):
        amax = np.float32(np.exp(g.uniform(-8, 8)))
        d = np.float32(amax / np.float32(127))
        inv = np.float32(np.float32(1) / d)
        ks = g.integers(-126, 126, 2000)
        cand = ((ks + 0.5) * np.float64(d)).astype(np.float32)
        cand = np.concatenate([cand, np.nextafter(cand, np.float32(np.inf)), np.nextafter(cand, np.float32(-np.inf))])
        sel = cand[(np.rint(cand / d) != np.rint(cand * inv)) & (np.abs(cand) < amax)]
        for v in sel[:4]:
            blk = np.zeros(32, np.float32)
            blk[0] = amax
            blk[1] = v
            xs.append(blk)
    assert len(xs) > 50
    x = np.concatenate(xs)
    qx, dx = q8.q8_quantize_act(dev(x))
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)


# --------------------------------------------------------------------------- Q8_0 GEMV


Q8_SHAPES = [(1, 32), (7, 64), (64, 1024), (300, 1536), (1024, 2048), (1025, 3584), (4096, 1024),
             (7168, 1024), (8193, 96), (33, 5120), (2, 4096 + 32)]


def q8_case(n, k, j):
    g = synth.rng_for(synth.TAG_TEST, 300 + j)
    qw, dw = synth.q8_weights(g, n, k)
    x = synth.activation_f32(g, k)
    r = synth.residual_f32(g, n)
    return qw, dw, x, r


@pytest.mark.parametrize("n,k", Q8_SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_q8_gemv_parity(q8, orc, n, k, resid):
    print_case("q8_gemv", n, k, resid)
    qw, dw, x, r = q8_case(n, k, n * 7 + k)
    qx, dx = q8.q8_quantize_act(dev(x))
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    y = q8.q8_gemv(dev(qw), h16(dw), qx, dx, residual=dev(r) if resid else None)
    yr, S = orc.q8_gemv(qw, dw, rq, rd, r if resid else None)
    within(host(y), yr, S, f"q8 {n}x{k}")


@pytest.mark.parametrize("n,k", [(7168, 1024), (1024, 3584), (333, 5120), (65, 96)])
def test_q8_integer_path_unit_scales(q8, orc, n, k):
    """Every scale 1.0: y[n] is the integer sum of the block sums (< 2^24), exact in f32
    under any summation order, so it must equal the oracle bit for bit."""
    print_case("q8 unit scales", n, k)
    g = synth.rng_for(synth.TAG_TEST, 400 + n)
    qw = g.integers(-128, 128, (n, k), dtype=np.int8)
    qx = g.integers(-127, 128, k, dtype=np.int8)
    ones_w = np.full((n, k // 32), 0x3C00, np.uint16)
    ones_x = np.full(k // 32, 0x3C00, np.uint16)
    y = q8.q8_gemv(dev(qw), h16(ones_w), dev(qx), h16(ones_x))
    yr, _ = orc.q8_gemv(qw, ones_w, qx, ones_x)
    isum = orc.block_isums(qw, qx)
    # every partial sum of block sums is an integer below 2^24, so exact in f32
    assert np.all(np.abs(isum).astype(np.int64).sum(axis=1) < 2**24)
    assert np.array_equal(host(y).astype(np.float64), yr)
    assert np.array_equal(yr, orc.block_isums(qw, qx).sum(axis=1).astype(np.float64))


def test_q8_per_block_sums_bit_exact(q8, orc):
    """Single-block isolation: only block b has a nonzero weight scale (1.0), so y[n] is
    exactly that block's int32 sum. Checked for every block of a 1024-wide matrix."""
    n, k = 515, 1024
    print_case("q8 per-block isolation", n, k)
    g = synth.rng_for(synth.TAG_TEST, 401)
    qw = g.integers(-128, 128, (n, k), dtype=np.int8)
    qx = g.integers(-127, 128, k, dtype=np.int8)
    isum = orc.block_isums(qw, qx)
    dqw, dqx = dev(qw), dev(qx)
    ones_x = h16(np.full(k // 32, 0x3C00, np.uint16))
    for b in range(k // 32):
        dw = np.zeros((n, k // 32), np.uint16)
        dw[:, b] = 0x3C00
        y = q8.q8_gemv(dqw, h16(dw), dqx, ones_x)
        assert np.array_equal(host(y), isum[:, b].astype(np.float32)), f"block {b}"


def test_q8_closed_form_all_ones(q8, orc):
    """All-ones blocks: each block gives 32*dw*dx."""
    n, k = 129, 2048
    print_case("q8 all ones", n, k)
    g = synth.rng_for(synth.TAG_TEST, 402)
    _, dw = synth.q8_weights(g, n, k)
    dx = synth.f32_to_f16_bits(np.abs(g.standard_normal(k // 32)).astype(np.float32))
    qw = np.ones((n, k), np.int8)
    qx = np.ones(k, np.int8)
    y = host(q8.q8_gemv(dev(qw), h16(dw), dev(qx), h16(dx))).astype(np.float64)
    ref = 32.0 * (oracle_pins.np_f16(dw).reshape(n, -1) * oracle_pins.np_f16(dx)[None, :]).sum(axis=1)
    _, S = orc.q8_gemv(qw, dw, qx, dx)
    within(y, ref, S, "all ones")


def test_q8_subnormal_scales(q8, orc):
    """Only binary16-subnormal scales on both sides: nothing may be flushed to zero."""
    n, k = 257, 1024
    print_case("q8 subnormal scales", n, k)
    g = synth.rng_for(synth.TAG_TEST, 403)
    qw = g.integers(-127, 128, (n, k), dtype=np.int8)
    qx = g.integers(-127, 128, k, dtype=np.int8)
    dw = g.integers(1, 0x400, (n, k // 32)).astype(np.uint16)
    dx = g.integers(1, 0x400, k // 32).astype(np.uint16)
    y = host(q8.q8_gemv(dev(qw), h16(dw), dev(qx), h16(dx)))
    yr, S = orc.q8_gemv(qw, dw, qx, dx)
    assert np.all(S > 0)
    within(y, yr, S, "subnormal scales")


def test_q8_invariants(q8, orc):
    n, k = 1000, 1024
    print_case("q8 invariants", n, k)
    qw, dw, x, _ = q8_case(n, k, 404)
    qx, dx = q8.q8_quantize_act(dev(x))
    W = dev(qw)
    y1 = host(q8.q8_gemv(W, h16(dw), qx, dx))
    y2 = host(q8.q8_gemv(W, h16(dw), qx, dx))
    assert np.array_equal(y1, y2), "run-to-run"
    yn = host(q8.q8_gemv(dev(-qw), h16(dw), qx, dx))
    assert np.array_equal(yn, -y1), "y(-W) = -y(W)"
    p = synth.rng_for(synth.TAG_TEST, 405).permutation(n)
    yp = host(q8.q8_gemv(dev(qw[p]), h16(dw[p]), qx, dx))
    assert np.array_equal(yp, y1[p]), "row permutation"


def test_q8_zero_weights_give_residual(q8):
    n, k = 77, 256
    print_case("q8 zero weights", n, k)
    _, dw, x, r = q8_case(n, k, 406)
    qx, dx = q8.q8_quantize_act(dev(x))
    y = host(q8.q8_gemv(dev(np.zeros((n, k), np.int8)), h16(dw), qx, dx, residual=dev(r)))
    assert np.array_equal(y, r)


# --------------------------------------------------------------------------- bf16 GEMV


BF16_SHAPES = [(1, 8), (5, 24), (64, 520), (300, 1024), (7168, 1024), (1025, 2560), (3, 4096 + 8)]


@pytest.mark.parametrize("n,k", BF16_SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_bf16_gemv_parity(q8, orc, n, k, resid):
    print_case("bf16_gemv", n, k, resid)
    g = synth.rng_for(synth.TAG_TEST, 500 + n + k)
    w = synth.bf16_weights(g, n, k)
    x = synth.bf16_activation(g, k)
    r = synth.residual_f32(g, n)
    y = q8.bf16_gemv(b16(w), b16(x), residual=dev(r) if resid else None)
    yr, S = orc.bf16_gemv(w, x, r if resid else None)
    within(host(y), yr, S, f"bf16 {n}x{k}")


@pytest.mark.parametrize("n,k", [(7168, 1024), (129, 2560), (9, 8)])
def test_bf16_integer_valued_bit_exact(q8, orc, n, k):
    print_case("bf16 integer-valued", n, k)
    g = synth.rng_for(synth.TAG_TEST, 501)
    wi = g.integers(-8, 9, (n, k))
    xi = g.integers(-8, 9, k)
    w = synth.f32_to_bf16_bits(wi.astype(np.float32))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    y = host(q8.bf16_gemv(b16(w), b16(x)))
    yr, _ = orc.bf16_gemv(w, x)
    assert np.array_equal(y.astype(np.float64), yr)


# --------------------------------------------------------------------------- f16 GEMV


@pytest.mark.parametrize("n,k", BF16_SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_f16_gemv_parity(q8, orc, n, k, resid):
    print_case("f16_gemv", n, k, resid)
    g = synth.rng_for(synth.TAG_TEST, 520 + n + k)
    w = synth.f16_weights(g, n, k)
    x = synth.f16_activation(g, k)
    r = synth.residual_f32(g, n)
    y = q8.f16_gemv(h16(w), h16(x), residual=dev(r) if resid else None)
    yr, S = orc.f16_gemv(w, x, r if resid else None)
    within(host(y), yr, S, f"f16 {n}x{k}")


@pytest.mark.parametrize("n,k", [(7168, 1024), (129, 2560), (9, 8)])
def test_f16_integer_valued_bit_exact(q8, orc, n, k):
    print_case("f16 integer-valued", n, k)
    g = synth.rng_for(synth.TAG_TEST, 521)
    wi = g.integers(-8, 9, (n, k))
    xi = g.integers(-8, 9, k)
    w = synth.f32_to_f16_bits(wi.astype(np.float32))
    x = synth.f32_to_f16_bits(xi.astype(np.float32))
    y = host(q8.f16_gemv(h16(w), h16(x)))
    yr, _ = orc.f16_gemv(w, x)
    assert np.array_equal(y.astype(np.float64), yr)


def test_f16_subnormal_weights(q8, orc):
    """Weights in the binary16 subnormal range must decode to their values, not to zero."""
    n, k = 77, 1024
    print_case("f16 subnormal weights", n, k)
    g = synth.rng_for(synth.TAG_TEST, 522)
    w = g.integers(1, 0x400, (n, k)).astype(np.uint16) | (g.integers(0, 2, (n, k)).astype(np.uint16) << 15)
    x = synth.f16_activation(g, k)
    y = host(q8.f16_gemv(h16(w), h16(x)))
    yr, S = orc.f16_gemv(w, x)
    assert np.all(S > 0)
    within(y, yr, S, "f16 subnormal")


def test_f16_stacked_halves(q8, orc):
    """The 1024 -> 7168 gate+up in binary16 as two 3584-row halves in one launch."""
    n, k = 7168, 1024
    print_case("f16 stacked halves", n, k)
    g = synth.rng_for(synth.TAG_TEST, 523)
    w = synth.f16_weights(g, n, k)
    x = synth.f16_activation(g, k)
    r = synth.residual_f32(g, n)
    Wt, Xt, Rt = h16(w), h16(x), dev(r)
    whole = host(q8.f16_gemv(Wt, Xt))
    outs = q8.gemv_stacked([{"w": Wt[:3584]}, {"w": Wt[3584:], "residual": Rt[3584:]}], Xt)
    lo, hi = host(outs[0]), host(outs[1])
    assert np.array_equal(lo, whole[:3584])
    assert np.array_equal(hi, host(q8.f16_gemv(Wt[3584:], Xt, residual=Rt[3584:])))
    yr, S = orc.f16_gemv(w, x)
    within(lo, yr[:3584], S[:3584], "f16 first half")
    within(hi, yr[3584:] + r[3584:], S[3584:] + np.abs(r[3584:].astype(np.float64)), "f16 second half")


# --------------------------------------------------------------------------- stacked


@pytest.mark.parametrize("sizes", [(3584, 3584), (2048, 1024, 1024), (1, 7, 100, 3), (0, 5, 0, 9)])
def test_q8_stacked_equals_single(q8, orc, sizes):
    k = 1024
    print_case("q8 stacked", sizes)
    n = sum(sizes)
    qw, dw, x, r = q8_case(n, k, 600 + len(sizes))
    qx, dx = q8.q8_quantize_act(dev(x))
    W, DW, Rr = dev(qw), h16(dw), dev(r)
    whole = host(q8.q8_gemv(W, DW, qx, dx, residual=Rr))
    parts, off = [], 0
    for i, s in enumerate(sizes):
        p = {"w": W[off:off + s], "dw": DW[off:off + s]}
        if i % 2:
            p["residual"] = Rr[off:off + s]
        parts.append(p)
        off += s
    outs = q8.gemv_stacked(parts, qx, dx)
    off = 0
    for i, (s, y) in enumerate(zip(sizes, outs)):
        yh = host(y)
        single = host(q8.q8_gemv(W[off:off + s], DW[off:off + s], qx, dx,
                                 residual=Rr[off:off + s] if i % 2 else None)) if s else yh
        assert np.array_equal(yh, single), f"part {i} differs from the single call"
        if i % 2:
            assert np.array_equal(yh, whole[off:off + s]), f"part {i} differs from the concatenated call"
        off += s
    yr, S = orc.q8_gemv(qw, dw, *orc.quantize_act(x))
    yall = np.concatenate([host(y) for y in outs]).astype(np.float64)
    Rmask = np.concatenate([np.full(s, i % 2 == 1) for i, s in enumerate(sizes)])
    yr = yr + np.where(Rmask, r.astype(np.float64), 0)
    S = S + np.where(Rmask, np.abs(r.astype(np.float64)), 0)
    within(yall, yr, S, "stacked vs oracle")


def test_bf16_stacked_halves(q8, orc):
    """The 1024 -> 7168 gate+up as two 3584-row halves in one launch."""
    n, k = 7168, 1024
    print_case("bf16 stacked halves", n, k)
    g = synth.rng_for(synth.TAG_TEST, 610)
    w = synth.bf16_weights(g, n, k)
    x = synth.bf16_activation(g, k)
    Wt, Xt = b16(w), b16(x)
    whole = host(q8.bf16_gemv(Wt, Xt))
    outs = q8.gemv_stacked([{"w": Wt[:3584]}, {"w": Wt[3584:]}], Xt)
    got = np.concatenate([host(o) for o in outs])
    assert np.array_equal(got, whole)
    yr, S = orc.bf16_gemv(w, x)
    within(got, yr, S, "bf16 halves")


# --------------------------------------------------------------------------- epilogue, guards, edges


def test_residual_in_place(q8):
    n, k = 1030, 2048
    print_case("in-place residual", n, k)
    qw, dw, x, r = q8_case(n, k, 700)
    qx, dx = q8.q8_quantize_act(dev(x))
    out_of_place = host(q8.q8_gemv(dev(qw), h16(dw), qx, dx, residual=dev(r)))
    yr = dev(r)
    q8.q8_gemv(dev(qw), h16(dw), qx, dx, y=yr, residual=yr)
    assert np.array_equal(host(yr), out_of_place)
    g = synth.rng_for(synth.TAG_TEST, 701)
    w = synth.bf16_weights(g, n, k)
    xb = synth.bf16_activation(g, k)
    oop = host(q8.bf16_gemv(b16(w), b16(xb), residual=dev(r)))
    yb = dev(r)
    q8.bf16_gemv(b16(w), b16(xb), y=yb, residual=yb)
    assert np.array_equal(host(yb), oop)


@pytest.mark.parametrize("n", [1, 7, 63, 64, 65, 3585, 7167, 8193])
def test_guards_untouched_and_poison_overwritten(q8, torch_mod, n):
    """Canaries around y stay intact; a NaN-poisoned y is fully overwritten."""
    torch = torch_mod
    k = 96
    print_case("guards", n)
    qw, dw, x, r = q8_case(n, k, 800 + n)
    qx, dx = q8.q8_quantize_act(dev(x))
    buf = torch.full((n + 128,), float("nan"), dtype=torch.float32, device="cuda")
    canary = torch.tensor([1234.5], device="cuda")
    buf[:64] = canary
    buf[64 + n:] = canary
    q8.q8_gemv(dev(qw), h16(dw), qx, dx, y=buf[64:64 + n], residual=dev(r))
    h = host(buf)
    assert np.all(h[:64] == 1234.5) and np.all(h[64 + n:] == 1234.5), "wrote outside y"
    assert not np.isnan(h[64:64 + n]).any(), "y not fully written"
    # the same for the quantizer's outputs
    qbuf = torch.full((k + 128,), 77, dtype=torch.int8, device="cuda")
    dbuf = torch.full((k // 32 + 16,), 7.0, dtype=torch.float16, device="cuda")
    q8.q8_quantize_act(dev(x), qx=qbuf[64:64 + k], dx=dbuf[8:8 + k // 32])
    hq, hd = host(qbuf), host(dbuf)
    assert np.all(hq[:64] == 77) and np.all(hq[64 + k:] == 77)
    assert np.all(hd[:8] == 7.0) and np.all(hd[8 + k // 32:] == 7.0)


def test_empty_and_k0(q8, torch_mod):
    torch = torch_mod
    print_case("empty and K=0")
    e8 = torch.empty((0, 64), dtype=torch.int8, device="cuda")
    y = q8.q8_gemv(e8, torch.empty((0, 2), dtype=torch.float16, device="cuda"),
                   torch.zeros(64, dtype=torch.int8, device="cuda"),
                   torch.zeros(2, dtype=torch.float16, device="cuda"))
    assert y.numel() == 0
    r = torch.arange(5, dtype=torch.float32, device="cuda")
    y = q8.q8_gemv(torch.empty((5, 0), dtype=torch.int8, device="cuda"),
                   torch.empty((5, 0), dtype=torch.float16, device="cuda"),
                   torch.empty(0, dtype=torch.int8, device="cuda"),
                   torch.empty(0, dtype=torch.float16, device="cuda"), residual=r)
    assert np.array_equal(host(y), host(r))
    y = q8.bf16_gemv(torch.empty((3, 0), dtype=torch.bfloat16, device="cuda"),
                     torch.empty(0, dtype=torch.bfloat16, device="cuda"))
    assert np.array_equal(host(y), np.zeros(3, np.float32))
    # fused f32 input with K == 0: every workgroup must still walk its row groups
    r2 = torch.arange(70000, dtype=torch.float32, device="cuda")
    y = q8.q8_gemv_f32(torch.empty((70000, 0), dtype=torch.int8, device="cuda"),
                       torch.empty((70000, 0), dtype=torch.float16, device="cuda"),
                       torch.empty(0, dtype=torch.float32, device="cuda"), residual=r2)
    assert np.array_equal(host(y), host(r2))


def test_misaligned_and_overlap_raise(q8, torch_mod):
    torch = torch_mod
    print_case("host-side rejects")
    buf = torch.zeros(4096 + 16, dtype=torch.int8, device="cuda")
    qw = buf[1:1 + 4096].view(1, 4096)  # 1-byte offset
    dw = torch.zeros((1, 128), dtype=torch.float16, device="cuda")
    qx = torch.zeros(4096, dtype=torch.int8, device="cuda")
    dx = torch.zeros(128, dtype=torch.float16, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_gemv(qw, dw, qx, dx)
    assert e.value.status == 3
    x = torch.zeros(1024, dtype=torch.float32, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_quantize_act(x, qx=x.view(torch.int8)[:1024], dx=dx[:32])
    assert e.value.status == 6


# --------------------------------------------------------------------------- fused quantize + GEMV


# 40000 x 1056: 4 waves per workgroup (n >= 32768) with two activation passes of 4 values per
# thread (1024 < K <= 2048)
@pytest.mark.parametrize("n,k", [(1, 32), (7, 96), (300, 1024), (1025, 3584), (4096, 1024), (64, 1024 + 96),
                                 (9, 16384), (8200, 1024), (200003, 64), (40000, 2080), (40000, 1056)])
def test_q8_fused_equals_quantize_then_gemv(q8, orc, n, k):
    """The f32-input launch (quantized inside) is bit-identical to q8_quantize_act + q8_gemv."""
    print_case("fused f32 gemv", n, k)
    qw, dw, x, r = q8_case(n, k, 900 + n + k)
    W, DW, X, Rr = dev(qw), h16(dw), dev(x), dev(r)
    qx, dx = q8.q8_quantize_act(X)
    two = host(q8.q8_gemv(W, DW, qx, dx, residual=Rr))
    one = host(q8.q8_gemv_f32(W, DW, X, residual=Rr))
    assert np.array_equal(one, two)
    yr, S = orc.q8_gemv(qw, dw, *orc.quantize_act(x), r)
    within(one, yr, S, f"fused {n}x{k}")


def test_q8_fused_stacked_parts(q8):
    print_case("fused stacked parts")
    n, k = 4096, 1024
    qw, dw, x, r = q8_case(n, k, 950)
    W, DW, X = dev(qw), h16(dw), dev(x)
    qx, dx = q8.q8_quantize_act(X)
    sizes = (2048, 1024, 1024)
    parts, off = [], 0
    for s in sizes:
        parts.append({"w": W[off:off + s], "dw": DW[off:off + s]})
        off += s
    a = [host(y) for y in q8.gemv_stacked(parts, qx, dx)]
    b = [host(y) for y in q8.gemv_stacked([{"w": p["w"], "dw": p["dw"]} for p in parts], X)]
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("sizes,with_res", [((3, 4093), (True, False)), ((2048, 1024, 1024), (False, True, False)),
                                            ((5, 1, 7), (False, True, True)), ((1000, 24), (True, True))])
def test_q8_fused_stacked_mixed_residuals(q8, orc, sizes, with_res):
    """Parts with and without a residual in one f32-input launch (the variant that requests
    the residual before the weights; a row without one reads an activation word instead,
    including a wave whose rows straddle the two kinds of part): bit-identical to the
    codes-input launch and to one call per part, within the tolerance of the oracle."""
    n, k = sum(sizes), 1024
    print_case("fused stacked mixed residuals", sizes, with_res)
    qw, dw, x, r = q8_case(n, k, 990 + len(sizes))
    W, DW, X, Rr = dev(qw), h16(dw), dev(x), dev(r)
    qx, dx = q8.q8_quantize_act(X)

    def parts():
        out, off = [], 0
        for s_, res in zip(sizes, with_res):
            p_ = {"w": W[off:off + s_], "dw": DW[off:off + s_]}
            if res:
                p_["residual"] = Rr[off:off + s_]
            out.append(p_)
            off += s_
        return out

    fused = [host(y) for y in q8.gemv_stacked(parts(), X)]
    codes = [host(y) for y in q8.gemv_stacked(parts(), qx, dx)]
    off = 0
    for i, (s_, res) in enumerate(zip(sizes, with_res)):
        assert np.array_equal(fused[i], codes[i]), f"part {i}: f32-input and codes-input launches differ"
        rp = Rr[off:off + s_] if res else None
        single = host(q8.q8_gemv_f32(W[off:off + s_], DW[off:off + s_], X, residual=rp))
        assert np.array_equal(fused[i], single), f"part {i} differs from its single call"
        off += s_
    yr, S = orc.q8_gemv(qw, dw, *orc.quantize_act(x))
    mask = np.concatenate([np.full(s_, res) for s_, res in zip(sizes, with_res)])
    yr = yr + np.where(mask, r.astype(np.float64), 0)
    S = S + np.where(mask, np.abs(r.astype(np.float64)), 0)
    within(np.concatenate(fused).astype(np.float64), yr, S, "fused stacked mixed residuals")


def test_q8_fused_rejects_long_k(q8, torch_mod):
    torch = torch_mod
    k = 16384 + 32
    w = torch.zeros((2, k), dtype=torch.int8, device="cuda")
    dw = torch.zeros((2, k // 32), dtype=torch.float16, device="cuda")
    x = torch.zeros(k, dtype=torch.float32, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.q8_gemv_f32(w, dw, x)
    assert e.value.status == 2
