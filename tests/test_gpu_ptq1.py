"""PTQ1_0 HIP path vs the CPU oracle, through the C ABI (needs an MI355X).

"Filling in the blanks: Inference using Phobos", section PrismML Ternary-Bonsai:
ternary weights, 128 in 28 bytes, against a Hadamard-rotated activation; one rotation
per input serves all the projections that consume it.

Bars: rotated values, codes and scale bits bit-exact (the rotation is an f64 sum in
index order on both sides, rounded once to f32); unit-scale results bit-exact (every
term is an integer and every partial sum stays below 2^24); other outputs within
1e-5 * sum|w*x| per row; stacked launches bit-identical to single launches; rows past
the end never written.
"""
import numpy as np
import pytest

import synth

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


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def h16(a):
    import torch

    return dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.float16)


def bits(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def within(y_gpu, y_ref, S, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * S
    assert not bad.any(), f"{what}: {bad.sum()} rows beyond 1e-5*S, worst err {err.max():.3e}"


def print_case(*a):
    print("case:", *a, flush=True)


# --------------------------------------------------------------------------- rotation


ROT_KS = [128, 256, 1024, 2560, 5120, 128 * 137]


@pytest.mark.parametrize("k", ROT_KS)
def test_rotation_bit_exact(q8, orc, k):
    print_case("ptq1 rotate", k)
    x = synth.activation_f32(synth.rng_for(synth.TAG_TEST, 900 + k), k)
    import torch

    rot = torch.empty(k, dtype=torch.float32, device="cuda")
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x), rot=rot)
    rr, rq, rd = orc.ptq1_activation(x)
    assert np.array_equal(host(rot).view(np.uint32), rr.view(np.uint32)), "rotated values differ"
    assert np.array_equal(host(qx), rq), f"{np.count_nonzero(host(qx) != rq)} codes differ"
    assert np.array_equal(bits(dx), rd), "scales differ"


def test_rotation_special_blocks(q8, orc):
    """Zero block, one-hot, all equal, an outlier, wide exponent range, f32-subnormal inputs."""
    print_case("ptq1 rotate special")
    g = synth.rng_for(synth.TAG_TEST, 950)
    blocks = [np.zeros(128, np.float32)]
    e = np.zeros(128, np.float32)
    e[37] = 3.0
    blocks.append(e)
    blocks.append(np.full(128, -1.5, np.float32))
    o = g.standard_normal(128).astype(np.float32)
    o[5] = 1000.0
    blocks.append(o)
    blocks.append((g.standard_normal(128) * np.exp(g.uniform(-30, 30, 128))).astype(np.float32))
    blocks.append((g.standard_normal(128) * 1e-39).astype(np.float32))
    blocks.append((g.standard_normal(128) * 1e30).astype(np.float32))
    x = np.concatenate(blocks)
    import torch

    rot = torch.empty(x.size, dtype=torch.float32, device="cuda")
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x), rot=rot)
    rr, rq, rd = orc.ptq1_activation(x)
    assert np.array_equal(host(rot).view(np.uint32), rr.view(np.uint32))
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(bits(dx), rd)
    assert not host(qx)[:128].any() and bits(dx)[0] == 0


# --------------------------------------------------------------------------- GEMV

# (N, K): block-column splits C x W = 1x1 (K 128), 2x1, 4x1 (384: 3 of 4 columns), 8x1 (1024),
# 16x1, 4x5 (2560), 4x7 (3584), 32x1, 8x5 (5120), 32x3 (12288), 16x9 (17408), 32x16 (65536);
# ragged row counts and part tails
SHAPES = [(1, 128), (7, 256), (65, 384), (300, 1024), (1000, 2048), (777, 2560), (513, 3584), (4096, 4096),
          (300, 5120), (257, 12288), (100, 17408), (3, 65536)]


def ptq1_case(seed, n, k):
    g = synth.rng_for(synth.TAG_TEST, seed)
    w, _, _ = synth.ptq1_weights(g, n, k)
    x = synth.activation_f32(g, k)
    r = synth.residual_f32(g, n)
    return w, x, r


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("res", [False, True])
def test_gemv_vs_oracle(q8, orc, n, k, res):
    print_case("ptq1 gemv", n, k, res)
    w, x, r = ptq1_case(1000 + n + k, n, k)
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    _, rq, rd = orc.ptq1_activation(x)
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    y = q8.ptq1_gemv(dev(w), qx, dx, residual=dev(r) if res else None)
    yr, S = orc.ptq1_gemv(w, rq, rd, r if res else None)
    within(host(y), yr, S, f"{n}x{k}")


@pytest.mark.parametrize("n,k", [(300, 1024), (777, 2560), (257, 12288), (64, 65536)])
def test_gemv_unit_scales_bit_exact(q8, orc, n, k):
    """Scales 1.0 on both sides: each block term is the integer block sum and every partial
    sum is an integer below 2^24, so the f32 result is exact whatever the order."""
    print_case("ptq1 unit scales", n, k)
    g = synth.rng_for(synth.TAG_TEST, 1100 + k)
    t = g.integers(-1, 2, size=(n, k), dtype=np.int8)
    one = np.full((n, k // 128), 0x3C00, np.uint16)
    w = synth.ptq1_pack(t, one)
    qx = g.integers(-127, 128, k).astype(np.int8)
    dx = np.full(k // 128, 0x3C00, np.uint16)
    y = host(q8.ptq1_gemv(dev(w), dev(qx), h16(dx)))
    yr, S = orc.ptq1_gemv(w, qx, dx)
    assert np.all(S < 2 ** 24)
    assert np.array_equal(y.astype(np.float64), yr)
    # and the integer sum is the plain trit . code product
    assert np.array_equal(yr, t.astype(np.int64) @ qx.astype(np.int64))


def test_gemv_invalid_bytes(q8, orc):
    """Byte values 243..255 (never written by an encoder) and nonzero unused digits of byte 25
    decode digit by digit, as the oracle reads them."""
    print_case("ptq1 invalid bytes")
    g = synth.rng_for(synth.TAG_TEST, 1200)
    n, k = 70, 1024
    w = g.integers(0, 256, size=(n, k // 128 * 28), dtype=np.uint8)
    sb = synth.f32_to_f16_bits(np.abs(g.standard_normal((n, k // 128))).astype(np.float32) * np.float32(0.02))
    wb = w.reshape(n, k // 128, 28)
    wb[:, :, 26] = (sb & 0xFF).astype(np.uint8)
    wb[:, :, 27] = (sb >> 8).astype(np.uint8)
    w = wb.reshape(n, -1)
    x = synth.activation_f32(g, k)
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    _, rq, rd = orc.ptq1_activation(x)
    y = q8.ptq1_gemv(dev(w), qx, dx)
    yr, S = orc.ptq1_gemv(w, rq, rd)
    within(host(y), yr, S, "invalid bytes")


@pytest.mark.parametrize("k", [1024, 2560, 5120])
def test_stacked_equals_single(q8, orc, k):
    """gemv_stacked over gate and up (and over 4 ragged parts) gives the bits of one
    ptq1_gemv per part: one rotation of the input serves every part."""
    print_case("ptq1 stacked", k)
    g = synth.rng_for(synth.TAG_TEST, 1300 + k)
    sizes = [300, 300, 7, 129]
    ws = [synth.ptq1_weights(g, n, k)[0] for n in sizes]
    x = synth.activation_f32(g, k)
    rs = [synth.residual_f32(g, n) for n in sizes]
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    singles = [host(q8.ptq1_gemv(dev(w), qx, dx, residual=dev(r))) for w, r in zip(ws, rs)]
    outs = q8.gemv_stacked([{"w": dev(w), "residual": dev(r)} for w, r in zip(ws, rs)], qx, dx)
    for a, b in zip(outs, singles):
        assert np.array_equal(host(a).view(np.uint32), b.view(np.uint32))
    two = q8.gemv_stacked([{"w": dev(ws[0])}, {"w": dev(ws[1])}], qx, dx)
    cat = host(q8.ptq1_gemv(dev(np.concatenate([ws[0], ws[1]])), qx, dx))
    assert np.array_equal(np.concatenate([host(two[0]), host(two[1])]).view(np.uint32), cat.view(np.uint32))
    _, rq, rd = orc.ptq1_activation(x)
    for w, r, yv in zip(ws, rs, singles):
        yr, S = orc.ptq1_gemv(w, rq, rd, r)
        within(yv, yr, S, f"part of {k}")


def test_residual_aliases_output(q8, orc):
    import torch

    print_case("ptq1 y == residual")
    w, x, r = ptq1_case(1400, 513, 2560)
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    y = dev(r.copy())
    q8.ptq1_gemv(dev(w), qx, dx, y=y, residual=y)
    _, rq, rd = orc.ptq1_activation(x)
    yr, S = orc.ptq1_gemv(w, rq, rd, r)
    within(host(y), yr, S, "aliased residual")
    assert torch.isfinite(y).all()


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1000])
def test_guards_untouched(q8, n):
    """Rows past N are never written; every row of y is."""
    import torch

    print_case("ptq1 guards", n)
    k = 2560
    w, x, _ = ptq1_case(1500 + n, n, k)
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    buf = torch.full((n + 128,), float("nan"), device="cuda")
    canary = 1234.5
    buf[:64] = canary
    buf[64 + n:] = canary
    q8.ptq1_gemv(dev(w), qx, dx, y=buf[64:64 + n])
    hb = host(buf)
    assert np.all(hb[:64] == canary) and np.all(hb[64 + n:] == canary)
    assert np.isfinite(hb[64:64 + n]).all()


def test_edges(q8):
    import torch

    print_case("ptq1 edges")
    # N == 0: nothing enqueued
    w = torch.empty((0, 28 * 8), dtype=torch.uint8, device="cuda")
    qx = torch.zeros(1024, dtype=torch.int8, device="cuda")
    dx = torch.zeros(8, dtype=torch.float16, device="cuda")
    assert q8.ptq1_gemv(w, qx, dx).numel() == 0
    # K == 0: y = residual
    r = torch.arange(5, dtype=torch.float32, device="cuda")
    y = q8.ptq1_gemv(torch.empty((5, 0), dtype=torch.uint8, device="cuda"),
                     torch.empty(0, dtype=torch.int8, device="cuda"),
                     torch.empty(0, dtype=torch.float16, device="cuda"), residual=r)
    assert torch.equal(y, r)
    y = q8.ptq1_gemv(torch.empty((5, 0), dtype=torch.uint8, device="cuda"),
                     torch.empty(0, dtype=torch.int8, device="cuda"),
                     torch.empty(0, dtype=torch.float16, device="cuda"))
    assert torch.equal(y, torch.zeros(5, device="cuda"))
    # all-zero activation: codes 0, scales 0, y = residual exactly
    n, k = 100, 1024
    wz = dev(synth.ptq1_weights(synth.rng_for(synth.TAG_TEST, 1600), n, k)[0])
    qz, dz = q8.ptq1_rotate_quantize_act(torch.zeros(k, dtype=torch.float32, device="cuda"))
    rr = torch.randn(n, device="cuda")
    assert torch.equal(q8.ptq1_gemv(wz, qz, dz, residual=rr), rr)


def test_full_size_sampled(q8, orc):
    """The bench's stacked gate+up at its full size (2 x 17408 rows, K = 5120), in the launch
    the bench times: sampled rows of every part against the oracle, every row finite."""
    import torch

    n, k = 17408, 5120
    print_case("ptq1 full size", n, k)
    g = synth.rng_for(synth.TAG_PTQ1, 0)
    wg, _, _ = synth.ptq1_weights(g, n, k)
    wu, _, _ = synth.ptq1_weights(g, n, k)
    x = synth.activation_f32(g, k)
    qx, dx = q8.ptq1_rotate_quantize_act(dev(x))
    _, rq, rd = orc.ptq1_activation(x)
    assert np.array_equal(host(qx), rq) and np.array_equal(bits(dx), rd)
    outs = q8.gemv_stacked([{"w": dev(wg)}, {"w": dev(wu)}], qx, dx)
    rows = np.unique(np.concatenate([np.arange(0, n, 97), [n - 1]]))
    for w, y in zip((wg, wu), outs):
        yh = host(y)
        assert np.isfinite(yh).all()
        yr, S = orc.ptq1_gemv(w[rows], rq, rd)
        within(yh[rows], yr, S, "full size")
    del outs
    torch.cuda.synchronize()
