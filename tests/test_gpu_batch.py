"""Small-batch Q8_0 GEMV (q8_gemv_batch, matrix cores) vs the CPU oracle (needs an MI355X).

Bars: f32 outputs within 1e-5 * sum|w*x| per (vector, row); integer-valued cases (all
scales 1.0) bit-exact; nothing written outside y; every shape class of the launch
(K split over four waves or whole-K tiles, several LDS tiles, an odd block count,
ragged row tails, B from 1 to 16).
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


def dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def h16(a):
    import torch

    return dev(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.float16)


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits16(t):
    import torch

    return host(t.view(torch.int16)).view(np.uint16)


def within(y_gpu, y_ref, S, what=""):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > TOL * S
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond 1e-5*S; worst err {err.max():.3e}"


def print_case(*a):
    print("case:", *a, flush=True)


def batch_case(n, k, nb, j, resid=True):
    g = synth.rng_for(synth.TAG_TEST, 900 + j)
    qw, dw = synth.q8_weights(g, n, k)
    x = np.stack([synth.activation_f32(g, k) for _ in range(nb)]) if nb else np.zeros((0, k), np.float32)
    r = np.stack([synth.residual_f32(g, n) for _ in range(nb)]) if resid and nb else None
    return qw, dw, x, r


def quantize_batch(q8, x):
    """One q8_quantize_act call over B*K values (blocks never straddle vectors)."""
    nb, k = x.shape
    qx, dx = q8.q8_quantize_act(dev(x.reshape(-1)))
    return qx.view(nb, k), dx.view(nb, k // 32)


SHAPES = [
    (16, 64, 1),       # one tile, one step
    (17, 96, 3),       # ragged rows, odd block count (last step has one block)
    (100, 1024, 16),   # K split over four waves
    (1024, 2048, 8),   # one full LDS tile
    (300, 3584, 5),    # two LDS tiles (2048 + 1536)
    (33, 5120, 16),    # three LDS tiles
    (4111, 160, 2),    # odd block count, ragged tail, many tiles
    (40000, 1024, 4),  # whole-K tiles (more than 2048 tiles)
    (7168, 1024, 16),  # the gate+up shape at full batch
    (64, 2080, 7),     # a last tile of one block (32 columns)
    (64, 4128, 16),    # three tiles, the last a single step
]


@pytest.mark.parametrize("n,k,nb", SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_batch_parity(q8, orc, n, k, nb, resid):
    print_case("q8_gemv_batch", n, k, nb, resid)
    qw, dw, x, r = batch_case(n, k, nb, n + k + nb, resid)
    qx, dx = quantize_batch(q8, x)
    y = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, residual=dev(r) if resid else None))
    qxh, dxh = host(qx), bits16(dx)
    # the batch was quantized by the library: check its codes against the oracle first
    for b in range(nb):
        oq, od = orc.quantize_act(x[b])
        assert np.array_equal(qxh[b], oq) and np.array_equal(dxh[b], od)
    yr, S = orc.q8_gemv_batch(qw, dw, qxh, dxh, r if resid else None, nthreads=8)
    within(y, yr, S, f"batch {n}x{k} B={nb}")


@pytest.mark.parametrize("n,k,nb", [(100, 1024, 16), (40000, 1024, 7), (33, 96, 16)])
def test_batch_unit_scales_bit_exact(q8, orc, n, k, nb):
    """All scales 1.0: every output is an integer below 2^24, exact under any summation order."""
    print_case("batch unit scales", n, k, nb)
    g = synth.rng_for(synth.TAG_TEST, 950)
    qw = g.integers(-128, 128, (n, k)).astype(np.int8)
    qx = g.integers(-127, 128, (nb, k)).astype(np.int8)
    dw = np.full((n, k // 32), 0x3C00, np.uint16)
    dx = np.full((nb, k // 32), 0x3C00, np.uint16)
    y = host(q8.q8_gemv_batch(dev(qw), h16(dw), dev(qx), h16(dx)))
    yr, _ = orc.q8_gemv_batch(qw, dw, qx, dx, nthreads=8)
    assert np.array_equal(y.astype(np.float64), yr)


def test_batch_vectors_independent(q8, orc):
    """Vector b's output depends on vector b only: permuting the batch permutes the rows
    of y bit for bit, and a batch of one equals the same vector inside a batch of 16
    within the tolerance (the K split may differ)."""
    n, k, nb = 2000, 1024, 16
    print_case("batch permutation", n, k, nb)
    qw, dw, x, _ = batch_case(n, k, nb, 960, resid=False)
    qx, dx = quantize_batch(q8, x)
    W, DW = dev(qw), h16(dw)
    y = host(q8.q8_gemv_batch(W, DW, qx, dx))
    perm = np.random.default_rng(3).permutation(nb)
    import torch

    pt = torch.from_numpy(perm).cuda()
    yp = host(q8.q8_gemv_batch(W, DW, qx[pt].contiguous(), dx[pt].contiguous()))
    assert np.array_equal(yp, y[perm])
    y1 = host(q8.q8_gemv_batch(W, DW, qx[5:6].contiguous(), dx[5:6].contiguous()))
    assert np.array_equal(y1[0], y[5])


def test_batch_residual_in_place(q8):
    n, k, nb = 1030, 2048, 6
    print_case("batch in-place residual", n, k, nb)
    qw, dw, x, r = batch_case(n, k, nb, 970)
    qx, dx = quantize_batch(q8, x)
    oop = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, residual=dev(r)))
    yr = dev(r)
    q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, y=yr, residual=yr)
    assert np.array_equal(host(yr), oop)


@pytest.mark.parametrize("n,nb", [(1, 1), (15, 16), (17, 3), (4097, 16), (40001, 5)])
def test_batch_guards(q8, n, nb):
    """Canaries around y stay intact; a NaN-poisoned y is fully overwritten."""
    import torch

    k = 96
    print_case("batch guards", n, nb)
    qw, dw, x, r = batch_case(n, k, nb, 980 + n)
    qx, dx = quantize_batch(q8, x)
    buf = torch.full((nb * n + 128,), float("nan"), dtype=torch.float32, device="cuda")
    buf[:64] = 1234.5
    buf[64 + nb * n:] = 1234.5
    q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, y=buf[64:64 + nb * n].view(nb, n), residual=dev(r))
    h = host(buf)
    assert np.all(h[:64] == 1234.5) and np.all(h[64 + nb * n:] == 1234.5), "wrote outside y"
    assert not np.isnan(h[64:64 + nb * n]).any(), "y not fully written"


def test_batch_edges(q8):
    import torch

    print_case("batch edges")
    d = "cuda"
    # K == 0: y = residual
    r = torch.arange(12, dtype=torch.float32, device=d).view(3, 4)
    y = q8.q8_gemv_batch(torch.empty((4, 0), dtype=torch.int8, device=d),
                         torch.empty((4, 0), dtype=torch.float16, device=d),
                         torch.empty((3, 0), dtype=torch.int8, device=d),
                         torch.empty((3, 0), dtype=torch.float16, device=d), residual=r)
    assert np.array_equal(host(y), host(r))
    # B == 0 and N == 0: nothing to do
    y = q8.q8_gemv_batch(torch.zeros((4, 64), dtype=torch.int8, device=d),
                         torch.zeros((4, 2), dtype=torch.float16, device=d),
                         torch.zeros((0, 64), dtype=torch.int8, device=d),
                         torch.zeros((0, 2), dtype=torch.float16, device=d))
    assert y.shape == (0, 4)
    y = q8.q8_gemv_batch(torch.zeros((0, 64), dtype=torch.int8, device=d),
                         torch.zeros((0, 2), dtype=torch.float16, device=d),
                         torch.zeros((2, 64), dtype=torch.int8, device=d),
                         torch.zeros((2, 2), dtype=torch.float16, device=d))
    assert y.shape == (2, 0)
    # more than 16 vectors is refused before anything runs
    with pytest.raises(q8.Q8GemvError):
        q8.q8_gemv_batch(torch.zeros((4, 64), dtype=torch.int8, device=d),
                         torch.zeros((4, 2), dtype=torch.float16, device=d),
                         torch.zeros((17, 64), dtype=torch.int8, device=d),
                         torch.zeros((17, 2), dtype=torch.float16, device=d))


def test_batch_full_size_head(q8, orc):
    """The 0.8B output head 151936 x 1024 at B = 16 (the launch bench.py times), and the
    131072 x 5120 head at B = 8: sampled rows of every vector against the oracle."""
    import torch

    for n, k, nb, tag in ((151936, 1024, 16, synth.TAG_Q8_HEAD), (131072, 5120, 8, synth.TAG_Q8_HEAD)):
        print_case("batch full-size head", n, k, nb)
        g = synth.rng_for(tag, 100 + nb)
        qw, dw = synth.q8_weights(g, n, k)
        x = np.stack([synth.activation_f32(g, k) for _ in range(nb)])
        qx, dx = quantize_batch(q8, x)
        y = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx))
        rows = np.unique(np.concatenate([[0, 15, 16, n - 1], np.random.default_rng(1).integers(0, n, 300)]))
        qxh, dxh = host(qx), bits16(dx)
        yr, S = orc.q8_gemv_batch(qw[rows], dw[rows], qxh, dxh)
        within(y[:, rows], yr, S, f"head {n}x{k} B={nb}")
        del qw, dw


# ----------------------------------------------------------------- tiled weight layout
# "Filling in the blanks", section GPU Performance Heisenbugs: the decode weights are stored
# eight columns side by side, which makes a warp's loads span full 128-byte lines
# (q8_pack_tile16, Q8G_LAYOUT_TILE16).
# Only the addresses differ from the row layout, so the outputs must match it bit for bit.


@pytest.mark.parametrize("n,k,nb", SHAPES)
def test_batch_tiled_equals_rows(q8, orc, n, k, nb):
    print_case("q8_gemv_batch tiled", n, k, nb)
    qw, dw, x, r = batch_case(n, k, nb, 2 * n + k + nb)
    qx, dx = quantize_batch(q8, x)
    y_rows = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, residual=dev(r)))
    t16 = q8.pack_tile16(qw, dw)
    y_tile = host(q8.q8_gemv_batch(t16, None, qx, dx, residual=dev(r)))
    assert np.array_equal(y_rows.view(np.uint32), y_tile.view(np.uint32)), "tiled layout differs from rows"
    yr, S = orc.q8_gemv_batch(qw, dw, host(qx), bits16(dx), r, nthreads=8)
    within(y_tile, yr, S, f"tiled {n}x{k} B={nb}")


@pytest.mark.parametrize("n,k,nb", [(100, 1024, 16), (40000, 1024, 7), (33, 96, 16)])
def test_batch_tiled_unit_scales_bit_exact(q8, orc, n, k, nb):
    print_case("tiled unit scales", n, k, nb)
    g = synth.rng_for(synth.TAG_TEST, 951)
    qw = g.integers(-128, 128, (n, k)).astype(np.int8)
    qx = g.integers(-127, 128, (nb, k)).astype(np.int8)
    dw = np.full((n, k // 32), 0x3C00, np.uint16)
    dx = np.full((nb, k // 32), 0x3C00, np.uint16)
    y = host(q8.q8_gemv_batch(q8.pack_tile16(qw, dw), None, dev(qx), h16(dx)))
    yr, _ = orc.q8_gemv_batch(qw, dw, qx, dx, nthreads=8)
    assert np.array_equal(y.astype(np.float64), yr)


@pytest.mark.parametrize("n,nb", [(1, 1), (17, 3), (4097, 16)])
def test_batch_tiled_guards(q8, n, nb):
    import torch

    k = 96
    print_case("tiled guards", n, nb)
    qw, dw, x, r = batch_case(n, k, nb, 990 + n)
    qx, dx = quantize_batch(q8, x)
    buf = torch.full((nb * n + 128,), float("nan"), dtype=torch.float32, device="cuda")
    buf[:64] = 1234.5
    buf[64 + nb * n:] = 1234.5
    q8.q8_gemv_batch(q8.pack_tile16(qw, dw), None, qx, dx, y=buf[64:64 + nb * n].view(nb, n), residual=dev(r))
    h = host(buf)
    assert np.all(h[:64] == 1234.5) and np.all(h[64 + nb * n:] == 1234.5), "wrote outside y"
    assert not np.isnan(h[64:64 + nb * n]).any(), "y not fully written"


# The persistent streaming form of the tiled layout: more than 2048 tiles, K of 8 or 16
# steps (K in (448, 512] or (960, 1024]) and 16-byte aligned scales. Each wave streams its
# tiles back to back; every step keeps the batched kernel's arithmetic, so the outputs equal
# the row layout's bit for bit.
STREAM_SHAPES = [
    (32785, 1024, 16),  # 2050 tiles, the last holding one row
    (33000, 992, 5),    # 16 steps, the last a single block
    (40000, 512, 1),    # 8 steps, one vector
    (36017, 480, 16),   # 8 steps, the last a single block; ragged rows
    (65536, 1024, 3),   # 4096 tiles: waves with unequal tile counts
]


@pytest.mark.parametrize("n,k,nb", STREAM_SHAPES)
@pytest.mark.parametrize("resid", [False, True])
def test_batch_tiled_stream(q8, orc, n, k, nb, resid):
    print_case("tiled stream", n, k, nb, resid)
    qw, dw, x, r = batch_case(n, k, nb, 7 * n + k + nb, resid)
    qx, dx = quantize_batch(q8, x)
    res = dev(r) if resid else None
    y_rows = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, residual=res))
    y_tile = host(q8.q8_gemv_batch(q8.pack_tile16(qw, dw), None, qx, dx, residual=res))
    assert np.array_equal(y_rows.view(np.uint32), y_tile.view(np.uint32)), "streamed tiles differ from rows"
    g = np.random.default_rng(n + k)
    last = (n - 1) // 16 * 16
    rows = np.unique(np.concatenate([[0, 15, 16, last, n - 1], np.arange(last, n), g.integers(0, n, 200)]))
    yr, S = orc.q8_gemv_batch(qw[rows], dw[rows], host(qx), bits16(dx), None if r is None else r[:, rows],
                              nthreads=8)
    within(y_tile[:, rows], yr, S, f"tiled stream {n}x{k} B={nb}")


@pytest.mark.parametrize("n,k,nb", [(33000, 1024, 7), (40001, 512, 16)])
def test_batch_tiled_stream_residual_in_place(q8, n, k, nb):
    """The streaming form reads each tile's residuals a tile ahead of its stores: y aliasing the
    residual gives the out-of-place bits."""
    print_case("tiled stream in-place residual", n, k, nb)
    qw, dw, x, r = batch_case(n, k, nb, 515 + n + nb)
    qx, dx = quantize_batch(q8, x)
    t16 = q8.pack_tile16(qw, dw)
    assert q8.batch_tiled_streams(n, k)
    oop = host(q8.q8_gemv_batch(t16, None, qx, dx, residual=dev(r)))
    yr = dev(r)
    q8.q8_gemv_batch(t16, None, qx, dx, y=yr, residual=yr)
    assert np.array_equal(host(yr).view(np.uint32), oop.view(np.uint32))


@pytest.mark.parametrize("n,k,nb,resid", [(32785, 1024, 4, False), (40001, 512, 16, True)])
def test_batch_tiled_stream_unaligned_scales(q8, n, k, nb, resid):
    """Tiled scales that are not 16-byte aligned take the whole-row shape instead: the same
    bits as the streaming form, and as the row layout."""
    import torch

    print_case("tiled stream vs whole-row shape (unaligned scales)", n, k, nb, resid)
    qw, dw, x, r = batch_case(n, k, nb, 4242 + n, resid=resid)
    qx, dx = quantize_batch(q8, x)
    res = dev(r) if resid else None
    t16 = q8.pack_tile16(qw, dw)
    y_a = host(q8.q8_gemv_batch(t16, None, qx, dx, residual=res))
    buf = torch.empty(t16.scales.numel() + 8, dtype=t16.scales.dtype, device="cuda")
    sc = buf[1:1 + t16.scales.numel()]
    sc.copy_(t16.scales)
    y_u = host(q8.q8_gemv_batch(q8.Tile16(t16.codes, sc, n, k), None, qx, dx, residual=res))
    assert np.array_equal(y_a.view(np.uint32), y_u.view(np.uint32))
    y_r = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx, residual=res))
    assert np.array_equal(y_a.view(np.uint32), y_r.view(np.uint32))


@pytest.mark.parametrize("n,k,nb", [(32785, 1024, 3), (40001, 512, 16)])
def test_batch_tiled_stream_guards(q8, n, k, nb):
    import torch

    print_case("tiled stream guards", n, k, nb)
    qw, dw, x, r = batch_case(n, k, nb, 77 + n)
    qx, dx = quantize_batch(q8, x)
    buf = torch.full((nb * n + 128,), float("nan"), dtype=torch.float32, device="cuda")
    buf[:64] = 1234.5
    buf[64 + nb * n:] = 1234.5
    q8.q8_gemv_batch(q8.pack_tile16(qw, dw), None, qx, dx, y=buf[64:64 + nb * n].view(nb, n), residual=dev(r))
    h = host(buf)
    assert np.all(h[:64] == 1234.5) and np.all(h[64 + nb * n:] == 1234.5), "wrote outside y"
    assert not np.isnan(h[64:64 + nb * n]).any(), "y not fully written"


def test_batch_tiled_full_size_head(q8, orc):
    """The 0.8B output head 151936 x 1024 at B = 16 in the tiled layout (the launch the
    bench's tiled head line times): identical to the row layout, sampled rows vs the oracle."""
    import torch

    n, k, nb = 151936, 1024, 16
    print_case("tiled full-size head", n, k, nb)
    g = synth.rng_for(synth.TAG_Q8_HEAD, 200 + nb)
    qw, dw = synth.q8_weights(g, n, k)
    x = np.stack([synth.activation_f32(g, k) for _ in range(nb)])
    qx, dx = quantize_batch(q8, x)
    y_rows = host(q8.q8_gemv_batch(dev(qw), h16(dw), qx, dx))
    y_tile = host(q8.q8_gemv_batch(q8.pack_tile16(qw, dw), None, qx, dx))
    assert np.array_equal(y_rows.view(np.uint32), y_tile.view(np.uint32))
    rows = np.unique(np.concatenate([np.arange(0, n, 1013), [n - 1]]))
    yr, S = orc.q8_gemv_batch(qw[rows], dw[rows], host(qx), bits16(dx), nthreads=8)
    within(y_tile[:, rows], yr, S, "tiled head")
    torch.cuda.synchronize()
