"""GEMV rows of one to many weight batches, every launch shape, vs the CPU oracle (needs an MI355X).

A wave owns R rows (4, 2 or 1, chosen by the row count) and requests them four items
(row x 1 KiB chunk) at a time, CB = 4 / R chunks per batch. A row longer than one batch
runs a loop of two batches per trip and ends with one or two more batches. The chunk
counts below put each launch shape on every ending: the row fits one batch; one more
batch after it; whole trips then one batch; whole trips then two; two trips and one.
The last chunk and the last batch are partial (K not a multiple of the chunk).

Bars: f32 outputs within 1e-5 * sum|w*x| per row, on every row of small launches and on
sampled rows (the first and last 16, random ones) of wide ones; the f32-input launch
bit-identical to q8_quantize_act then q8_gemv; integer-valued bf16 bit-exact.
"""
import numpy as np
import pytest

import synth

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

TOL = 1e-5
KB = 1024  # bytes per row chunk

# rows for each rows-per-wave (a ragged last wave in each)
ROWS = {4: 8192 + 5, 2: 4096 + 3, 1: 301}
# chunk counts that reach every ending of the row loop for CB = 4 / R
CHUNKS = {4: [1, 2, 3, 4, 5], 2: [2, 3, 5, 7, 9], 1: [4, 6, 11, 15, 17]}


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


def print_case(*a):
    print("case:", *a, flush=True)


def sample_rows(n, seed):
    if n <= 512:
        return np.arange(n)
    pick = np.random.default_rng(seed).integers(0, n, 160)
    return np.unique(np.concatenate([np.arange(16), np.arange(n - 16, n), pick]))


def within(y, yr, S, what):
    err = np.abs(y.astype(np.float64) - yr)
    bad = err > TOL * S
    assert not bad.any(), f"{what}: {bad.sum()} rows beyond 1e-5*S; worst err {err.max():.3e}"


def q8_cases():
    for r, chunks in CHUNKS.items():
        for c in chunks:
            yield r, c


@pytest.mark.parametrize("r,nchunk", list(q8_cases()))
def test_q8_row_loop(q8, orc, r, nchunk):
    """Q8_0 codes input and the f32-input launch (quantized inside): K = (nchunk - 1) KiB + 96."""
    n, k = ROWS[r], (nchunk - 1) * KB + 96
    assert q8.gemv_config(q8.Q8G_Q8_0, n, k)[0] == r
    print_case("q8 row loop", n, k, r, nchunk)
    g = synth.rng_for(synth.TAG_TEST, 1200 + 16 * r + nchunk)
    qw, dw = synth.q8_weights(g, n, k)
    x = synth.activation_f32(g, k)
    res = synth.residual_f32(g, n)
    W, DW, X, RES = dev(qw), h16(dw), dev(x), dev(res)
    qx, dx = q8.q8_quantize_act(X)
    y = host(q8.q8_gemv(W, DW, qx, dx, residual=RES))
    rows = sample_rows(n, r * 100 + nchunk)
    rq, rd = orc.quantize_act(x)
    yr, S = orc.q8_gemv(qw[rows], dw[rows], rq, rd, res[rows])
    within(y[rows], yr, S, f"q8 {n}x{k} R={r}")
    if k <= q8.FUSED_MAX_K:
        assert q8.gemv_config(q8.Q8G_Q8_0_F32, n, k)[0] == r
        one = host(q8.q8_gemv_f32(W, DW, X, residual=RES))
        assert np.array_equal(one, y), "f32-input launch differs from quantize + codes GEMV"


def b16_cases():
    for r in (2, 1):
        for c in CHUNKS[r]:
            yield r, c


@pytest.mark.parametrize("kind", ["bf16", "f16"])
@pytest.mark.parametrize("r,nchunk", list(b16_cases()))
def test_16bit_row_loop(q8, orc, kind, r, nchunk):
    """bf16 and f16 rows (2 bytes per weight): K = 512 (nchunk - 1) + 40."""
    import torch

    n, k = ROWS[r], 512 * (nchunk - 1) + 40
    dtype = q8.Q8G_BF16 if kind == "bf16" else q8.Q8G_F16
    assert q8.gemv_config(dtype, n, k)[0] == r
    print_case(f"{kind} row loop", n, k, r, nchunk)
    g = synth.rng_for(synth.TAG_TEST, 1300 + 16 * r + nchunk + (0 if kind == "bf16" else 500))
    if kind == "bf16":
        w, x = synth.bf16_weights(g, n, k), synth.bf16_activation(g, k)
        tdt, fn, ref = torch.bfloat16, q8.bf16_gemv, orc.bf16_gemv
    else:
        w, x = synth.f16_weights(g, n, k), synth.f16_activation(g, k)
        tdt, fn, ref = torch.float16, q8.f16_gemv, orc.f16_gemv
    res = synth.residual_f32(g, n)
    y = host(fn(dev(w.view(np.int16)).view(tdt), dev(x.view(np.int16)).view(tdt), residual=dev(res)))
    rows = sample_rows(n, r * 100 + nchunk)
    yr, S = ref(w[rows], x, res[rows])
    within(y[rows], yr, S, f"{kind} {n}x{k} R={r}")


@pytest.mark.parametrize("r,nchunk", [(2, 9), (1, 17)])
def test_bf16_row_loop_integer_valued(q8, orc, r, nchunk):
    """Integer-valued bf16 weights and activation: every output is an integer below 2^24,
    exact under any summation order, so the long-row loop must match bit for bit."""
    n, k = ROWS[r], 512 * (nchunk - 1) + 40
    print_case("bf16 row loop integer-valued", n, k, r, nchunk)
    g = synth.rng_for(synth.TAG_TEST, 1400 + nchunk)
    w = synth.f32_to_bf16_bits(g.integers(-8, 9, (n, k)).astype(np.float32))
    x = synth.f32_to_bf16_bits(g.integers(-8, 9, k).astype(np.float32))
    import torch

    y = host(q8.bf16_gemv(dev(w.view(np.int16)).view(torch.bfloat16), dev(x.view(np.int16)).view(torch.bfloat16)))
    rows = sample_rows(n, nchunk)
    yr, _ = orc.bf16_gemv(w[rows], x)
    assert np.array_equal(y[rows].astype(np.float64), yr)
