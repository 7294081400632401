"""Parity at the benchmark's full sizes and launch configurations (needs an MI355X).

Each case runs the call bench.py times, on the first seeded matrix of the workload,
and compares rows with the oracle within 1e-5 * sum|w*x|: every row where the oracle
finishes in seconds, otherwise a seeded sample plus the first and last rows.
"""
import numpy as np
import pytest

import synth

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def q8():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_q8_amd as m

    m.load_library()
    return m


def host(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def dev16(a, dtype):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(dtype)


def test_bf16_4b_gateup_full(q8, orc):
    """18432x2560 bf16 as two 9216-row halves in one gemv_stacked launch: all rows."""
    import torch

    print("case: bf16 18432x2560 stacked halves, all rows", flush=True)
    n, k = 18432, 2560
    g = synth.rng_for(synth.TAG_BF16_4B_GATEUP, 0)
    w = synth.bf16_weights(g, n, k)
    x = synth.bf16_activation(g, k)
    W, X = dev16(w, torch.bfloat16), dev16(x, torch.bfloat16)
    outs = q8.gemv_stacked([{"w": W[: n // 2]}, {"w": W[n // 2:]}], X)
    y = np.concatenate([host(o) for o in outs]).astype(np.float64)
    yr, S = orc.bf16_gemv(w, x, nthreads=8)
    assert np.all(np.abs(y - yr) <= 1e-5 * S)


def test_q8_head_131072x5120_sampled(q8, orc):
    """The 680 MiB Q8_0 head: q8_quantize_act + q8_gemv, 4096 sampled rows + ends."""
    import torch

    print("case: q8 head 131072x5120, sampled rows", flush=True)
    n, k = 131072, 5120
    g = synth.rng_for(synth.TAG_Q8_HEAD, 0)
    qw, dw = synth.q8_weights(g, n, k)
    x = synth.activation_f32(g, k)
    qx, dx = q8.q8_quantize_act(torch.from_numpy(x).cuda())
    rq, rd = orc.quantize_act(x)
    assert np.array_equal(host(qx), rq)
    assert np.array_equal(host(dx.view(torch.int16)).view(np.uint16), rd)
    y = host(q8.q8_gemv(torch.from_numpy(qw).cuda(), dev16(dw, torch.float16), qx, dx)).astype(np.float64)
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], np.random.default_rng(41).integers(0, n, 4096)]))
    yr, S = orc.q8_gemv(qw[rows], dw[rows], rq, rd)
    assert np.all(np.abs(y[rows] - yr) <= 1e-5 * S)
    # the fused f32-input launch gives the same bits
    y2 = host(q8.q8_gemv_f32(torch.from_numpy(qw).cuda(), dev16(dw, torch.float16), torch.from_numpy(x).cuda()))
    assert np.array_equal(y2.astype(np.float64), y)


def test_q8_gateup_config_all_rows(q8, orc):
    """7168x1024 Q8_0 (the gate+up shape), the first seeded copy of its workload: all rows."""
    import torch

    print("case: q8 7168x1024, all rows", flush=True)
    n, k = 7168, 1024
    g = synth.rng_for(synth.TAG_Q8_GATEUP, 0)
    qw, dw = synth.q8_weights(g, n, k)
    x = synth.activation_f32(g, k)
    qx, dx = q8.q8_quantize_act(torch.from_numpy(x).cuda())
    y = host(q8.q8_gemv(torch.from_numpy(qw).cuda(), dev16(dw, torch.float16), qx, dx)).astype(np.float64)
    yr, S = orc.q8_gemv(qw, dw, *orc.quantize_act(x))
    assert np.all(np.abs(y - yr) <= 1e-5 * S)


def test_08b_stack_fused_graph_step(q8, orc):
    """The step bench.py reports: the full 0.8B stack as one fused launch per projection,
    replayed from a HIP graph; every output equals quantize + gemv_stacked bit for bit, and
    sampled rows of every projection are within tolerance of the oracle."""
    import torch

    from block_quantized_weight_q8_amd.stack import Q8DecodeStack

    print("case: 0.8B stack, fused graph step", flush=True)
    ops = synth.q8_stack_08b()
    hostin = synth.q8_stack_inputs(ops)
    st = Q8DecodeStack(ops, hostin)
    st.step()
    ref = [host(b["y"]).copy() for b in st.bufs]
    for b in st.bufs:
        b["y"].fill_(float("nan"))
    st.capture(fused=True)
    for rep in range(3):  # every replay checked, eager work and synchronizations between them
        for b in st.bufs:
            b["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        st.replay()
        got = [host(b["y"]) for b in st.bufs]
        for op, r, y in zip(ops, ref, got):
            assert np.array_equal(r, y), f"replay {rep}: {op.name}"
        st.step()
        torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for op, h, y in zip(ops, hostin, got):
        rq, rd = orc.quantize_act(h["x"])
        rows = np.unique(np.concatenate([[0, op.n - 1], rng.integers(0, op.n, 32)]))
        yr, S = orc.q8_gemv(h["qw"][rows], h["dw"][rows], rq, rd, h["r"][rows] if op.residual else None)
        assert np.all(np.abs(y[rows].astype(np.float64) - yr) <= 1e-5 * S), op.name
