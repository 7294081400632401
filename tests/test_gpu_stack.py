"""The decode step as one launch (q8_decode_stack) vs launch-per-projection, vs the oracle.

q8_decode_stack must give bit-identical outputs to q8_quantize_act + gemv_stacked on
the same inputs (same per-row instructions and order), and so be within 1e-5*S of
the oracle. Needs an MI355X.
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


def bits16(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def run_both(q8, ops, tag, launches=1):
    from block_quantized_weight_q8_amd.stack import Q8DecodeStack

    hostin = synth.q8_stack_inputs(ops, tag)
    st = Q8DecodeStack(ops, hostin)
    st.step()
    ref = [(host(b["y"]).copy(), host(b["qx"]).copy(), bits16(b["dx"]).copy()) for b in st.bufs]
    for b in st.bufs:
        b["y"].fill_(float("nan"))
        b["qx"].fill_(0)
        b["dx"].fill_(0)
    st.make_plan()
    for _ in range(launches):
        st.step_persistent()
    assert st.plan.error_flag() == 0
    got = [(host(b["y"]), host(b["qx"]), bits16(b["dx"])) for b in st.bufs]
    return hostin, st, ref, got


def check_oracle(orc, ops, hostin, got, rows_per_op=None):
    for op, h, (y, qx, dx) in zip(ops, hostin, got):
        rq, rd = orc.quantize_act(h["x"])
        assert np.array_equal(qx, rq) and np.array_equal(dx, rd), op.name
        rows = np.arange(op.n) if rows_per_op is None or op.n <= rows_per_op else np.unique(
            np.concatenate([[0, op.n - 1], np.random.default_rng(op.n).integers(0, op.n, rows_per_op)]))
        yr, S = orc.q8_gemv(h["qw"][rows], h["dw"][rows], rq, rd, h["r"][rows] if op.residual else None)
        err = np.abs(y[rows].astype(np.float64) - yr)
        assert np.all(err <= 1e-5 * S), f"{op.name}: {err.max()}"


def test_small_stack_bit_identical(q8, orc):
    print("case: 2-layer stack + 5000-row head", flush=True)
    ops = synth.q8_stack_08b(layers=2, vocab=5000)
    hostin, _, ref, got = run_both(q8, ops, synth.TAG_TEST + 1)
    for op, (y0, q0, d0), (y1, q1, d1) in zip(ops, ref, got):
        assert np.array_equal(q0, q1) and np.array_equal(d0, d1), f"{op.name}: codes differ"
        assert np.array_equal(y0, y1), f"{op.name}: outputs differ from gemv_stacked"
    check_oracle(orc, ops, hostin, got)


def test_odd_shapes_and_repeated_launches(q8, orc):
    """Ragged K (tail chunks), tiny and empty parts, four parts, more rows than waves,
    fewer rows than workgroups; five launches in a row reuse the workspace."""
    print("case: odd-shaped stack, 5 launches", flush=True)
    ops = [
        synth.Gemv("a", (1,), 96),
        synth.Gemv("b", (7, 0, 100, 3), 1024 + 96, residual=True),
        synth.Gemv("c", (300,), 3584),
        synth.Gemv("d", (70000,), 64),
        synth.Gemv("e", (2,), 5120),
        synth.Gemv("f", (1000, 1000), 2048, residual=True),
    ]
    hostin, _, ref, got = run_both(q8, ops, synth.TAG_TEST + 2, launches=5)
    for op, (y0, q0, d0), (y1, q1, d1) in zip(ops, ref, got):
        assert np.array_equal(q0, q1) and np.array_equal(d0, d1), f"{op.name}: codes differ"
        assert np.array_equal(y0, y1), f"{op.name}: outputs differ"
    check_oracle(orc, ops, hostin, got)


def test_single_projection(q8, orc):
    """One op: no barrier inside the launch, so the workspace's barrier count and
    counters stay zero over three launches."""
    print("case: single projection", flush=True)
    ops = [synth.Gemv("only", (4096,), 1024)]
    hostin, st, ref, got = run_both(q8, ops, synth.TAG_TEST + 3, launches=3)
    assert np.array_equal(ref[0][0], got[0][0])
    check_oracle(orc, ops, hostin, got)
    ws = host(st.plan.sync)
    assert ws[0] == 0 and np.all(ws[64:64 + 16 * 64:64] == 0)


def test_workspace_counts_barriers(q8):
    """Three launches of a 5-op stack: the barrier count is 3 * 4, and each of the 16
    counters holds 12 times the number of workgroups that add to it."""
    import torch

    print("case: barrier count over three launches", flush=True)
    ops = synth.q8_stack_08b(layers=1, vocab=2000)
    hostin, st, ref, got = run_both(q8, ops, synth.TAG_TEST + 7, launches=3)
    for (y0, _, _), (y1, _, _) in zip(ref, got):
        assert np.array_equal(y0, y1)
    ws = host(st.plan.sync).view(np.uint32)
    G = torch.cuda.get_device_properties(0).multi_processor_count
    nb = 3 * (len(ops) - 1)
    assert ws[0] == nb
    per = np.array([(G - c + 15) // 16 for c in range(16)], dtype=np.int64)
    assert np.array_equal(ws[64:64 + 16 * 64:64].astype(np.int64), nb * per)


def test_full_08b_stack(q8, orc):
    """The 0.8B-shaped stack: all 97 outputs bit-identical to launch-per-projection,
    sampled rows within tolerance of the oracle."""
    print("case: full 0.8B-shaped stack", flush=True)
    ops = synth.q8_stack_08b()
    hostin, _, ref, got = run_both(q8, ops, synth.TAG_Q8_STACK, launches=2)
    for op, (y0, q0, d0), (y1, q1, d1) in zip(ops, ref, got):
        assert np.array_equal(q0, q1) and np.array_equal(d0, d1), f"{op.name}: codes differ"
        assert np.array_equal(y0, y1), f"{op.name}: outputs differ"
    check_oracle(orc, ops, hostin, got, rows_per_op=64)


def test_stack_rejects_bad_descriptors(q8):
    import torch

    print("case: stack validation", flush=True)
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    w = torch.zeros((4, 64), dtype=torch.int8, device="cuda")
    dw = torch.zeros((4, 2), dtype=torch.float16, device="cuda")
    y = torch.zeros(4, dtype=torch.float32, device="cuda")
    ok = {"x": x, "parts": [{"w": w, "dw": dw, "y": y}]}
    q8.DecodeStackPlan([ok]).run()
    # an output over an input of the same op
    with pytest.raises(q8.Q8GemvError) as e:
        q8.DecodeStackPlan([{"x": x, "parts": [{"w": w, "dw": dw, "y": x[:4]}]}]).run()
    assert e.value.status == 6
    # an output over a later op's weights (those are fetched before the barrier)
    wbuf = torch.zeros(4 * 64, dtype=torch.int8, device="cuda")
    w1 = wbuf.view(4, 64)
    y0 = wbuf[:16].view(torch.float32)
    with pytest.raises(q8.Q8GemvError) as e:
        q8.DecodeStackPlan([{"x": x, "parts": [{"w": w, "dw": dw, "y": y0}]},
                            {"x": x, "parts": [{"w": w1, "dw": dw, "y": y}]}]).run()
    assert e.value.status == 6
    # two outputs on one buffer
    with pytest.raises(q8.Q8GemvError) as e:
        q8.DecodeStackPlan([ok, {"x": x, "parts": [{"w": w, "dw": dw, "y": y}]}]).run()
    assert e.value.status == 6
    # K outside [32, 16384]
    big = torch.zeros(16384 + 32, dtype=torch.float32, device="cuda")
    wb = torch.zeros((1, 16384 + 32), dtype=torch.int8, device="cuda")
    dwb = torch.zeros((1, (16384 + 32) // 32), dtype=torch.float16, device="cuda")
    with pytest.raises(q8.Q8GemvError) as e:
        q8.DecodeStackPlan([{"x": big, "parts": [{"w": wb, "dw": dwb, "y": y[:1]}]}]).run()
    assert e.value.status == 2


def test_chained_projection_sees_previous_output(q8):
    """Op 1 reads op 0's output as its activation (a real decode chain): the barrier
    must make op 0's outputs visible to every workgroup before op 1 quantizes them."""
    import torch

    print("case: chained projections", flush=True)
    g = synth.rng_for(synth.TAG_TEST, 4)
    k0, n0, n1 = 1024, 2048, 3000
    qw0, dw0 = synth.q8_weights(g, n0, k0)
    qw1, dw1 = synth.q8_weights(g, n1, n0)
    x0 = synth.activation_f32(g, k0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    W0, D0, W1, D1, X0 = dev(qw0), h16(dw0), dev(qw1), h16(dw1), dev(x0)
    y0 = torch.full((n0,), float("nan"), device="cuda")
    y1 = torch.full((n1,), float("nan"), device="cuda")
    plan = q8.DecodeStackPlan([{"x": X0, "parts": [{"w": W0, "dw": D0, "y": y0}]},
                               {"x": y0, "parts": [{"w": W1, "dw": D1, "y": y1}]}])
    for _ in range(3):
        plan.run()
    assert plan.error_flag() == 0
    qa, da = q8.q8_quantize_act(X0)
    r0 = q8.q8_gemv(W0, D0, qa, da)
    qb, db = q8.q8_quantize_act(r0)
    r1 = q8.q8_gemv(W1, D1, qb, db)
    assert np.array_equal(host(y0), host(r0))
    assert np.array_equal(host(y1), host(r1))


def test_fused_step_matches(q8):
    """The one-launch-per-projection step (quantize inside the GEMV) gives the same bits."""
    from block_quantized_weight_q8_amd.stack import Q8DecodeStack

    print("case: fused per-projection step", flush=True)
    ops = synth.q8_stack_08b(layers=3, vocab=20000)
    st = Q8DecodeStack(ops, synth.q8_stack_inputs(ops, synth.TAG_TEST + 5))
    st.step()
    ref = [host(b["y"]).copy() for b in st.bufs]
    for b in st.bufs:
        b["y"].fill_(float("nan"))
    st.step(fused=True)
    for op, r, b in zip(ops, ref, st.bufs):
        assert np.array_equal(r, host(b["y"])), op.name


def test_batch_stack_graph_replay(q8, orc):
    """The 16-stream step as bench.py runs it: captured into a HIP graph and replayed three
    times, every replay checked bit for bit against the eager step, with eager work and
    synchronizations between replays; sampled rows against the oracle."""
    import torch

    from block_quantized_weight_q8_amd.stack import Q8BatchStack, Q8DecodeStack

    print("case: 2-layer stack + 5000-row head, 16 streams, graph replay", flush=True)
    nb = 16
    ops = synth.q8_stack_08b(layers=2, vocab=5000)
    hostin = synth.q8_stack_inputs(ops, synth.TAG_TEST + 5)
    batch = synth.q8_batch_inputs(ops, nb, synth.TAG_TEST + 6)
    bs = Q8BatchStack(Q8DecodeStack(ops, hostin), batch)
    bs.step()
    ref = [host(b["y"]).copy() for b in bs.bufs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bs.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bs.step()
    for rep in range(3):
        for b in bs.bufs:
            b["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for op, r, b in zip(ops, ref, bs.bufs):
            assert np.array_equal(host(b["y"]), r), f"replay {rep}: {op.name}"
        bs.step()
        torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for op, h, hb, r in zip(ops, hostin, batch, ref):
        rows = np.unique(np.concatenate([[0, op.n - 1], rng.integers(0, op.n, 24)]))
        for v in (0, nb - 1):
            rq, rd = orc.quantize_act(hb["x"][v])
            yr, S = orc.q8_gemv(h["qw"][rows], h["dw"][rows], rq, rd, hb["r"][v][rows] if op.residual else None)
            err = np.abs(r[v][rows].astype(np.float64) - yr)
            assert np.all(err <= 1e-5 * S), f"{op.name} stream {v}: {err.max()}"


def test_batch_stack_tiled_equals_rows(q8):
    """The 16-stream step on weights packed into the tiled layout (the default) equals the step
    on the row layout bit for bit, the 40000-row head taking the streaming form."""
    from block_quantized_weight_q8_amd.stack import Q8BatchStack, Q8DecodeStack

    print("case: 1-layer stack + 40000-row head, 16 streams, tiled vs row layout", flush=True)
    ops = synth.q8_stack_08b(layers=1, vocab=40000)
    hostin = synth.q8_stack_inputs(ops, synth.TAG_TEST + 7)
    batch = synth.q8_batch_inputs(ops, 16, synth.TAG_TEST + 8)
    stack = Q8DecodeStack(ops, hostin)
    rows = Q8BatchStack(stack, batch, tiled=False)
    rows.step()
    ref = [host(b["y"]).copy() for b in rows.bufs]
    tiled = Q8BatchStack(stack, batch)
    assert tiled.tiled
    tiled.step()
    for op, r, b in zip(ops, ref, tiled.bufs):
        assert np.array_equal(host(b["y"]).view(np.uint32), r.view(np.uint32)), op.name
