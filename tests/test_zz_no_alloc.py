"""q8_decode_stack_static (no allocation: the library's own static workspace, cleared by
each call) against q8_decode_stack (a caller workspace), through the C ABI.

Two stacks are first run through q8_decode_stack and their outputs kept; then
q8_decode_stack_static runs both, back to back (the second stack smaller), and every
output, code and scale must equal the reference bit for bit (same kernel, same
instructions). Needs an MI355X.
"""
import numpy as np
import pytest

import synth

pytestmark = [pytest.mark.gpu]


@pytest.fixture(scope="module")
def q8():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_q8_amd as m

    m.load_library()
    return m


def snapshot(st):
    import torch

    torch.cuda.synchronize()
    return [(b["y"].cpu().numpy().copy(), b["qx"].cpu().numpy().copy(),
             b["dx"].cpu().view(torch.int16).numpy().copy()) for b in st.bufs]


def poison(st):
    for b in st.bufs:
        b["y"].fill_(float("nan"))
        b["qx"].fill_(0)
        b["dx"].fill_(0)


def test_static_workspace_matches_caller_workspace(q8):
    import torch

    from block_quantized_weight_q8_amd.stack import Q8DecodeStack

    print("case: static-workspace decode stack, 3 layers + 20000-row head, then 1 layer + 3000-row head",
          flush=True)
    stacks, refs = [], []
    for n, (layers, vocab) in enumerate([(3, 20000), (1, 3000)]):
        ops = synth.q8_stack_08b(layers=layers, vocab=vocab)
        st = Q8DecodeStack(ops, synth.q8_stack_inputs(ops, synth.TAG_TEST + 40 + n))
        st.make_plan()
        st.plan.run()
        refs.append(snapshot(st))
        assert st.plan.error_flag() == 0
        stacks.append(st)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for st in stacks:
        poison(st)
    for st in stacks:  # two calls in a row, the second smaller
        st.plan.run_static(status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a static-workspace launch gave up waiting"
    for n, (st, ref) in enumerate(zip(stacks, refs)):
        got = snapshot(st)
        for op, (y0, q0, d0), (y1, q1, d1) in zip(st.ops, ref, got):
            assert np.array_equal(q0, q1) and np.array_equal(d0, d1), f"stack {n} {op.name}: codes differ"
            assert np.array_equal(y0, y1), f"stack {n} {op.name}: outputs differ"
    # and once more on the first stack: the cleared workspace carries nothing over
    poison(stacks[0])
    stacks[0].plan.run_static()
    got = snapshot(stacks[0])
    for op, (y0, _, _), (y1, _, _) in zip(stacks[0].ops, refs[0], got):
        assert np.array_equal(y0, y1), f"repeat {op.name}: outputs differ"
