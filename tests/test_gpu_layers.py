"""Decode layers with their neighbour steps, HIP path vs the oracle (needs an MI355X).

The chain of Q8LayerChain (QKV with its normalization, the out projection into the
residual stream, the MLP front with silu(gate) * up quantized in the gate+up epilogue,
the down projection into the residual stream; then the final normalization and the head)
must give the same bits fused (4 launches per layer) and unfused (8 launches per layer),
eager and replayed from a HIP graph. Every step of the unfused run is checked against
the oracle on the GPU's own input to that step: codes and scales bit-exact, f32 outputs
within 1e-5 * S.
"""
import numpy as np
import pytest

import synth
from tests.test_gpu_parity import print_case, within

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

EPS = 1e-6
LAYERS, VOCAB = 2, 8192


@pytest.fixture(scope="module")
def chain():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_q8_amd as m
    from block_quantized_weight_q8_amd.layers import Q8LayerChain
    from block_quantized_weight_q8_amd.stack import Q8DecodeStack

    m.load_library()
    ops = synth.q8_stack_08b(layers=LAYERS, vocab=VOCAB)
    host = synth.q8_stack_inputs(ops)
    stack = Q8DecodeStack(ops, host)
    inputs = synth.layer_chain_inputs(layers=LAYERS)
    return Q8LayerChain(stack, inputs, eps=EPS), ops, host, inputs


def by_name(trace):
    return {(n, l): t.numpy() for n, l, t in trace}


def codes_split(buf, k):
    """(codes int8 [k], scale bits uint16 [k/32]) from a snapshot of codes then scales as bytes."""
    b = np.asarray(buf, dtype=np.uint8)
    return b[:k].view(np.int8), b[k:].view(np.uint16)


def test_fused_equals_unfused_bit_for_bit(chain):
    print_case("layer chain fused vs unfused")
    ch, ops, host, inputs = chain
    tf, tu = [], []
    ch.step(fused=True, trace=tf)
    lf = ch.logits.cpu().numpy().copy()
    ch.step(fused=False, trace=tu)
    lu = ch.logits.cpu().numpy().copy()
    assert np.array_equal(lf, lu)
    f, u = by_name(tf), by_name(tu)
    for key in f:
        assert np.array_equal(f[key], u[key]), f"{key} differs between fused and unfused"


def test_every_step_against_the_oracle(chain, orc):
    print_case("layer chain steps vs oracle")
    ch, ops, host, inputs = chain
    tr = []
    ch.step(fused=False, trace=tr)
    t = by_name(tr)
    k, f = ch.hidden, ch.ffn
    for l in range(LAYERS):
        qkv, out, gu, down = (host[4 * l + j] for j in range(4))
        h_in = t[("h_in", l)]
        rq, rd = orc.quantize_act(orc.rmsnorm(h_in, inputs["gamma_attn"][l], EPS))
        gq, gd = codes_split(t[("qkv_codes", l)], k)
        assert np.array_equal(gq, rq) and np.array_equal(gd, rd), f"layer {l}: normalized codes"
        yr, S = orc.q8_gemv(qkv["qw"], qkv["dw"], rq, rd)
        within(t[("qkv", l)], yr, S, f"layer {l} qkv")
        oq, od = orc.quantize_act(inputs["attn"][l])
        yr, S = orc.q8_gemv(out["qw"], out["dw"], oq, od, h_in)
        h_mid = t[("h_mid", l)]
        within(h_mid, yr, S, f"layer {l} out + residual")
        mq, md = orc.quantize_act(orc.rmsnorm(h_mid, inputs["gamma_mlp"][l], EPS))
        yr, S = orc.q8_gemv(gu["qw"], gu["dw"], mq, md)
        g = t[("gu", l)]
        within(g, yr, S, f"layer {l} gate+up")
        aq, ad = orc.quantize_act(orc.silu_mul(g))
        gq, gd = codes_split(t[("a_codes", l)], f)
        assert np.array_equal(gq, aq) and np.array_equal(gd, ad), f"layer {l}: activation codes"
        yr, S = orc.q8_gemv(down["qw"], down["dw"], aq, ad, h_mid)
        h_next = t[("h_in", l + 1)] if l + 1 < LAYERS else t[("h_out", l)]
        within(h_next, yr, S, f"layer {l} down + residual")
    fq, fd = orc.quantize_act(orc.rmsnorm(t[("h_out", LAYERS - 1)], inputs["gamma_final"], EPS))
    yr, S = orc.q8_gemv(host[-1]["qw"], host[-1]["dw"], fq, fd)
    within(t[("logits", LAYERS)], yr, S, "head")


def test_graph_replays_match_eager(chain):
    import torch

    print_case("layer chain graph replay")
    ch, ops, host, inputs = chain
    ch.step(fused=True)
    torch.cuda.synchronize()
    ref = ch.logits.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ch.step(fused=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ch.step(fused=True)
    for _ in range(3):
        ch.logits.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(ch.logits.cpu().numpy(), ref)
        ch.step(fused=False)  # eager work between replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------- 16 streams


NB = 16


@pytest.fixture(scope="module")
def batch_chain(chain):
    from block_quantized_weight_q8_amd.layers import Q8BatchLayerChain

    ch, ops, host, inputs = chain
    binp = synth.layer_chain_batch_inputs(NB, layers=LAYERS)
    return Q8BatchLayerChain(ch.stack, inputs, binp, eps=EPS), host, inputs, binp


def test_batched_neighbour_quantize_rows_equal_single(q8_mod):
    """The batched normalize/silu quantize launches give each row exactly the single-vector bits."""
    import torch

    print_case("batched neighbour quantize rows")
    g = synth.rng_for(synth.TAG_NEIGHBOUR, 6000)
    k = 1024
    x = np.stack([synth.activation_f32(g, k) for _ in range(5)])
    gamma = synth.norm_gamma(g, k)
    gu = np.stack([synth.gate_up_f32(g, k) for _ in range(5)])
    X, G, GU = (torch.from_numpy(a).cuda() for a in (x, gamma, gu))
    qb, db = q8_mod.q8_rmsnorm_quantize_act(X, G, EPS)
    qs, ds = q8_mod.q8_silu_mul_quantize_act(GU)
    for i in range(5):
        q1, d1 = q8_mod.q8_rmsnorm_quantize_act(X[i], G, EPS)
        assert torch.equal(qb[i], q1) and torch.equal(db[i].view(torch.int16), d1.view(torch.int16))
        q2, d2 = q8_mod.q8_silu_mul_quantize_act(GU[i])
        assert torch.equal(qs[i], q2) and torch.equal(ds[i].view(torch.int16), d2.view(torch.int16))


@pytest.fixture(scope="module")
def q8_mod(chain):
    import block_quantized_weight_q8_amd as m

    return m


def test_batched_chain_every_step_against_the_oracle(batch_chain, orc):
    print_case("batched layer chain steps vs oracle")
    bc, host, inputs, binp = batch_chain
    tr = []
    bc.step(trace=tr)
    t = by_name(tr)
    k, f = bc.hidden, bc.ffn
    for l in range(LAYERS):
        qkv, out, gu, down = (host[4 * l + j] for j in range(4))
        for v in (0, 7, NB - 1):
            h_in = t[("h_in", l)][v]
            rq, rd = orc.quantize_act(orc.rmsnorm(h_in, inputs["gamma_attn"][l], EPS))
            gq, gd = codes_split(t[("qkv_codes", l)][v], k)
            assert np.array_equal(gq, rq) and np.array_equal(gd, rd), f"layer {l} stream {v}: normalized codes"
            yr, S = orc.q8_gemv(qkv["qw"], qkv["dw"], rq, rd)
            within(t[("qkv", l)][v], yr, S, f"layer {l} stream {v} qkv")
            oq, od = orc.quantize_act(binp["attn"][l][v])
            yr, S = orc.q8_gemv(out["qw"], out["dw"], oq, od, h_in)
            h_mid = t[("h_mid", l)][v]
            within(h_mid, yr, S, f"layer {l} stream {v} out + residual")
            mq, md = orc.quantize_act(orc.rmsnorm(h_mid, inputs["gamma_mlp"][l], EPS))
            yr, S = orc.q8_gemv(gu["qw"], gu["dw"], mq, md)
            g = t[("gu", l)][v]
            within(g, yr, S, f"layer {l} stream {v} gate+up")
            aq, ad = orc.quantize_act(orc.silu_mul(g))
            gq, gd = codes_split(t[("a_codes", l)][v], f)
            assert np.array_equal(gq, aq) and np.array_equal(gd, ad), f"layer {l} stream {v}: activation codes"
            yr, S = orc.q8_gemv(down["qw"], down["dw"], aq, ad, h_mid)
            h_next = t[("h_in", l + 1)][v] if l + 1 < LAYERS else t[("h_out", l)][v]
            within(h_next, yr, S, f"layer {l} stream {v} down + residual")
    for v in (0, NB - 1):
        fq, fd = orc.quantize_act(orc.rmsnorm(t[("h_out", LAYERS - 1)][v], inputs["gamma_final"], EPS))
        yr, S = orc.q8_gemv(host[-1]["qw"], host[-1]["dw"], fq, fd)
        within(t[("logits", LAYERS)][v], yr, S, f"head stream {v}")


def test_batched_chain_graph_replays_match_eager(batch_chain):
    import torch

    print_case("batched layer chain graph replay")
    bc, host, inputs, binp = batch_chain
    bc.step()
    torch.cuda.synchronize()
    ref = bc.logits.cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bc.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bc.step()
    for _ in range(3):
        bc.logits.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bc.logits.cpu().numpy(), ref)
        bc.step()
        torch.cuda.synchronize()
