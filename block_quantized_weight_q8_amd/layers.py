"""Decode layers with their neighbour steps, run through the C ABI.

"One level down: #002 the same compiler on a GPU", section Emitting for a GPU: for
decode, two kernels each merge a neighbour step into the next projection, one the
normalization and one the activation. "Filling in the blanks: Inference using
Phobos", section Q4_K_M, names a block's operations: RMS normalization before the
attention and MLP projections, and the gated MLP; section Fast Decode: one activation
quantization reused by all consumers, the residual added inside the matmul, the whole pass
recorded once and replayed as a graph.

Q8LayerChain runs the projections of every layer with the real data flow through
the residual stream h (attention itself is not part of this path; its output is a
seeded stand-in per layer). One token, fused (4 launches per layer):
    QKV    gemv_stacked_rmsnorm(h, gamma_attn)                 q, k, v
    out    gemv_stacked(attn f32), residual h, in place          h += W_o attn
    MLP    q8_gateup_rmsnorm_silu(h, gamma_mlp)                  a = silu(gate) up, f32
    down   gemv_stacked(a f32), residual h, in place             h += W_d a
then the head with the final normalization in its prologue (gemv_stacked_rmsnorm).
Unfused (8 launches per layer) runs every normalization, activation and quantize as
its own launch, and the head as q8_rmsnorm_quantize_act then q8_gemv. Both give the
same bits.

Q8BatchLayerChain runs the same layers for nb decode streams at once over the same
weights (8 launches per layer): every projection is one q8_gemv_batch over the nb
vectors, each neighbour step one batched launch (normalize + quantize, silu * up +
quantize, quantize), and the residual streams are updated in place.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (gemv_stacked, gemv_stacked_rmsnorm, q8_gateup_silu, q8_gemv, q8_gemv_batch, q8_quantize_act,
               q8_rmsnorm_quantize_act, q8_silu_mul_quantize_act)


def _dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class Q8LayerChain:
    """Layer chain over the weights of a Q8DecodeStack laid out per layer as [qkv (3 parts),
    out, gate+up (2 parts: gate, up), down], then the head. inputs: synth.layer_chain_inputs."""

    def __init__(self, stack, inputs, eps: float = 1e-6):
        self.stack = stack
        self.eps = float(eps)
        dev = stack.device
        ops = stack.ops
        if (len(ops) - 1) % 4:
            raise ValueError("expected 4 projections per layer and a head")
        self.layers = (len(ops) - 1) // 4
        for l in range(self.layers):
            qkv, out, gu, down = ops[4 * l:4 * l + 4]
            if len(gu.parts) != 2 or gu.parts[0] != gu.parts[1] or down.k != gu.parts[0]:
                raise ValueError(f"layer {l}: gate+up must be two equal parts feeding down")
            if out.n != qkv.k or down.n != qkv.k or gu.k != qkv.k:
                raise ValueError(f"layer {l}: projections do not share the hidden width")
        self.hidden = ops[0].k
        self.ffn = ops[2].parts[0]
        self.h0 = _dev(inputs["h"], dev)
        self.h = torch.empty_like(self.h0)
        self.gamma_attn = [_dev(g, dev) for g in inputs["gamma_attn"]]
        self.gamma_mlp = [_dev(g, dev) for g in inputs["gamma_mlp"]]
        self.attn = [_dev(a, dev) for a in inputs["attn"]]
        self.gamma_final = _dev(inputs["gamma_final"], dev)
        k, f = self.hidden, self.ffn
        self.qx = torch.empty(k, dtype=torch.int8, device=dev)
        self.dx = torch.empty(k // 32, dtype=torch.float16, device=dev)
        self.qo = torch.empty(ops[1].k, dtype=torch.int8, device=dev)
        self.do = torch.empty(ops[1].k // 32, dtype=torch.float16, device=dev)
        self.qa = torch.empty(f, dtype=torch.int8, device=dev)
        self.da = torch.empty(f // 32, dtype=torch.float16, device=dev)
        self.gu = torch.empty(2 * f, dtype=torch.float32, device=dev)
        self.a = torch.empty(f, dtype=torch.float32, device=dev)  # silu(gate) * up, f32

    def _b(self, l, j):
        return self.stack.bufs[4 * l + j]

    def qkv_parts(self, l):
        return self._b(l, 0)["parts"]

    def out_parts(self, l, h_in):
        """The out projection writes h = h_in + W_o attn (h_in is h0 for layer 0, else h)."""
        p = self._b(l, 1)["parts"][0]
        return [{"w": p["w"], "dw": p["dw"], "y": self.h, "residual": h_in}]

    def gate_up(self, l):
        b = self._b(l, 2)
        f = self.ffn
        return b["qw"][:f], b["dw"][:f], b["qw"][f:], b["dw"][f:]

    def head(self):
        return self.stack.bufs[-1]

    @property
    def logits(self):
        return self.head()["y"]

    def step(self, fused: bool = True, stream=None, trace=None):
        """One token. trace (a list) receives host copies after every step, for parity checks."""
        eps = self.eps

        def snap(name, l, t):
            if trace is not None:
                torch.cuda.synchronize()
                trace.append((name, l, t.detach().cpu().clone()))

        for l in range(self.layers):
            h_in = self.h0 if l == 0 else self.h
            snap("h_in", l, h_in)
            if fused:
                gemv_stacked_rmsnorm(self.qkv_parts(l), h_in, self.gamma_attn[l], eps, stream=stream)
                gemv_stacked(self.out_parts(l, h_in), self.attn[l], stream=stream)
                q8_gateup_silu(*self.gate_up(l), self.h, gamma=self.gamma_mlp[l], eps=eps, a=self.a, stream=stream)
                if trace is not None:  # the codes the down projection forms from a, for the snapshots
                    q8_quantize_act(self.a, self.qa, self.da, stream=stream)
            else:
                q8_rmsnorm_quantize_act(h_in, self.gamma_attn[l], eps, qx=self.qx, dx=self.dx, stream=stream)
                snap("qkv_codes", l, torch.cat([self.qx.view(torch.uint8), self.dx.view(torch.uint8)]))
                gemv_stacked(self.qkv_parts(l), self.qx, self.dx, stream=stream)
                q8_quantize_act(self.attn[l], self.qo, self.do, stream=stream)
                gemv_stacked(self.out_parts(l, h_in), self.qo, self.do, stream=stream)
                snap("h_mid", l, self.h)
                q8_rmsnorm_quantize_act(self.h, self.gamma_mlp[l], eps, qx=self.qx, dx=self.dx, stream=stream)
                f = self.ffn
                wg, dg, wu, du = self.gate_up(l)
                gemv_stacked([{"w": wg, "dw": dg, "y": self.gu[:f]}, {"w": wu, "dw": du, "y": self.gu[f:]}],
                             self.qx, self.dx, stream=stream)
                snap("gu", l, self.gu)
                q8_silu_mul_quantize_act(self.gu, self.qa, self.da, stream=stream)
            snap("qkv", l, self._b(l, 0)["y"])
            snap("a_codes", l, torch.cat([self.qa.view(torch.uint8), self.da.view(torch.uint8)]))
            b = self._b(l, 3)
            if fused:  # f32 input, quantized in the launch
                gemv_stacked([{"w": b["qw"], "dw": b["dw"], "y": self.h, "residual": self.h}], self.a, stream=stream)
            else:
                q8_gemv(b["qw"], b["dw"], self.qa, self.da, y=self.h, residual=self.h, stream=stream)
        snap("h_out", self.layers - 1, self.h)
        hb = self.head()
        if fused:
            gemv_stacked_rmsnorm([{"w": hb["qw"], "dw": hb["dw"], "y": hb["y"]}], self.h, self.gamma_final, eps,
                                 stream=stream)
        else:
            q8_rmsnorm_quantize_act(self.h, self.gamma_final, eps, qx=self.qx, dx=self.dx, stream=stream)
            q8_gemv(hb["qw"], hb["dw"], self.qx, self.dx, y=hb["y"], stream=stream)
        snap("logits", self.layers, hb["y"])

    def launches_per_token(self, fused: bool = True) -> int:
        return self.layers * 4 + 1 if fused else self.layers * 8 + 2


class Q8BatchLayerChain:
    """nb decode streams through the layers of a Q8DecodeStack (weights shared, not copied).
    inputs: synth.layer_chain_inputs (its normalization weights serve every stream);
    batch_inputs: synth.layer_chain_batch_inputs (per stream the residual stream entering
    layer 0, h f32 [nb, hidden], and per layer the attention stand-in, f32 [nb, attn_width]).
    tiled: the GEMVs read the weights in the tiled layout (packed once here); the outputs are
    the row layout's bit for bit."""

    def __init__(self, stack, inputs, batch_inputs, eps: float = 1e-6, tiled: bool = True):
        self.stack = stack
        self.eps = float(eps)
        self.tiled = bool(tiled)
        dev = stack.device
        ops = stack.ops
        if self.tiled:  # the weights packed once into the tiled layout (same outputs, faster)
            for i in range(len(ops)):
                stack.tiled(i)
        self.layers = (len(ops) - 1) // 4
        self.hidden = ops[0].k
        self.ffn = ops[2].parts[0]
        self.nb = batch_inputs["h"].shape[0]
        nb, k, f = self.nb, self.hidden, self.ffn
        self.h0 = _dev(batch_inputs["h"], dev)
        self.h = torch.empty_like(self.h0)
        self.attn = [_dev(a, dev) for a in batch_inputs["attn"]]
        self.gamma_attn = [_dev(g, dev) for g in inputs["gamma_attn"]]
        self.gamma_mlp = [_dev(g, dev) for g in inputs["gamma_mlp"]]
        self.gamma_final = _dev(inputs["gamma_final"], dev)
        self.qx = torch.empty((nb, k), dtype=torch.int8, device=dev)
        self.dx = torch.empty((nb, k // 32), dtype=torch.float16, device=dev)
        aw = ops[1].k
        self.qo = torch.empty((nb, aw), dtype=torch.int8, device=dev)
        self.do = torch.empty((nb, aw // 32), dtype=torch.float16, device=dev)
        self.qa = torch.empty((nb, f), dtype=torch.int8, device=dev)
        self.da = torch.empty((nb, f // 32), dtype=torch.float16, device=dev)
        self.qkv = torch.empty((nb, ops[0].n), dtype=torch.float32, device=dev)
        self.gu = torch.empty((nb, 2 * f), dtype=torch.float32, device=dev)
        self.logits = torch.empty((nb, ops[-1].n), dtype=torch.float32, device=dev)

    def _w(self, i):
        if self.tiled:
            return self.stack.tiled(i), None
        b = self.stack.bufs[i]
        return b["qw"], b["dw"]

    def step(self, stream=None, trace=None):
        eps = self.eps

        def snap(name, l, t):
            if trace is not None:
                torch.cuda.synchronize()
                trace.append((name, l, t.detach().cpu().clone()))

        for l in range(self.layers):
            h_in = self.h0 if l == 0 else self.h
            snap("h_in", l, h_in)
            q8_rmsnorm_quantize_act(h_in, self.gamma_attn[l], eps, qx=self.qx, dx=self.dx, stream=stream)
            snap("qkv_codes", l, torch.cat([self.qx.view(torch.uint8), self.dx.view(torch.uint8)], dim=1))
            q8_gemv_batch(*self._w(4 * l), self.qx, self.dx, y=self.qkv, stream=stream)
            snap("qkv", l, self.qkv)
            q8_quantize_act(self.attn[l].view(-1), self.qo.view(-1), self.do.view(-1), stream=stream)
            q8_gemv_batch(*self._w(4 * l + 1), self.qo, self.do, y=self.h, residual=h_in, stream=stream)
            snap("h_mid", l, self.h)
            q8_rmsnorm_quantize_act(self.h, self.gamma_mlp[l], eps, qx=self.qx, dx=self.dx, stream=stream)
            q8_gemv_batch(*self._w(4 * l + 2), self.qx, self.dx, y=self.gu, stream=stream)
            snap("gu", l, self.gu)
            q8_silu_mul_quantize_act(self.gu, self.qa, self.da, stream=stream)
            snap("a_codes", l, torch.cat([self.qa.view(torch.uint8), self.da.view(torch.uint8)], dim=1))
            q8_gemv_batch(*self._w(4 * l + 3), self.qa, self.da, y=self.h, residual=self.h, stream=stream)
        snap("h_out", self.layers - 1, self.h)
        q8_rmsnorm_quantize_act(self.h, self.gamma_final, eps, qx=self.qx, dx=self.dx, stream=stream)
        q8_gemv_batch(*self._w(len(self.stack.ops) - 1), self.qx, self.dx, y=self.logits, stream=stream)
        snap("logits", self.layers, self.logits)

    def launches_per_token_step(self) -> int:
        return self.layers * 8 + 2
