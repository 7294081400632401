"""A decode step of stacked Q8_0 projections, run through the C ABI.

"Filling in the blanks: Inference using Phobos", section Fast Decode, describes the
decode pass as recorded once and replayed (with nothing allocated during recording), with
each activation quantized a single time, projections with a common input run together and
the residual joined to the product's output.
This module lays one step out three ways over the same buffers, allocated up front:
  * per projection one q8_quantize_act and one gemv_stacked (or q8_gemv) launch on
    one stream, in dependency order; the step can be captured into a HIP graph;
  * per projection one gemv_stacked launch that quantizes the f32 input itself
    (except matrices with very many rows, where quantize + GEMV is faster);
  * the whole step as one q8_decode_stack launch (persistent workgroups, a device-wide
    barrier between projections, each input quantized once by the workgroups of the
    projection before it, the next projection's weights fetched during the barrier).
All three produce bit-identical outputs. Q8BatchStack runs nb decode streams at once
over the same weights: per projection one q8_quantize_act over all nb inputs and one
q8_gemv_batch launch (stacked parts are row ranges of one matrix, so one launch
covers them), on weights packed once into the tiled layout.

Each projection's input is its own buffer: the layers in between (norms, attention,
activations) are not part of this path, so the inputs are seeded synthetic vectors.
"""
from __future__ import annotations

import numpy as np
import torch

from . import DecodeStackPlan, gemv_stacked, pack_tile16, q8_gemv, q8_gemv_batch, q8_quantize_act


def _dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class Q8DecodeStack:
    """Device-resident weights, inputs and outputs for a list of projections.

    ops: sequence of objects with .name, .parts (row counts sharing one input), .k,
    .residual (bool). host: per op a dict with "qw" int8 [n, k], "dw" uint16 [n, k/32],
    "x" f32 [k], and "r" f32 [n] when the op folds in a residual.
    """

    def __init__(self, ops, host, device="cuda"):
        self.ops = list(ops)
        self.device = torch.device(device)
        self.bufs = []
        for op, h in zip(self.ops, host):
            n, k = op.n, op.k
            b = {
                "qw": _dev(h["qw"], self.device),
                "dw": _dev(h["dw"].view(np.int16), self.device).view(torch.float16),
                "x": _dev(h["x"], self.device),
                "qx": torch.empty(k, dtype=torch.int8, device=self.device),
                "dx": torch.empty(k // 32, dtype=torch.float16, device=self.device),
                "y": torch.empty(n, dtype=torch.float32, device=self.device),
                "r": _dev(h["r"], self.device) if op.residual else None,
            }
            parts, off = [], 0
            for s in op.parts:
                parts.append({
                    "w": b["qw"][off:off + s],
                    "dw": b["dw"][off:off + s],
                    "y": b["y"][off:off + s],
                    "residual": b["r"][off:off + s] if b["r"] is not None else None,
                })
                off += s
            b["parts"] = parts
            self.bufs.append(b)
        self.graph = None
        self.plan = None

    def tiled(self, i):
        """Op i's weights in the 16-row tiled layout of q8_gemv_batch (a Tile16), packed once
        on first use from the row-layout copy, as a loader would when the weights arrive."""
        b = self.bufs[i]
        if "t16" not in b:
            qw = b["qw"].cpu().numpy()
            dw = b["dw"].cpu().view(torch.int16).numpy().view(np.uint16)
            b["t16"] = pack_tile16(qw, dw, device=self.device)
        return b["t16"]

    def make_plan(self):
        """Descriptors for the one-launch executor (q8_decode_stack) over the same buffers."""
        ops = []
        for b in self.bufs:
            ops.append({"x": b["x"], "qx": b["qx"], "dx": b["dx"], "parts": b["parts"]})
        self.plan = DecodeStackPlan(ops, device=self.device)
        return self.plan

    def step_persistent(self, stream=None):
        """One token as a single launch of q8_decode_stack."""
        if self.plan is None:
            self.make_plan()
        self.plan.run(stream)

    def launch_op(self, i, stream=None):
        """Quantize op i's input once, then one launch over its stacked parts."""
        b = self.bufs[i]
        q8_quantize_act(b["x"], b["qx"], b["dx"], stream=stream)
        if len(b["parts"]) == 1:
            p = b["parts"][0]
            q8_gemv(p["w"], p["dw"], b["qx"], b["dx"], y=p["y"], residual=p["residual"], stream=stream)
        else:
            gemv_stacked(b["parts"], b["qx"], b["dx"], stream=stream)

    def launch_op_gemv_only(self, i, stream=None):
        """The GEMV launch of op i alone (its activation already quantized)."""
        b = self.bufs[i]
        if len(b["parts"]) == 1:
            p = b["parts"][0]
            q8_gemv(p["w"], p["dw"], b["qx"], b["dx"], y=p["y"], residual=p["residual"], stream=stream)
        else:
            gemv_stacked(b["parts"], b["qx"], b["dx"], stream=stream)

    def launch_op_fused(self, i, stream=None):
        """One launch for op i: the f32 input is quantized inside the GEMV launch."""
        b = self.bufs[i]
        gemv_stacked(b["parts"], b["x"], stream=stream)

    def step(self, stream=None, fused=False):
        # fused: every projection one launch, the 151936-row head included (each of its
        # workgroups quantizes the whole input again for 16 rows of output, while its first
        # weights are in flight; on MI355X 27.0 us against 27.2 + 1.6 us as quantize + GEMV)
        for i, op in enumerate(self.ops):
            if fused:
                self.launch_op_fused(i, stream)
            else:
                self.launch_op(i, stream)

    def capture(self, fused=False):
        """Record one step into a HIP graph (nothing is allocated while recording)."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            self.step(fused=fused)  # warm: loads the code objects before recording
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(fused=fused)
        torch.cuda.synchronize(self.device)
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()


class Q8BatchStack:
    """nb activation vectors per projection over the weights of a Q8DecodeStack (shared,
    not copied). batch: per op a dict with "x" f32 [nb, k] and "r" f32 [nb, n] or None.
    tiled: run the GEMVs on the tiled weight layout (packed here, once); the outputs are
    the row layout's bit for bit, and on MI355X every projection of the 0.8B shape runs
    faster (4-24%, the head most)."""

    def __init__(self, stack: Q8DecodeStack, batch, tiled: bool = True):
        self.stack = stack
        self.tiled = bool(tiled)
        self.nb = batch[0]["x"].shape[0]
        dev = stack.device
        self.bufs = []
        for b, h in zip(stack.bufs, batch):
            nb, k = h["x"].shape
            n = b["qw"].shape[0]
            self.bufs.append({
                "x": _dev(h["x"].reshape(-1), dev),
                "qx": torch.empty(nb * k, dtype=torch.int8, device=dev),
                "dx": torch.empty(nb * k // 32, dtype=torch.float16, device=dev),
                "y": torch.empty((nb, n), dtype=torch.float32, device=dev),
                "r": _dev(h["r"], dev) if h["r"] is not None else None,
                "k": k,
            })
        if self.tiled:
            for i in range(len(self.bufs)):
                stack.tiled(i)

    def launch_quantize(self, i, stream=None):
        b = self.bufs[i]
        q8_quantize_act(b["x"], b["qx"], b["dx"], stream=stream)

    def weights(self, i):
        """(qw, dw) for q8_gemv_batch: op i's Tile16 and None, or its row-layout planes."""
        if self.tiled:
            return self.stack.tiled(i), None
        s = self.stack.bufs[i]
        return s["qw"], s["dw"]

    def launch_gemv(self, i, stream=None):
        b = self.bufs[i]
        k = b["k"]
        q8_gemv_batch(*self.weights(i), b["qx"].view(self.nb, k), b["dx"].view(self.nb, k // 32), y=b["y"],
                      residual=b["r"], stream=stream)

    def step(self, stream=None):
        for i in range(len(self.bufs)):
            self.launch_quantize(i, stream)
            self.launch_gemv(i, stream)
