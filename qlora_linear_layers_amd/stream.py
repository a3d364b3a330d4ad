"""Layer-by-layer quantization of a weight stack with one layer resident.

The pages' memory arithmetic ("QLoRA 原理精讲", section 2.2 with its storage
figure, and the memory table of section 2.4: about 35 GB of 4-bit weights for
70B parameters, against about 140 GB in bf16) is about the stored format; the
bf16 source never needs to be resident as a whole.  This driver walks the
layers in order: it obtains one layer's bf16
weights from a caller-supplied function, quantizes all its tensors with one
``nf4_quantize_dq_grouped`` launch into storage that is reused for every layer,
dequantizes them back with one ``nf4_dequantize_dq_grouped`` launch into reused
bf16 buffers, hands both to an
optional per-layer callback (to keep, check or copy out what it needs), and then
drops the layer's weights before the next one is drawn.

All arithmetic runs in the library's kernels; this module only orders calls and
allocates the reused buffers once.
"""
import torch

from . import api


class LayerStream:
    """Reused storage for the tensors of one layer: shapes are (N, K) pairs."""

    def __init__(self, shapes, device="cuda"):
        self.shapes = [tuple(s) for s in shapes]
        self.qws = []
        self.wds = []
        for N, K in self.shapes:
            numel = N * K
            if numel % 64:
                raise ValueError(f"tensor {N}x{K}: element count must be a multiple of 64")
            self.qws.append(api.NF4Weight(
                torch.empty(numel // 2, dtype=torch.uint8, device=device),
                torch.empty(numel // 64, dtype=torch.uint8, device=device),
                torch.empty(-(-numel // 16384), dtype=torch.float32, device=device), N, K))
            self.wds.append(torch.empty((N, K), dtype=torch.bfloat16, device=device))

    def run(self, weights_of_layer, n_layers, on_layer=None, timed=True):
        """Quantize then dequantize every tensor of layers 0 .. n_layers-1.

        weights_of_layer(l) -> list of bf16 [N, K] device tensors in self.shapes
        order.  on_layer(l, weights, qws, wds) runs after layer l's kernels are
        enqueued (it may synchronize).  With timed=False nothing waits for the
        last layer's kernels.  Returns a dict with the seconds spent in
        the quantize + dequantize launches (HIP events on the current stream, the
        weight generation between layers excluded) and the packed bytes of every
        layer's storage."""
        stream = torch.cuda.current_stream() if timed else None
        events = []
        packed = 0
        for l in range(n_layers):
            ws = weights_of_layer(l)
            if len(ws) != len(self.shapes):
                raise ValueError(f"layer {l}: {len(ws)} tensors, expected {len(self.shapes)}")
            for w, (N, K) in zip(ws, self.shapes):
                if tuple(w.shape) != (N, K):
                    raise ValueError(f"layer {l}: tensor of shape {tuple(w.shape)}, expected {(N, K)}")
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
            if ev:
                ev[0].record(stream)
            # all tensors of the layer in one launch per step (at most 16 per launch)
            for i in range(0, len(ws), api.MAX_TENSORS):
                api.nf4_quantize_dq_grouped(ws[i:i + api.MAX_TENSORS], self.qws[i:i + api.MAX_TENSORS])
            for i in range(0, len(ws), api.MAX_TENSORS):
                api.nf4_dequantize_dq_grouped(self.qws[i:i + api.MAX_TENSORS], self.wds[i:i + api.MAX_TENSORS])
            if ev:
                ev[1].record(stream)
                events.append(ev)
            packed += sum(qw.nbytes() for qw in self.qws)
            if on_layer is not None:
                on_layer(l, ws, self.qws, self.wds)
            del ws
        secs = None
        if events:
            torch.cuda.synchronize()
            secs = sum(a.elapsed_time(b) for a, b in events) / 1e3
        return {"seconds": secs, "packed_bytes": packed, "layers": n_layers}
