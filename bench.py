#!/usr/bin/env python
"""Benchmark of the QLoRA frozen-base linear layer hot path on one MI355X.

Workload (one "step"): the seven linears of a LLaMA-7B-shaped transformer
layer (q/k/v/o 4096x4096, gate/up 11008x4096, down 4096x11008) at training
shape T = 8 x 512 = 4096 tokens, LoRA rank 64, alpha 16 (s = 0.25).  The step
runs the whole path: NF4 + double quantization of the seven bf16 weights (one
grouped launch), their double dequantization back to bf16 (one grouped
launch), and for each linear the fused forward Y = X W'^T + s (X A) B and the
backward dX = dY W' + s (dY B^T) A^T with the LoRA gradients dA, dB.  Inputs are seeded synthetic tensors (W ~ N(0, 0.02),
X, dY ~ N(0, 1), A, B ~ N(0, 0.01)), resident in HBM before timing starts.

Output: one JSON line.  `value` is the step's attainment of the MI355X
roofline: the sum over all phases of their roofline time (algorithmic bytes at
8 TB/s for quantize / dequantize, algorithmic flops at 2.5 PFLOP/s bf16 dense
for the GEMM phases) divided by the measured step time.  Per-phase durations
come from HIP events recorded on the stream the kernels run on.  Outside the
step, `components` also carries the decode forward (T = 1 / 4 / 8), the LoRA
merge, the single-quantization variant, the fp16 compute type and the
NF4-vs-INT4 data-type ablation measured on the same seven linears, the
65B-shaped layer and the 70B-shaped streaming quantization.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense
GEMM_SOURCE = os.path.join(ROOT, "qlora_linear_layers_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fwd_llama7b_T4096_traffic.txt")
COPY_BYTES = 256 << 20     # calibration copy for the HBM byte counters


def source_hash():
    import hashlib
    with open(GEMM_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def stored_traffic():
    """HBM bytes per k_fwd launch from the committed counter summary, if it was taken
    on the current GEMM source (otherwise None)."""
    try:
        kv = dict(l.strip().split("=", 1) for l in open(TRAFFIC_FILE) if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get("gemm_source_sha256_16") != source_hash():
        return None
    return float(kv["hbm_bytes_per_launch"])


def measure_roofline_kernel(api, torch, layers, bufs, reps):
    """k_fwd alone: the forward with r = 0 is exactly one launch of the fused
    NF4-dequant MFMA GEMM.  Returns (flops per launch, seconds per launch)."""
    ys = [torch.empty((b["x"].shape[0], b["lin"].N), dtype=torch.bfloat16, device="cuda") for b in bufs]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps * len(bufs))]
    for i, b in enumerate(bufs):
        api.qlora_linear_fwd(b["x"], b["qw"], out=ys[i])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for k in range(reps):
        for i, b in enumerate(bufs):
            e = ev[k * len(bufs) + i]
            e[0].record(stream)
            api.qlora_linear_fwd(b["x"], b["qw"], out=ys[i])
            e[1].record(stream)
    torch.cuda.synchronize()
    secs = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3 / len(ev)
    flops = sum(2 * b["x"].shape[0] * b["lin"].N * b["lin"].K for b in bufs) / len(bufs)
    return flops, secs


def storage_bytes(numel):
    return numel // 2 + numel // 64 + 4 * (-(-numel // 16384))


def phase_work(lin, T, r):
    """Algorithmic bytes (HBM phases) and flops (GEMM phases) of one linear."""
    N, K = lin.N, lin.K
    nk = N * K
    st = storage_bytes(nk)
    return {
        "quantize": ("hbm", 2 * nk + st),
        "dequantize": ("hbm", st + 2 * nk),
        "forward": ("mfma", 2 * T * N * K + 2 * T * K * r + 2 * T * r * N),
        # dX (base + LoRA), dY B^T, X A recompute, dA, dB
        "backward": ("mfma", 2 * T * N * K + 2 * T * N * r + 2 * T * r * K + 2 * T * K * r + 2 * T * K * r
                     + 2 * T * r * N),
    }


def roofline_seconds(kind, amount):
    return amount / (HBM_PEAK if kind == "hbm" else MFMA_BF16_PEAK)


def decode_bytes(lin, T, r):
    """Algorithmic bytes of one decode-size forward: the packed weight, X, Y and the adapters."""
    return storage_bytes(lin.N * lin.K) + 2 * T * lin.K + 2 * T * lin.N + 2 * r * (lin.K + lin.N)


def weight_copies(api, qws, copies=6):
    """`copies` copies of the quantized weights of the seven linears (about 100 MB
    each), rotated so that the 256 MB last-level cache cannot serve repeats."""
    return [[api.NF4Weight(q.codes.clone(), q.absmax_fp8.clone(), q.superscale.clone(), q.N, q.K) for q in qws]
            for _ in range(copies)]


DECODE_STAGES = ((0, 1, 2), (3,), (4, 5), (6,))    # q/k/v, o, gate/up, down: what a decode step can group


def measure_decode(api, torch, layers, sets, r, s, tokens=(1, 4, 8), reps=10, mode="single"):
    """Decode-size forward over the seven linears, one weight copy per pass.
    mode "single": one qlora_linear_fwd per linear; "staged": one grouped call
    per dependency stage (q/k/v, o, gate/up, down); "all": one grouped call for
    all seven.  A GPU spin ahead of the timed region lets the host enqueue every
    pass first, so the events see device time only.
    Returns {T: (seconds per layer set, bytes per layer set)}."""
    copies = len(sets)
    out = {}
    for T in tokens:
        g = torch.Generator(device="cuda").manual_seed(T)
        xs = [torch.randn((T, l.K), generator=g, device="cuda").to(torch.bfloat16) for l in layers]
        a = [torch.randn((l.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        b = [torch.randn((r, l.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        ys = [torch.empty((T, l.N), dtype=torch.bfloat16, device="cuda") for l in layers]
        stages = [tuple(range(len(layers)))] if mode == "all" else DECODE_STAGES
        if mode == "single":
            ws = torch.empty(max(api.qlora_workspace_bytes(T, l.K, l.N, r) for l in layers), dtype=torch.uint8,
                             device="cuda")
        else:
            ws = torch.empty(max(api.qlora_grouped_workspace_bytes(
                [(xs[i], sets[0][i], a[i], b[i], s, ys[i]) for i in st]) for st in stages), dtype=torch.uint8,
                device="cuda")

        def one(c):
            if mode == "single":
                for i, l in enumerate(layers):
                    api.qlora_linear_fwd(xs[i], sets[c][i], a[i], b[i], s, workspace=ws, out=ys[i])
            else:
                for st in stages:
                    api.qlora_linear_fwd_grouped([(xs[i], sets[c][i], a[i], b[i], s, ys[i]) for i in st],
                                                 workspace=ws)
        for c in range(copies):
            one(c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda._sleep(20_000_000)
        ev[0].record()
        for k in range(reps):
            one(k % copies)
        ev[1].record()
        torch.cuda.synchronize()
        secs = ev[0].elapsed_time(ev[1]) / 1e3 / reps
        out[T] = (secs, sum(decode_bytes(l, T, r) for l in layers))
    return out


def merge_bytes(lin, r):
    """Algorithmic bytes of one LoRA merge: the packed weight and the adapters in, bf16 W_m out."""
    return storage_bytes(lin.N * lin.K) + 2 * lin.N * lin.K + 2 * r * (lin.K + lin.N)


def measure_prefill(api, torch, layers, sets, r, s, tokens=(32, 64), reps=6):
    """Small-prefill forward (16 < T <= 128 runs 16-token windows as one grouped
    decode launch) over the seven linears, one weight copy per pass.
    Returns {T: (seconds per layer set, bytes per layer set, flops per layer set)}."""
    copies = len(sets)
    out = {}
    for T in tokens:
        g = torch.Generator(device="cuda").manual_seed(100 + T)
        xs = [torch.randn((T, l.K), generator=g, device="cuda").to(torch.bfloat16) for l in layers]
        a = [torch.randn((l.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        b = [torch.randn((r, l.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        ws = [torch.empty(api.qlora_workspace_bytes(T, l.K, l.N, r), dtype=torch.uint8, device="cuda") for l in layers]
        ys = [torch.empty((T, l.N), dtype=torch.bfloat16, device="cuda") for l in layers]

        def one(c):
            for i in range(len(layers)):
                api.qlora_linear_fwd(xs[i], sets[c][i], a[i], b[i], s, workspace=ws[i], out=ys[i])
        for c in range(copies):
            one(c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for k in range(reps):
            one(k % copies)
        ev[1].record()
        torch.cuda.synchronize()
        out[T] = (ev[0].elapsed_time(ev[1]) / 1e3 / reps, sum(decode_bytes(l, T, r) for l in layers),
                  sum(2 * T * l.N * l.K + 2 * T * r * (l.K + l.N) for l in layers))
    return out


def measure_merge(api, torch, layers, sets, r, s, reps=6):
    """W_m = RNE_bf16(W' + s (A B)^T) for the seven linears, one weight copy per pass
    (the 405 MB of outputs are written once per pass).  Returns (seconds, bytes) per layer set."""
    copies = len(sets)
    g = torch.Generator(device="cuda").manual_seed(7)
    a = [torch.randn((l.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
    b = [torch.randn((r, l.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
    outs = [torch.empty((l.N, l.K), dtype=torch.bfloat16, device="cuda") for l in layers]

    def one(c):
        for i in range(len(layers)):
            api.qlora_merge_lora(sets[c][i], a[i], b[i], s, out=outs[i])
    for c in range(copies):
        one(c)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for k in range(reps):
        one(k % copies)
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / 1e3 / reps, sum(merge_bytes(l, r) for l in layers)


def measure_sq(api, torch, bufs, T, r, s, ws, reps=5):
    """The single-quantization variant (codes + fp32 absmax per block) on the same
    seven linears: quantize, dequantize, forward and backward, each timed over
    `reps` passes with HIP events.  Returns {phase: (seconds per layer set, amount)}."""
    qs = [api.nf4_quantize(b["w"]) for b in bufs]
    ops = {
        "quantize_sq": ("hbm", lambda b, q: api.nf4_quantize(b["w"]),
                        lambda l: 2 * l.N * l.K + storage_bytes_sq(l.N * l.K)),
        "dequantize_sq": ("hbm", lambda b, q: api.nf4_dequantize(q, out=b["wd"]),
                          lambda l: 2 * l.N * l.K + storage_bytes_sq(l.N * l.K)),
        "forward_sq": ("mfma", lambda b, q: api.qlora_linear_fwd(b["x"], q, b["a"], b["b"], s, workspace=ws,
                                                                  out=b["y"]),
                       lambda l: phase_work(l, T, r)["forward"][1]),
        "backward_sq": ("mfma", lambda b, q: api.qlora_linear_bwd_input(b["dy"], q, b["a"], b["b"], s, x=b["x"],
                                                                         lora_grads=True, workspace=ws, dx=b["dx"],
                                                                         d_lora_a=b["da"], d_lora_b=b["db"]),
                        lambda l: phase_work(l, T, r)["backward"][1]),
    }
    out = {}
    for name, (kind, fn, work) in ops.items():
        for b, q in zip(bufs, qs):
            fn(b, q)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            for b, q in zip(bufs, qs):
                fn(b, q)
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = (kind, ev[0].elapsed_time(ev[1]) / 1e3 / reps, sum(work(b["lin"]) for b in bufs))
    return out


def measure_ablation(api, torch, synth, np, bufs, reps=5):
    """Data-type ablation on the seven 7B weights (N(0, 0.02)) and on a seeded
    outlier tensor (the 70B stream recipe, k-projection shape 1024 x 8192):
    relative rms error sqrt(sum (w' - w)^2 / sum w^2) of NF4 and INT4 absmax
    quantization (both with an fp32 absmax per 64 weights, so only the levels
    differ), and the INT4 quantize throughput.  The error sums are fp64
    reductions of the GPU-dequantized weights (measurement, not the path)."""
    def rel_err(w, wd):
        d = wd.double() - w.double()
        return (d * d).sum(), (w.double() * w.double()).sum()

    out = {}
    for name, ws in (("normal_7b", [b["w"] for b in bufs]),
                     ("outliers_70b_k", [torch.from_numpy(synth.outlier_weight_bf16(
                         synth.rng_for(5, 0, 1, synth.ROLE_W), (1024, 8192)).view(np.int16))
                         .view(torch.bfloat16).cuda()])):
        acc = {"nf4": [0.0, 0.0], "int4": [0.0, 0.0]}
        for w in ws:
            for dt, q, dq in (("nf4", api.nf4_quantize, api.nf4_dequantize),
                              ("int4", api.int4_quantize, api.int4_dequantize)):
                e, n = rel_err(w, dq(q(w)))
                acc[dt][0] += float(e)
                acc[dt][1] += float(n)
        out[name] = {dt: (a[0] / a[1]) ** 0.5 for dt, a in acc.items()}
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    qs = [api.int4_quantize(b["w"]) for b in bufs]
    ev[0].record()
    for _ in range(reps):
        for b, q in zip(bufs, qs):
            api.int4_quantize(b["w"])
    ev[1].record()
    torch.cuda.synchronize()
    secs = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    nbytes = sum(2 * b["lin"].N * b["lin"].K + storage_bytes_sq(b["lin"].N * b["lin"].K) for b in bufs)
    return out, secs, nbytes


def measure_f16(api, torch, bufs, T, r, s, ws, reps=5):
    """The fp16 compute type on the same seven linears (the step's tensors
    converted to fp16; the storage format is the bf16 path's): quantize from
    fp16 weights, dequantize to fp16, forward and backward with s X A reused,
    each over `reps` passes with HIP events.  Returns {phase: (kind, seconds, amount)}."""
    h = [{k: b[k].to(torch.float16) for k in ("w", "x", "dy", "a", "b")} for b in bufs]
    for hb, b in zip(h, bufs):
        hb["qw"] = api.nf4_quantize_dq(hb["w"])
        for k in ("wd", "y", "dx", "da", "db"):
            hb[k] = torch.empty_like(b[k], dtype=torch.float16)
    ops = {
        "quantize_f16": ("hbm", lambda hb: api.nf4_quantize_dq_into(hb["w"], hb["qw"]),
                         lambda l: phase_work(l, T, r)["quantize"][1]),
        "dequantize_f16": ("hbm", lambda hb: api.nf4_dequantize_dq(hb["qw"], out=hb["wd"]),
                           lambda l: phase_work(l, T, r)["dequantize"][1]),
        "forward_f16": ("mfma", lambda hb: api.qlora_linear_fwd(hb["x"], hb["qw"], hb["a"], hb["b"], s, workspace=ws,
                                                                 out=hb["y"]),
                        lambda l: phase_work(l, T, r)["forward"][1]),
        "backward_f16": ("mfma", lambda hb: (api.qlora_linear_fwd(hb["x"], hb["qw"], hb["a"], hb["b"], s, workspace=ws,
                                                                   out=hb["y"]),
                                             api.qlora_linear_bwd_input(hb["dy"], hb["qw"], hb["a"], hb["b"], s,
                                                                        x=hb["x"], lora_grads=True, workspace=ws,
                                                                        dx=hb["dx"], d_lora_a=hb["da"],
                                                                        d_lora_b=hb["db"], reuse_forward=True)),
                         lambda l: phase_work(l, T, r)["forward"][1] + phase_work(l, T, r)["backward"][1]),
    }
    out = {}
    for name, (kind, fn, work) in ops.items():
        for hb in h:
            fn(hb)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            for hb in h:
                fn(hb)
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = (kind, ev[0].elapsed_time(ev[1]) / 1e3 / reps, sum(work(b["lin"]) for b in bufs))
    return out


def measure_65b(api, torch, synth, reps=3):
    """The 65B-shaped layer (q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016;
    T = 2048, r = 64, s = 0.25): full-layer quantize and dequantize (one grouped
    launch each), the fused
    forward, and the backward input gradient dX = dY W' + s (dY B^T) A^T, each
    timed over `reps` passes of the seven linears with HIP events.  Inputs are
    drawn on the device (809.5 M weights).  Returns {phase: (kind, seconds, amount)}."""
    cfg = synth.LAYER_65B
    layers, T, r, s = cfg["layers"], cfg["T"], cfg["r"], cfg["scaling"]
    ws = torch.empty(max(api.qlora_workspace_bytes(T, l.K, l.N, r) for l in layers), dtype=torch.uint8,
                     device="cuda")
    bufs = []
    for ti, lin in enumerate(layers):
        g = synth.device_generator(cfg["config"], 0, ti, synth.ROLE_W)
        b = synth.device_layer_inputs(cfg["config"], 0, ti, lin, T, r, with_dy=True)
        b["lin"] = lin
        b["w"] = synth.device_normal_bf16(g, (lin.N, lin.K), 0.02)
        b["qw"] = api.nf4_quantize_dq(b["w"])
        b["wd"] = torch.empty((lin.N, lin.K), dtype=torch.bfloat16, device="cuda")
        b["y"] = torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda")
        b["dx"] = torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda")
        bufs.append(b)

    def bwd_flops(l):
        return 2 * T * l.N * l.K + 2 * T * l.N * r + 2 * T * r * l.K

    wl, ql, dl = [b["w"] for b in bufs], [b["qw"] for b in bufs], [b["wd"] for b in bufs]
    # quantize / dequantize: the whole layer in one grouped launch (run once per pass)
    ops = {
        "quantize": ("hbm", lambda b: b is bufs[0] and api.nf4_quantize_dq_grouped(wl, ql),
                     lambda l: phase_work(l, T, r)["quantize"][1]),
        "dequantize": ("hbm", lambda b: b is bufs[0] and api.nf4_dequantize_dq_grouped(ql, dl),
                       lambda l: phase_work(l, T, r)["dequantize"][1]),
        "forward": ("mfma", lambda b: api.qlora_linear_fwd(b["x"], b["qw"], b["a"], b["b"], s, workspace=ws,
                                                            out=b["y"]),
                    lambda l: phase_work(l, T, r)["forward"][1]),
        "backward_input": ("mfma", lambda b: api.qlora_linear_bwd_input(b["dy"], b["qw"], b["a"], b["b"], s,
                                                                         workspace=ws, dx=b["dx"]),
                           bwd_flops),
    }
    out = {}
    for name, (kind, fn, work) in ops.items():
        for b in bufs:
            fn(b)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            for b in bufs:
                fn(b)
        ev[1].record()
        torch.cuda.synchronize()
        out[name] = (kind, ev[0].elapsed_time(ev[1]) / 1e3 / reps, sum(work(b["lin"]) for b in bufs))
    del bufs, ws
    torch.cuda.empty_cache()
    return out


def measure_stream_70b(torch, synth, n_layers=80):
    """The 70B-shaped streaming workload: 80 layers of {q 8192x8192, k/v 1024x8192,
    o 8192x8192, gate/up 28672x8192, down 8192x28672}, each drawn on the device
    as N(0, 0.02) with 0.1% 0.1 * t3 outliers, quantized (NF4 + double
    quantization) and dequantized tensor by tensor with one layer resident.
    Returns (kernel seconds, algorithmic bytes moved, packed bytes, parameters)."""
    from qlora_linear_layers_amd.stream import LayerStream
    cfg = synth.STREAM_70B
    layers = cfg["layers"]
    st = LayerStream([(l.N, l.K) for l in layers])
    res = st.run(lambda l: synth.device_layer_weights(cfg["config"], l, layers, outliers=True), n_layers)
    params = n_layers * sum(l.N * l.K for l in layers)
    moved = n_layers * sum(2 * (2 * l.N * l.K + storage_bytes(l.N * l.K)) for l in layers)
    del st
    torch.cuda.empty_cache()
    return res["seconds"], moved, res["packed_bytes"], params


def storage_bytes_sq(numel):
    """Codes + one fp32 absmax per 64 weights."""
    return numel // 2 + 4 * (numel // 64)


def cpu_baseline(layers, T, r, s, t_sample):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from qlora_linear_layers_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    roof = 0.0
    t0 = time.perf_counter()
    for li, lin in enumerate(layers):
        d = synth.layer_inputs(3, 0, li, lin, T, r, with_dy=True)
        x, dy = d["x"][:t_sample], d["dy"][:t_sample]
        rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
        wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(lin.N, lin.K)
        oracle.linear_fwd(x, wd, d["a"], d["b"], s)
        oracle.linear_bwd(dy, x, wd, d["a"], d["b"], s)
        for name, (kind, amt) in phase_work(lin, t_sample, r).items():
            roof += roofline_seconds(kind, amt)
    dt = time.perf_counter() - t0
    # generation of the synthetic inputs is inside dt; it is small next to the oracle
    return {"value": 100.0 * roof / dt, "unit": "% of MI355X roofline", "cores": int(threads), "kind": "oracle",
            "sample": f"all 7 linears: full quantize + dequantize, forward and backward on {t_sample} of {T} tokens",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


def calibration_copy(torch):
    """Three device copies of COPY_BYTES: counter runs scale their byte counts by
    what the same counters read for this copy of known size."""
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    for _ in range(3):
        c.copy_(a)
    torch.cuda.synchronize()


def only_component(name, api, torch, synth, layers, r, s):
    """One component alone, on weights drawn on the device (for kernel traces and counter runs)."""
    if name.startswith("decode"):
        g = torch.Generator(device="cuda").manual_seed(1)
        qws = [api.nf4_quantize_dq(torch.randn((l.N, l.K), generator=g, device="cuda").mul_(0.02)
                                   .to(torch.bfloat16)) for l in layers]
        mode = {"decode": "staged", "decode_single": "single", "decode_all7": "all"}[name]
        res = measure_decode(api, torch, layers, weight_copies(api, qws), r, s, mode=mode)
        return {f"T{Td}": {"GB/s": round(nb / secs / 1e9, 1), "us_per_layer_set": round(1e6 * secs, 2)}
                for Td, (secs, nb) in res.items()}
    if name == "layer_65b":
        out = {}
        for k, (kind, secs, amt) in measure_65b(api, torch, synth).items():
            out[k] = ({"GB/s": round(amt / secs / 1e9, 1)} if kind == "hbm" else
                      {"TFLOP/s": round(amt / secs / 1e12, 1)})
        return out
    secs, moved, packed, params = measure_stream_70b(torch, synth)
    return {"GB/s": round(moved / secs / 1e9, 1), "ms": round(1e3 * secs, 3), "packed_bytes": packed,
            "params": params}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the step and the roofline kernel (for a kernel trace of the step alone)")
    ap.add_argument("--cpu-tokens", type=int, default=256)
    ap.add_argument("--only", choices=("decode", "decode_single", "decode_all7", "layer_65b", "stream_70b"),
                    help="run one component alone (no step, roofline loop or CPU baseline), e.g. for a kernel trace")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the calibration copy and the k_fwd launches (for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is single-GPU by design); --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from qlora_linear_layers_amd import api, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    api.lib()
    cfg = synth.TRAIN_7B
    layers, T, r, s = cfg["layers"], cfg["T"], cfg["r"], cfg["scaling"]

    if args.only:
        calibration_copy(torch)
        print(json.dumps({"component": args.only, **only_component(args.only, api, torch, synth, layers, r, s)}),
              flush=True)
        return

    def dev(bits, shape):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).reshape(shape).cuda()

    bufs = []
    ws_bytes = max(api.qlora_workspace_bytes(T, l.K, l.N, r) for l in layers)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for li, lin in enumerate(layers):
        d = synth.layer_inputs(3, 0, li, lin, T, r, with_dy=True)
        b = dict(lin=lin, w=dev(d["w"], (lin.N, lin.K)), x=dev(d["x"], (T, lin.K)), dy=dev(d["dy"], (T, lin.N)),
                 a=dev(d["a"], (lin.K, r)), b=dev(d["b"], (r, lin.N)))
        b["qw"] = api.nf4_quantize_dq(b["w"])
        b["wd"] = torch.empty((lin.N, lin.K), dtype=torch.bfloat16, device="cuda")
        b["y"] = torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda")
        b["dx"] = torch.empty((T, lin.K), dtype=torch.bfloat16, device="cuda")
        b["da"] = torch.empty((lin.K, r), dtype=torch.bfloat16, device="cuda")
        b["db"] = torch.empty((r, lin.N), dtype=torch.bfloat16, device="cuda")
        bufs.append(b)
    torch.cuda.synchronize()

    if args.roofline_only:
        calibration_copy(torch)
        flops, secs = measure_roofline_kernel(api, torch, layers, bufs, args.steps)
        print(json.dumps({"roofline_kernel": "k_fwd", "tflops": flops / secs / 1e12, "us_per_launch": secs * 1e6,
                          "copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                          "gemm_source_sha256_16": source_hash()}), flush=True)
        return

    phases = ("quantize", "dequantize", "forward", "backward")
    stream = torch.cuda.current_stream()

    wlist, qlist, dlist = [b["w"] for b in bufs], [b["qw"] for b in bufs], [b["wd"] for b in bufs]

    def step(ev=None):
        # ev: [quantize start, quantize end = dequantize start, dequantize end, then per linear
        # forward end and backward end]
        if ev: ev[0].record(stream)
        api.nf4_quantize_dq_grouped(wlist, qlist)          # the seven weights in one launch
        if ev: ev[1].record(stream)
        api.nf4_dequantize_dq_grouped(qlist, dlist)
        if ev: ev[2].record(stream)
        for li, b in enumerate(bufs):
            api.qlora_linear_fwd(b["x"], b["qw"], b["a"], b["b"], s, workspace=ws, out=b["y"])
            if ev: ev[3 + 2 * li].record(stream)
            api.qlora_linear_bwd_input(b["dy"], b["qw"], b["a"], b["b"], s, x=b["x"], lora_grads=True,
                                       workspace=ws, dx=b["dx"], d_lora_a=b["da"], d_lora_b=b["db"],
                                       reuse_forward=True)
            if ev: ev[4 + 2 * li].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nev = 3 + 2 * len(bufs)
    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(all_events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # per-phase average durations (ms) from the events: quantize and dequantize of the
    # seven weights (one launch each), forward and backward per linear
    dur = {p: 0.0 for p in phases}
    for ev in all_events:
        dur["quantize"] += ev[0].elapsed_time(ev[1]) / args.steps
        dur["dequantize"] += ev[1].elapsed_time(ev[2]) / args.steps
        for li in range(len(bufs)):
            dur["forward"] += ev[2 + 2 * li].elapsed_time(ev[3 + 2 * li]) / args.steps
            dur["backward"] += ev[3 + 2 * li].elapsed_time(ev[4 + 2 * li]) / args.steps

    comp = {}
    roof_step = 0.0
    for p in phases:
        kind = None
        amt = 0
        for b in bufs:
            kind, a = phase_work(b["lin"], T, r)[p]
            amt += a
        secs = dur[p] / 1e3
        rs = roofline_seconds(kind, amt)
        roof_step += rs
        if kind == "hbm":
            comp[p] = {"GB/s": round(amt / secs / 1e9, 1), "frac_of_hbm_peak": round(rs / secs, 4),
                       "ms": round(1e3 * secs, 4)}
        else:
            comp[p] = {"TFLOP/s": round(amt / secs / 1e12, 1), "frac_of_mfma_peak": round(rs / secs, 4),
                       "ms": round(1e3 * secs, 4)}

    # roofline of the dominant kernel: k_fwd, timed alone (r = 0 forward = one launch)
    rf_flops, rf_secs = measure_roofline_kernel(api, torch, layers, bufs, max(args.steps // 2, 3))
    achieved = rf_flops / rf_secs / 1e12
    traffic = stored_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(achieved / 2500.0, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "k_fwd: fused NF4 double-dequant + MFMA bf16 GEMM, 7B layer shapes at T=4096 "
                          "(per-launch average over the 7 linears)",
                "us_per_launch": round(1e6 * rf_secs, 2),
                "flops_per_launch": rf_flops}

    out = {
        "metric": "QLoRA linear fwd TFLOP/s + NF4 quant/dequant GB/s, as % of MI355X roofline",
        "value": round(100.0 * roof_step / (wall / args.steps), 3),
        "unit": "% of MI355X roofline",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LLaMA-7B-shaped layer, 7 linears (q/k/v/o 4096x4096, gate/up 11008x4096, "
                               "down 4096x11008), T=4096 tokens, LoRA r=64 alpha=16; step = quantize + dequantize (grouped) "
                               "+ forward + backward (dX, dA, dB; s X A kept from the forward) of every linear",
                   "global_batch": 8, "seq_len": 512, "parallelism": "none (1 GPU)"},
        "components": comp,
        "roofline": roofline,
    }
    if not args.no_extras:      # decode, single quantization, fp16, ablation, merge (outside the step)
        sets = weight_copies(api, [b["qw"] for b in bufs])
        notes = {"single": "one launch pair per linear",
                 "staged": "grouped launches per dependency stage: q/k/v, o, gate/up, down",
                 "all": "all 7 linears in one grouped launch pair (independent inputs)"}
        for mode, prefix in (("staged", "decode"), ("single", "decode_single"), ("all", "decode_all7")):
            for Td, (secs, nbytes) in measure_decode(api, torch, layers, sets, r, s, mode=mode).items():
                comp[f"{prefix}_T{Td}"] = {
                    "GB/s": round(nbytes / secs / 1e9, 1), "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                    "us_per_layer_set": round(1e6 * secs, 2),
                    "note": "7 linears, fused dequant + small-M MFMA (16x16x32) incl. LoRA; " + notes[mode]
                            + "; weights rotated over 6 copies"}
        for name, (kind, secs, amt) in measure_sq(api, torch, bufs, T, r, s, ws).items():
            if kind == "hbm":
                comp[name] = {"GB/s": round(amt / secs / 1e9, 1), "frac_of_hbm_peak": round(amt / secs / HBM_PEAK, 4),
                              "ms": round(1e3 * secs, 4), "note": "single quantization (fp32 absmax per 64 weights)"}
            else:
                comp[name] = {"TFLOP/s": round(amt / secs / 1e12, 1),
                              "frac_of_mfma_peak": round(amt / secs / MFMA_BF16_PEAK, 4), "ms": round(1e3 * secs, 4),
                              "note": "single quantization (fp32 absmax per 64 weights)"}
        for name, (kind, secs, amt) in measure_f16(api, torch, bufs, T, r, s, ws).items():
            note = "fp16 compute type" + (" (forward + backward pass, s X A reused)" if name == "backward_f16" else "")
            if kind == "hbm":
                comp[name] = {"GB/s": round(amt / secs / 1e9, 1), "frac_of_hbm_peak": round(amt / secs / HBM_PEAK, 4),
                              "ms": round(1e3 * secs, 4), "note": note}
            else:
                comp[name] = {"TFLOP/s": round(amt / secs / 1e12, 1),
                              "frac_of_mfma_peak": round(amt / secs / MFMA_BF16_PEAK, 4), "ms": round(1e3 * secs, 4),
                              "note": note}
        abl, secs, nbytes = measure_ablation(api, torch, synth, np, bufs)
        comp["int4_ablation"] = {
            "relative_rms_error": {k: {dt: round(e, 5) for dt, e in v.items()} for k, v in abl.items()},
            "int4_quantize_GB/s": round(nbytes / secs / 1e9, 1),
            "note": "NF4 vs INT4 absmax levels, fp32 absmax per 64 weights for both"}
        secs, nbytes = measure_merge(api, torch, layers, sets, r, s)
        comp["merge"] = {"GB/s": round(nbytes / secs / 1e9, 1), "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                         "us_per_layer_set": round(1e6 * secs, 2),
                         "note": "7 linears, W_m = RNE_bf16(W' + s (A B)^T), r=64; weights rotated over 6 copies"}
        for Tp, (secs, nbytes, flops) in measure_prefill(api, torch, layers, sets, r, s).items():
            comp[f"prefill_T{Tp}"] = {"TFLOP/s": round(flops / secs / 1e12, 1), "GB/s": round(nbytes / secs / 1e9, 1),
                                      "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                                      "us_per_layer_set": round(1e6 * secs, 2),
                                      "note": "7 linears, r=64, forward at a small-prefill T: 16-token windows as one "
                                              "grouped decode launch pair; weights rotated over 6 copies"}
        del sets
        for name, (kind, secs, amt) in measure_65b(api, torch, synth).items():
            key = name + "_65b"
            if kind == "hbm":
                comp[key] = {"GB/s": round(amt / secs / 1e9, 1), "frac_of_hbm_peak": round(amt / secs / HBM_PEAK, 4),
                             "ms": round(1e3 * secs, 4)}
            else:
                comp[key] = {"TFLOP/s": round(amt / secs / 1e12, 1),
                             "frac_of_mfma_peak": round(amt / secs / MFMA_BF16_PEAK, 4), "ms": round(1e3 * secs, 4)}
            comp[key]["note"] = ("65B-shaped layer (q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016), "
                                 "T=2048, r=64; 7 linears per pass (quantize / dequantize: one grouped launch)")
        secs, moved, packed, params = measure_stream_70b(torch, synth)
        closed = params * (4 + 8 / 64 + 32 / 16384) / 8
        comp["stream_70b"] = {"GB/s": round(moved / secs / 1e9, 1), "frac_of_hbm_peak": round(moved / secs / HBM_PEAK, 4),
                              "ms": round(1e3 * secs, 3), "params": params, "packed_bytes": packed,
                              "closed_form_bytes": int(closed), "bits_per_param": round(8 * packed / params, 9),
                              "note": "80 layers x 7 tensors (70B shapes, 0.1% t3 outliers), grouped quantize_dq then "
                                      "grouped dequantize per layer, one layer resident; kernel time only"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, T, r, s, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
