#!/usr/bin/env python
"""Benchmark of the QLoRA frozen-base linear layer hot path on one MI355X.

Headline workload (one "step"): the seven linears of a LLaMA-65B-shaped
transformer layer (q/k/v/o 8192x8192, gate/up 22016x8192, down 8192x22016;
809.5 M weights) at T = 2048 tokens, LoRA rank 64, s = alpha / r = 0.25.  A
step runs NF4 + double quantization of the seven bf16 weights (one grouped
launch), their double dequantization back to bf16 (one grouped launch), and
for each linear the fused forward Y = X W'^T + s (X A) B and the backward
input gradient dX = dY W' + s (dY B^T) A^T.  Inputs are seeded synthetic
tensors drawn on the device (W ~ N(0, 0.02), X, dY ~ N(0, 1), A, B ~ N(0,
0.01)), resident in HBM before timing starts.

Output: one JSON line.  `value` is the step's attainment of the MI355X
roofline: the sum over its phases of their roofline time (algorithmic bytes at
8 TB/s for quantize / dequantize, algorithmic flops at 2.5 PFLOP/s bf16 dense
for the GEMM phases) divided by the measured step time.  Per-phase durations
come from HIP events recorded on the stream the kernels run on.  `roofline`
is the fused NF4-dequant MFMA GEMM (k_fwd) at the same shapes, timed alone.
`components` carries the other workloads measured on the same device: the
single 4096 x 4096 layer (T = 16, r = 16), the decode forward of the 7B layer
set (T = 1 / 4 / 8), the 7B training step (T = 4096, forward + backward with
the LoRA gradients), the 70B-shaped streaming quantization, the LoRA merge,
the single-quantization and fp16 variants, the NF4-vs-INT4 ablation, and the
calibration legs (a 128-bit streaming copy, an MFMA-only loop, and torch.matmul
on the dequantized weight as the unfused context).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, published
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16, published
# k_fwd's source: the kernel file and the headers it includes
GEMM_SOURCES = [os.path.join(ROOT, "qlora_linear_layers_amd", "csrc", f)
                for f in ("gemm.hip", "common.hpp", "grad.hpp", "plan.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_fwd_llama65b_T2048_traffic.txt")
COPY_BYTES = 256 << 20     # calibration copy for the HBM byte counters


def source_hash():
    """sha256[:16] over k_fwd's source files in order: the stored HBM traffic is used
    only while it was measured on exactly this code."""
    import hashlib
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


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


def storage_bytes(numel):
    return numel // 2 + numel // 64 + 4 * (-(-numel // 16384))


def phase_work(lin, T, r):
    """Algorithmic (kind, amount, bytes) of each phase of one linear: bytes for the
    HBM phases, flops for the GEMM phases (with the algorithmic bytes they move,
    for the arithmetic intensity).  The backward with the LoRA gradients takes
    s X A from the forward (saved activation), so it has no X A recompute."""
    N, K = lin.N, lin.K
    nk = N * K
    st = storage_bytes(nk)
    ad = 2 * r * (K + N)
    return {
        "quantize": ("hbm", 2 * nk + st, 2 * nk + st),
        "dequantize": ("hbm", st + 2 * nk, st + 2 * nk),
        "forward": ("mfma", 2 * T * N * K + 2 * T * K * r + 2 * T * r * N, st + 2 * T * K + 2 * T * N + ad),
        # dX = dY W' + (s dY B^T) A^T
        "backward_input": ("mfma", 2 * T * N * K + 2 * T * N * r + 2 * T * r * K, st + 2 * T * N + 2 * T * K + ad),
        # dX as above, dA = X^T G and dB = P^T dY (P = s X A saved by the forward)
        "backward": ("mfma", 2 * T * N * K + 2 * T * N * r + 2 * T * r * K + 2 * T * K * r + 2 * T * r * N,
                     st + 2 * T * N + 4 * T * K + 2 * ad),
    }


def roofline_seconds(kind, amount):
    return amount / (HBM_PEAK if kind == "hbm" else MFMA_BF16_PEAK)


def attainable(kind, amount, nbytes):
    """min(P_MFMA, BW x AI_alg) for a GEMM phase (flop/s), BW for an HBM phase (B/s)."""
    if kind == "hbm":
        return HBM_PEAK
    return min(MFMA_BF16_PEAK, HBM_PEAK * amount / nbytes)


def phase_entry(kind, amount, nbytes, secs, calib=None):
    """One component entry: rate, fraction of the published peak, of the attainable
    roofline and (when measured) of the device's measured peak."""
    rate = amount / secs
    e = ({"GB/s": round(rate / 1e9, 1), "frac_of_hbm_peak": round(rate / HBM_PEAK, 4)} if kind == "hbm" else
         {"TFLOP/s": round(rate / 1e12, 1), "frac_of_mfma_peak": round(rate / MFMA_BF16_PEAK, 4)})
    if nbytes:
        e["frac_of_attainable"] = round(rate / attainable(kind, amount, nbytes), 4)
    if calib:
        meas = calib.get("copy_B/s") if kind == "hbm" else calib.get("mfma_flop/s")
        if meas:
            e["frac_of_measured_peak"] = round(rate / meas, 4)
    e["ms"] = round(1e3 * secs, 4)
    return e


def measure_roofline_kernel(api, torch, bufs, reps):
    """k_fwd alone: the forward with r = 0 is exactly one launch of the fused
    NF4-dequant MFMA GEMM.  HIP events on the launch stream around every launch.
    Returns (flops per launch, seconds per launch)."""
    ys = [torch.empty((b["x"].shape[0], b["lin"].N), dtype=torch.bfloat16, device="cuda") for b in bufs]
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")          # r = 0 needs none
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps * len(bufs))]
    for i, b in enumerate(bufs):
        api.qlora_linear_fwd(b["x"], b["qw"], workspace=ws, out=ys[i])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for k in range(reps):
        for i, b in enumerate(bufs):
            e = ev[k * len(bufs) + i]
            e[0].record(stream)
            api.qlora_linear_fwd(b["x"], b["qw"], workspace=ws, out=ys[i])
            e[1].record(stream)
    torch.cuda.synchronize()
    secs = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3 / len(ev)
    flops = sum(2 * b["x"].shape[0] * b["lin"].N * b["lin"].K for b in bufs) / len(bufs)
    return flops, secs


def layer_65b_buffers(api, torch, synth):
    """The 65B-shaped layer's tensors, drawn on the device (809.5 M weights)."""
    cfg = synth.LAYER_65B
    layers, T, r = cfg["layers"], cfg["T"], cfg["r"]
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
    torch.cuda.synchronize()
    return bufs


def run_step(torch, step, nev, steps, warmup):
    """`warmup` untimed steps, then `steps` timed ones with nothing but the step's
    own launches on the stream, then `steps` more with an event after every phase
    for the per-phase breakdown (each event record costs the stream a few
    microseconds, so the timed steps carry none); returns (wall seconds of the
    timed region, per-step event lists of the instrumented steps)."""
    for _ in range(warmup):
        step()
    all_events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for k in range(steps):
        step(all_events[k])
    torch.cuda.synchronize()
    return wall, all_events


def layer_step(api, bufs, T, r, s, ws, stream, with_grads, fused=False):
    """One step over the seven linears: grouped quantize, grouped dequantize, then
    per linear the forward and the backward (input gradient only, or with the LoRA
    gradients and s X A reused from the forward).  Event layout: [quantize start,
    quantize end = dequantize start, dequantize end, per linear forward end and
    backward end]."""
    wl, ql, dl = [b["w"] for b in bufs], [b["qw"] for b in bufs], [b["wd"] for b in bufs]

    def step(ev=None):
        if ev: ev[0].record(stream)
        api.nf4_quantize_dq_grouped(wl, ql)
        if ev: ev[1].record(stream)
        api.nf4_dequantize_dq_grouped(ql, dl)
        if ev: ev[2].record(stream)
        for li, b in enumerate(bufs):
            api.qlora_linear_fwd(b["x"], b["qw"], b["a"], b["b"], s, workspace=ws, out=b["y"])
            if ev: ev[3 + 2 * li].record(stream)
            if with_grads:
                api.qlora_linear_bwd_input(b["dy"], b["qw"], b["a"], b["b"], s, x=b["x"], lora_grads=True,
                                           workspace=ws, dx=b["dx"], d_lora_a=b["da"], d_lora_b=b["db"],
                                           reuse_forward=True, fused_grads=fused)
            else:
                api.qlora_linear_bwd_input(b["dy"], b["qw"], b["a"], b["b"], s, workspace=ws, dx=b["dx"])
            if ev: ev[4 + 2 * li].record(stream)
    return step, 3 + 2 * len(bufs)


def step_phases(bufs, all_events, steps, T, r, bwd_name, calib=None):
    """Per-phase durations from the step events, their components entries and the
    step's total roofline time."""
    dur = {"quantize": 0.0, "dequantize": 0.0, "forward": 0.0, bwd_name: 0.0}
    for ev in all_events:
        dur["quantize"] += ev[0].elapsed_time(ev[1]) / steps
        dur["dequantize"] += ev[1].elapsed_time(ev[2]) / steps
        for li in range(len(bufs)):
            dur["forward"] += ev[2 + 2 * li].elapsed_time(ev[3 + 2 * li]) / steps
            dur[bwd_name] += ev[3 + 2 * li].elapsed_time(ev[4 + 2 * li]) / steps
    comp, roof = {}, 0.0
    for p, ms in dur.items():
        kind, amt, nb = None, 0, 0
        for b in bufs:
            kind, a, n = phase_work(b["lin"], T, r)[p]
            amt += a
            nb += n
        roof += roofline_seconds(kind, amt)
        comp[p] = phase_entry(kind, amt, nb, ms / 1e3, calib)
    return comp, roof


def measure_train_7b(api, torch, synth, np, steps, calib, fused=False):
    """The 7B training-shaped step (T = 4096, r = 64, alpha = 16): grouped quantize and
    dequantize, then forward and backward with dX, dA, dB (s X A kept from the forward)
    for each of the seven linears; with `fused`, the backward forms dA and dB inside
    the dX kernel (QLORA_BWD_FUSED_GRADS).  Inputs from the host generators (the
    oracle's bytes).  Returns (components of the phases, ms per step, step attainment)."""
    cfg = synth.TRAIN_7B
    layers, T, r, s = cfg["layers"], cfg["T"], cfg["r"], cfg["scaling"]

    def dev(bits, shape):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).reshape(shape).cuda()

    flags = api.REUSE_FORWARD | (api.FUSED_GRADS if fused else 0)
    ws = torch.empty(max(max(api.qlora_workspace_bytes(T, l.K, l.N, r), api.qlora_workspace_bytes_bwd(
        T, l.K, l.N, r, flags)) for l in layers), dtype=torch.uint8, device="cuda")
    bufs = []
    for li, lin in enumerate(layers):
        d = synth.layer_inputs(cfg["config"], 0, li, lin, T, r, with_dy=True)
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
    step, nev = layer_step(api, bufs, T, r, s, ws, torch.cuda.current_stream(), with_grads=True, fused=fused)
    wall, evs = run_step(torch, step, nev, steps, 3)
    comp, roof = step_phases(bufs, evs, steps, T, r, "backward", calib)
    return comp, 1e3 * wall / steps, roof / (wall / steps), bufs, ws


def measure_single_layer(api, torch, synth, launches=100, rotate_bytes=512 << 20):
    """The single 4096 x 4096 layer (T = 16, r = 16, s = 1): quantize, dequantize and
    forward, each as `launches` back-to-back launches over input/output sets that
    together exceed `rotate_bytes` (so the 256 MB memory-side cache cannot serve
    repeats), behind a GPU spin so that the events see device time only.
    Returns {phase: (kind, seconds per launch, amount, algorithmic bytes)}."""
    cfg = synth.SINGLE_LAYER
    lin, T, r, s = cfg["layers"][0], cfg["T"], cfg["r"], cfg["scaling"]
    g = synth.device_generator(cfg["config"], 0, 0, synth.ROLE_W)
    w = synth.device_normal_bf16(g, (lin.N, lin.K), 0.02)
    inp = synth.device_layer_inputs(cfg["config"], 0, 0, lin, T, r)
    work = phase_work(lin, T, r)
    qset = -(-rotate_bytes // work["quantize"][2])
    fset = -(-rotate_bytes // work["forward"][2])
    ws_in = [w.clone() for _ in range(qset)]
    q_out = [api.nf4_quantize_dq(w) for _ in range(max(qset, fset))]
    d_out = [torch.empty_like(w) for _ in range(qset)]
    ys = torch.empty((T, lin.N), dtype=torch.bfloat16, device="cuda")
    wsp = torch.empty(max(api.qlora_workspace_bytes(T, lin.K, lin.N, r), 256), dtype=torch.uint8, device="cuda")
    ops = {
        "quantize": (qset, lambda i: api.nf4_quantize_dq_into(ws_in[i], q_out[i])),
        "dequantize": (qset, lambda i: api.nf4_dequantize_dq(q_out[i], out=d_out[i])),
        "forward": (fset, lambda i: api.qlora_linear_fwd(inp["x"], q_out[i], inp["a"], inp["b"], s, workspace=wsp,
                                                        out=ys)),
    }
    out = {}
    for name, (nset, fn) in ops.items():
        for i in range(nset):
            fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda._sleep(50_000_000)
        ev[0].record()
        for k in range(launches):
            fn(k % nset)
        ev[1].record()
        torch.cuda.synchronize()
        kind, amt, nb = work[name]
        out[name] = (kind, ev[0].elapsed_time(ev[1]) / 1e3 / launches, amt, nb, nset)
    return out


def measure_calibration(torch, calib, bufs=None, reps=10):
    """The device's achievable peaks: the 128-bit streaming copy of 1 GiB (read +
    write bytes over time), the MFMA-only loop (4 rounds of one 4-wave workgroup per
    CU), and, as the unfused context, torch.matmul (hipBLASLt) of X by the
    dequantized bf16 W' on the 65B layer's shapes."""
    res = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    calib.stream_copy(src, dst)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        calib.stream_copy(src, dst)
    ev[1].record()
    torch.cuda.synchronize()
    secs = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    res["copy_B/s"] = 2 * n / secs
    del src, dst
    seed = torch.randint(-2 ** 30, 2 ** 30, (128,), dtype=torch.int32, device="cuda") & 0x3F803F80
    wgs, iters = 256 * 4, 4096
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    flops = calib.mfma_loop(seed, out, wgs, iters)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(3):
        calib.mfma_loop(seed, out, wgs, iters)
    ev[1].record()
    torch.cuda.synchronize()
    res["mfma_flop/s"] = flops / (ev[0].elapsed_time(ev[1]) / 1e3 / 3)
    if bufs is not None:
        flops = 0
        for b in bufs:
            torch.matmul(b["x"], b["wd"].t())
            flops += 2 * b["x"].shape[0] * b["lin"].N * b["lin"].K
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(3):
            for b in bufs:
                torch.matmul(b["x"], b["wd"].t())
        ev[1].record()
        torch.cuda.synchronize()
        res["torch_matmul_flop/s"] = flops / (ev[0].elapsed_time(ev[1]) / 1e3 / 3)
    return res


def calibration_copy(torch, calib):
    """Three streaming copies of COPY_BYTES: counter runs scale their byte counts by
    what the same counters read for this copy of known size."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    c = torch.empty_like(a)
    for _ in range(3):
        calib.stream_copy(a, c)
    torch.cuda.synchronize()


def cpu_baseline(layers, T, r, s, row_frac=8, t_sample=32):
    """The oracle, as it stands, on a bounded sample of the headline workload: NF4 +
    double quantization and double dequantization of the first 1/row_frac of the
    rows of each of the seven 65B-shaped weights, and the forward and backward-input
    GEMMs of those rows on t_sample of the T tokens (inputs from the host generators
    in the same distributions).  Scaled to the same unit as `value`."""
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
        sub = synth.Linear(lin.name, lin.N // row_frac, lin.K)
        d = synth.layer_inputs(4, 0, li, sub, t_sample, r, with_dy=True)
        rc, rf, rs = oracle.quantize_nf4_dq(d["w"])
        wd = oracle.dequantize_nf4_dq(rc, rf, rs).reshape(sub.N, sub.K)
        oracle.linear_fwd(d["x"], wd, d["a"], d["b"], s)
        oracle.linear_bwd(d["dy"], None, wd, d["a"], d["b"], s)
        for p in ("quantize", "dequantize", "forward", "backward_input"):
            kind, amt, _ = phase_work(sub, t_sample, r)[p]
            roof += roofline_seconds(kind, amt)
    dt = time.perf_counter() - t0
    return {"value": 100.0 * roof / dt, "unit": "% of MI355X roofline", "cores": int(threads), "kind": "oracle",
            "sample": f"65B layer: quantize + dequantize of 1/{row_frac} of the rows of each of the 7 weights, "
                      f"forward and backward-input of those rows on {t_sample} of {T} tokens",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count()}


def decode_bytes(lin, T, r):
    """Algorithmic bytes of one decode-size forward: the packed weight, X, Y and the adapters."""
    return storage_bytes(lin.N * lin.K) + 2 * T * lin.K + 2 * T * lin.N + 2 * r * (lin.K + lin.N)


def weight_copies(api, qws, copies=6):
    """`copies` copies of the quantized weights of the seven linears (about 100 MB
    each), rotated so that the 256 MB last-level cache cannot serve repeats."""
    return [[api.NF4Weight(q.codes.clone(), q.absmax_fp8.clone(), q.superscale.clone(), q.N, q.K) for q in qws]
            for _ in range(copies)]



DECODE_STAGES = ((0, 1, 2), (3,), (4, 5), (6,))    # q/k/v, o, gate/up, down: what a decode step can group


def measure_decode(api, torch, layers, sets, r, s, tokens=(1, 4, 8), reps=10, mode="single", product=None):
    """Decode-size forward over the seven linears, one weight copy per pass.
    mode "single": one qlora_linear_fwd per linear; "staged": one grouped call
    per dependency stage (q/k/v, o, gate/up, down); "all": one grouped call for
    all seven.  `product` ("mfma", "valu" or None for the library's choice)
    applies to the grouped modes.  A GPU spin ahead of the timed region lets the
    host enqueue every pass first, so the events see device time only.
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
                                                 workspace=ws, product=product)
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



def measure_forward_midt(api, torch, layers, sets, r, s, tokens=(256, 512, 1024, 2048), reps=6):
    """Forward of the seven linears at token counts whose 256 x 256 tiles fill part of
    the chip (the split-k forward), one weight copy per pass.
    Returns {T: (seconds per layer set, flops per layer set)}."""
    copies = len(sets)
    out = {}
    for T in tokens:
        g = torch.Generator(device="cuda").manual_seed(200 + T)
        xs = [torch.randn((T, l.K), generator=g, device="cuda").to(torch.bfloat16) for l in layers]
        a = [torch.randn((l.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        b = [torch.randn((r, l.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        ws = torch.empty(max(api.qlora_workspace_bytes(T, l.K, l.N, r) for l in layers), dtype=torch.uint8,
                         device="cuda")
        ys = [torch.empty((T, l.N), dtype=torch.bfloat16, device="cuda") for l in layers]

        def one(c):
            for i in range(len(layers)):
                api.qlora_linear_fwd(xs[i], sets[c][i], a[i], b[i], s, workspace=ws, out=ys[i])
        for c in range(copies):
            one(c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for k in range(reps):
            one(k % copies)
        ev[1].record()
        torch.cuda.synchronize()
        secs = ev[0].elapsed_time(ev[1]) / 1e3 / reps
        out[T] = (secs, sum(2 * T * l.N * l.K + 4 * T * r * (l.K + l.N) for l in layers))
        del xs, a, b, ws, ys
    return out


def measure_step_midt(api, torch, layers, sets, r, s, tokens=(256, 512, 1024, 2048), reps=4):
    """Training step of the seven linears (forward, then dX, dA and dB with the
    forward's s X A reused) at token counts whose tiles fill part of the chip
    (split-k forward and dX), one weight copy per pass.
    Returns {T: (seconds per layer set, flops per layer set)}."""
    copies = len(sets)
    out = {}
    for T in tokens:
        g = torch.Generator(device="cuda").manual_seed(300 + T)
        xs = [torch.randn((T, l.K), generator=g, device="cuda").to(torch.bfloat16) for l in layers]
        dys = [torch.randn((T, l.N), generator=g, device="cuda").to(torch.bfloat16) for l in layers]
        a = [torch.randn((l.K, r), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        b = [torch.randn((r, l.N), generator=g, device="cuda").mul_(0.01).to(torch.bfloat16) for l in layers]
        ws = [torch.empty(api.qlora_workspace_bytes_bwd(T, l.K, l.N, r, api.REUSE_FORWARD), dtype=torch.uint8,
                          device="cuda") for l in layers]
        ys = [torch.empty((T, l.N), dtype=torch.bfloat16, device="cuda") for l in layers]
        dxs = [torch.empty((T, l.K), dtype=torch.bfloat16, device="cuda") for l in layers]
        das = [torch.empty((l.K, r), dtype=torch.bfloat16, device="cuda") for l in layers]
        dbs = [torch.empty((r, l.N), dtype=torch.bfloat16, device="cuda") for l in layers]

        def one(c):
            for i in range(len(layers)):
                api.qlora_linear_fwd(xs[i], sets[c][i], a[i], b[i], s, workspace=ws[i], out=ys[i])
            for i in reversed(range(len(layers))):
                api.qlora_linear_bwd_input(dys[i], sets[c][i], a[i], b[i], s, x=xs[i], lora_grads=True,
                                           workspace=ws[i], reuse_forward=True, dx=dxs[i], d_lora_a=das[i],
                                           d_lora_b=dbs[i])
        for c in range(copies):
            one(c)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for k in range(reps):
            one(k % copies)
        ev[1].record()
        torch.cuda.synchronize()
        secs = ev[0].elapsed_time(ev[1]) / 1e3 / reps
        out[T] = (secs, sum(3 * 2 * T * l.N * l.K + 3 * 4 * T * r * (l.K + l.N) for l in layers))
        del xs, dys, a, b, ws, ys, dxs, das, dbs
    return out


def measure_prefill(api, torch, layers, sets, r, s, tokens=(32, 64), reps=6):
    """Small-prefill forward (16 < T <= 96 runs 16-token windows as one grouped
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


def only_component(name, api, torch, synth, calib, args):
    """One component alone (for kernel traces and counter runs)."""
    layers7, r, s = synth.TRAIN_7B["layers"], synth.TRAIN_7B["r"], synth.TRAIN_7B["scaling"]
    if name.startswith("decode"):
        g = torch.Generator(device="cuda").manual_seed(1)
        qws = [api.nf4_quantize_dq(torch.randn((l.N, l.K), generator=g, device="cuda").mul_(0.02)
                                   .to(torch.bfloat16)) for l in layers7]
        mode = {"decode": "staged", "decode_single": "single", "decode_all7": "all", "decode_valu": "staged",
                "decode_all7_valu": "all", "decode_mfma": "staged", "decode_all7_mfma": "all"}[name]
        product = "valu" if name.endswith("_valu") else "mfma" if name.endswith("_mfma") else None
        res = measure_decode(api, torch, layers7, weight_copies(api, qws), r, s, mode=mode, product=product)
        return {f"T{Td}": {"GB/s": round(nb / secs / 1e9, 1), "us_per_layer_set": round(1e6 * secs, 2)}
                for Td, (secs, nb) in res.items()}
    if name == "forward_midt":
        g = torch.Generator(device="cuda").manual_seed(1)
        qws = [api.nf4_quantize_dq(torch.randn((l.N, l.K), generator=g, device="cuda").mul_(0.02)
                                   .to(torch.bfloat16)) for l in layers7]
        res = measure_forward_midt(api, torch, layers7, weight_copies(api, qws), r, s)
        return {f"T{Tm}": {"TFLOP/s": round(fl / secs / 1e12, 1), "us_per_layer_set": round(1e6 * secs, 2)}
                for Tm, (secs, fl) in res.items()}
    if name == "train_midt":
        g = torch.Generator(device="cuda").manual_seed(1)
        qws = [api.nf4_quantize_dq(torch.randn((l.N, l.K), generator=g, device="cuda").mul_(0.02)
                                   .to(torch.bfloat16)) for l in layers7]
        res = measure_step_midt(api, torch, layers7, weight_copies(api, qws), r, s)
        return {f"T{Tm}": {"TFLOP/s": round(fl / secs / 1e12, 1), "us_per_layer_set": round(1e6 * secs, 2)}
                for Tm, (secs, fl) in res.items()}
    if name == "single_layer":
        return {k: {"GB/s": round(nb / secs / 1e9, 1), "us_per_launch": round(1e6 * secs, 3)}
                for k, (kind, secs, amt, nb, _) in measure_single_layer(api, torch, synth).items()}
    if name in ("train_7b", "train_7b_fused"):
        import numpy as np
        comp, ms, att, _, _ = measure_train_7b(api, torch, synth, np, args.steps, None, fused=name.endswith("fused"))
        return {"ms_per_step": round(ms, 4), "attainment": round(att, 4), "phases": comp}
    if name == "merge":
        g = torch.Generator(device="cuda").manual_seed(1)
        qws = [api.nf4_quantize_dq(torch.randn((l.N, l.K), generator=g, device="cuda").mul_(0.02)
                                   .to(torch.bfloat16)) for l in layers7]
        secs, nbytes = measure_merge(api, torch, layers7, weight_copies(api, qws), r, s)
        return {"GB/s": round(nbytes / secs / 1e9, 1), "us_per_layer_set": round(1e6 * secs, 2)}
    if name == "calibration":
        return {k: round(v / 1e9, 1) for k, v in measure_calibration(torch, calib).items()}
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
                    help="only the headline step and the roofline kernel (for a kernel trace of the step alone)")
    ap.add_argument("--only", choices=("decode", "decode_single", "decode_all7", "decode_valu", "decode_all7_valu",
                                       "decode_mfma", "decode_all7_mfma", "single_layer", "train_7b", "train_7b_fused", "forward_midt", "train_midt",
                                       "merge", "calibration", "stream_70b"),
                    help="run one component alone (no step, roofline loop or CPU baseline), e.g. for a kernel trace")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the calibration copy and the k_fwd launches at the 65B shapes (for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path is single-GPU by design); --gpus {args.gpus} is not "
              f"supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from qlora_linear_layers_amd import api, calib, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    api.lib()

    if args.only:
        calibration_copy(torch, calib)
        print(json.dumps({"component": args.only, **only_component(args.only, api, torch, synth, calib, args)}),
              flush=True)
        return

    cfg = synth.LAYER_65B
    layers, T, r, s = cfg["layers"], cfg["T"], cfg["r"], cfg["scaling"]
    bufs = layer_65b_buffers(api, torch, synth)

    if args.roofline_only:
        calibration_copy(torch, calib)
        flops, secs = measure_roofline_kernel(api, torch, bufs, args.steps)
        print(json.dumps({"roofline_kernel": "k_fwd", "tflops": flops / secs / 1e12, "us_per_launch": secs * 1e6,
                          "copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                          "gemm_source_sha256_16": source_hash()}), flush=True)
        return

    # headline: the 65B-shaped layer step
    ws = torch.empty(max(api.qlora_workspace_bytes(T, l.K, l.N, r) for l in layers), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    step, nev = layer_step(api, bufs, T, r, s, ws, stream, with_grads=False)
    wall, evs = run_step(torch, step, nev, args.steps, args.warmup)
    ms_per_step = 1e3 * wall / args.steps
    calib_res = None if args.no_extras else measure_calibration(torch, calib, bufs)
    comp, roof_step = step_phases(bufs, evs, args.steps, T, r, "backward_input", calib_res)

    # roofline of the dominant kernel: k_fwd at the same shapes, timed alone (r = 0 forward = one launch)
    rf_flops, rf_secs = measure_roofline_kernel(api, torch, bufs, max(args.steps // 2, 3))
    achieved = rf_flops / rf_secs / 1e12
    traffic = stored_traffic()
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(achieved / 2500.0, 4),
                "traffic": None if traffic is None else round(traffic),
                "kernel": "k_fwd: fused NF4 double-dequant + MFMA bf16 GEMM, 65B layer shapes at T=2048 "
                          "(per-launch average over the 7 linears)",
                "us_per_launch": round(1e6 * rf_secs, 2),
                "flops_per_launch": rf_flops}
    if calib_res:
        roofline["frac_of_measured_mfma_peak"] = round(achieved * 1e12 / calib_res["mfma_flop/s"], 4)

    out = {
        "metric": "QLoRA linear fwd TFLOP/s + NF4 quant/dequant GB/s, as % of MI355X roofline",
        "value": round(100.0 * roof_step / (wall / args.steps), 3),
        "unit": "% of MI355X roofline",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "LLaMA-65B-shaped layer, 7 linears (q/k/v/o 8192x8192, gate/up 22016x8192, "
                               "down 8192x22016), T=2048 tokens, LoRA r=64 alpha=16; step = quantize + dequantize "
                               "(grouped) + forward + backward input (dX) of every linear",
                   "tokens": T, "rank": r, "parallelism": "none (1 GPU)"},
        "components": comp,
        "roofline": roofline,
    }
    if not args.no_extras:
        comp["calibration"] = {
            "stream_copy_GB/s": round(calib_res["copy_B/s"] / 1e9, 1),
            "stream_copy_frac_of_hbm_peak": round(calib_res["copy_B/s"] / HBM_PEAK, 4),
            "mfma_loop_TFLOP/s": round(calib_res["mfma_flop/s"] / 1e12, 1),
            "mfma_loop_frac_of_mfma_peak": round(calib_res["mfma_flop/s"] / MFMA_BF16_PEAK, 4),
            "torch_matmul_on_dequantized_W_TFLOP/s": round(calib_res["torch_matmul_flop/s"] / 1e12, 1),
            "note": "128-bit streaming copy of 1 GiB (read + write bytes); MFMA-only loop (v_mfma_f32_32x32x16_bf16, "
                    "16 independent chains per wave, one wave per SIMD); torch.matmul (hipBLASLt) of X by the "
                    "dequantized bf16 W' on the 65B shapes, T=2048 (unfused context, no LoRA term)"}
        for b in bufs:
            b.pop("w", None)
        del bufs, ws
        torch.cuda.empty_cache()
        # config 1: the single 4096 x 4096 layer
        for name, (kind, secs, amt, nb, nset) in measure_single_layer(api, torch, synth).items():
            e = phase_entry(kind, amt, nb, secs, calib_res)
            e.pop("ms")
            e["us_per_launch"] = round(1e6 * secs, 3)
            if kind == "mfma":
                e["GB/s"] = round(nb / secs / 1e9, 1)
                e["frac_of_hbm_peak"] = round(nb / secs / HBM_PEAK, 4)
            e["note"] = (f"4096x4096, T=16, r=16, s=1; 100 back-to-back launches over {nset} buffer sets "
                         f"(>= 512 MB rotated)")
            comp[f"single_layer_{name}"] = e
        # config 3: the 7B training step (forward + backward with dA, dB)
        c7, ms7, att7, bufs7, ws7 = measure_train_7b(api, torch, synth, np, args.steps, calib_res)
        comp["train_7b"] = {"ms_per_step": round(ms7, 4), "attainment": round(att7, 4), "phases": c7,
                            "note": "LLaMA-7B-shaped layer, T=4096, r=64 alpha=16: quantize + dequantize (grouped) "
                                    "+ forward + backward (dX, dA, dB; s X A kept from the forward)"}
        c7f, ms7f, att7f, bf, wsf = measure_train_7b(api, torch, synth, np, args.steps, calib_res, fused=True)
        comp["train_7b_fused"] = {"ms_per_step": round(ms7f, 4), "attainment": round(att7f, 4), "phases": c7f,
                                  "note": "the same step with the fused backward: dA and dB formed inside the dX "
                                          "kernel (QLORA_BWD_FUSED_GRADS), 4 launches per linear instead of 5"}
        del bf, wsf
        # config 2: decode, three launch patterns
        sets = weight_copies(api, [b["qw"] for b in bufs7])
        layers7, r7, s7 = synth.TRAIN_7B["layers"], synth.TRAIN_7B["r"], synth.TRAIN_7B["scaling"]
        notes = {"single": "one launch pair per linear",
                 "staged": "grouped launches per dependency stage: q/k/v, o, gate/up, down",
                 "all": "all 7 linears in one grouped launch pair (independent inputs)"}
        products = {None: "the library's decode product for T", "mfma": "small-M MFMA (16x16x32) product",
                    "valu": "VALU dot-product form (v_dot2, no MFMA)"}
        for mode, prefix, product in (("staged", "decode", None), ("single", "decode_single", None),
                                      ("all", "decode_all7", None), ("staged", "decode_mfma", "mfma"),
                                      ("all", "decode_all7_mfma", "mfma"), ("staged", "decode_valu", "valu"),
                                      ("all", "decode_all7_valu", "valu")):
            for Td, (secs, nbytes) in measure_decode(api, torch, layers7, sets, r7, s7, mode=mode,
                                                     product=product).items():
                comp[f"{prefix}_T{Td}"] = {
                    "GB/s": round(nbytes / secs / 1e9, 1), "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                    "frac_of_measured_peak": round(nbytes / secs / calib_res["copy_B/s"], 4),
                    "us_per_layer_set": round(1e6 * secs, 2),
                    "note": "7 linears, fused NF4 double dequant + " + products[product] + " incl. LoRA; "
                            + notes[mode] + "; weights rotated over 6 copies"}
        for name, (kind, secs, amt) in measure_sq(api, torch, bufs7, synth.TRAIN_7B["T"], r7, s7, ws7).items():
            comp[name] = phase_entry(kind, amt, None, secs)
            comp[name]["note"] = "single quantization (fp32 absmax per 64 weights), 7B layer set, T=4096"
        for name, (kind, secs, amt) in measure_f16(api, torch, bufs7, synth.TRAIN_7B["T"], r7, s7, ws7).items():
            comp[name] = phase_entry(kind, amt, None, secs)
            comp[name]["note"] = "fp16 compute type, 7B layer set, T=4096" + (
                " (forward + backward pass, s X A reused)" if name == "backward_f16" else "")
        abl, secs, nbytes = measure_ablation(api, torch, synth, np, bufs7)
        comp["int4_ablation"] = {
            "relative_rms_error": {k: {dt: round(e, 5) for dt, e in v.items()} for k, v in abl.items()},
            "int4_quantize_GB/s": round(nbytes / secs / 1e9, 1),
            "note": "NF4 vs INT4 absmax levels, fp32 absmax per 64 weights for both"}
        secs, nbytes = measure_merge(api, torch, layers7, sets, r7, s7)
        comp["merge"] = {"GB/s": round(nbytes / secs / 1e9, 1), "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                         "us_per_layer_set": round(1e6 * secs, 2),
                         "note": "7 linears, W_m = RNE_bf16(W' + s (A B)^T), r=64; weights rotated over 6 copies"}
        for Tm, (secs, flops) in measure_forward_midt(api, torch, layers7, sets, r7, s7).items():
            comp[f"forward_T{Tm}"] = {"TFLOP/s": round(flops / secs / 1e12, 1),
                                      "frac_of_mfma_peak": round(flops / secs / MFMA_BF16_PEAK, 4),
                                      "us_per_layer_set": round(1e6 * secs, 2),
                                      "note": "7 linears, r=64, forward at a token count whose 256x256 tiles fill "
                                              "part of the chip (split-k where it pays); weights rotated over 6 copies"}
        for Tm, (secs, flops) in measure_step_midt(api, torch, layers7, sets, r7, s7).items():
            comp[f"train_step_T{Tm}"] = {"TFLOP/s": round(flops / secs / 1e12, 1),
                                         "frac_of_mfma_peak": round(flops / secs / MFMA_BF16_PEAK, 4),
                                         "us_per_layer_set": round(1e6 * secs, 2),
                                         "note": "7 linears, r=64: forward, then dX, dA, dB with s X A reused, at a "
                                                 "token count whose tiles fill part of the chip (split-k forward and "
                                                 "dX); weights rotated over 6 copies"}
        for Tp, (secs, nbytes, flops) in measure_prefill(api, torch, layers7, sets, r7, s7).items():
            comp[f"prefill_T{Tp}"] = {"TFLOP/s": round(flops / secs / 1e12, 1), "GB/s": round(nbytes / secs / 1e9, 1),
                                      "frac_of_hbm_peak": round(nbytes / secs / HBM_PEAK, 4),
                                      "us_per_layer_set": round(1e6 * secs, 2),
                                      "note": "7 linears, r=64, forward at a small-prefill T: 16-token windows as one "
                                              "grouped decode launch pair; weights rotated over 6 copies"}
        del sets, bufs7, ws7
        torch.cuda.empty_cache()
        # config 5: the 70B-shaped stream
        secs, moved, packed, params = measure_stream_70b(torch, synth)
        closed = params * (4 + 8 / 64 + 32 / 16384) / 8
        comp["stream_70b"] = {"GB/s": round(moved / secs / 1e9, 1), "frac_of_hbm_peak": round(moved / secs / HBM_PEAK, 4),
                              "frac_of_measured_peak": round(moved / secs / calib_res["copy_B/s"], 4),
                              "ms": round(1e3 * secs, 3), "params": params, "packed_bytes": packed,
                              "closed_form_bytes": int(closed), "bits_per_param": round(8 * packed / params, 9),
                              "note": "80 layers x 7 tensors (70B shapes, 0.1% t3 outliers), grouped quantize_dq then "
                                      "grouped dequantize per layer, one layer resident; kernel time only"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, T, r, s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
