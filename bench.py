#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 CausalConv3d hot path on one MI355X.

A step is one pass of the whole per-layer path over one batch of synthetic
input that is already resident in HBM:
    absmax (HBM pass) -> quantize (HBM pass) -> implicit-GEMM conv with fused
    FP32 rescale + bias + bf16 store.
Weight quantization happens once at load, outside the timed region.

Default workload: the latent-level layer, Cin=Cout=384, 3x3x3, input
[1,384,1,128,128] bf16 with 5 % x20 outliers and an explicit 2-frame zero
cache (all 27 taps are data).  ``--workload`` picks another layer.

Prints ONE JSON line.  ``value`` is INT8 TOPS of the whole step (algorithmic
conv ops / step time); the ``roofline`` object covers the dominant kernel
(the conv), timed with HIP events around every launch on the stream it runs
on; ``cpu_baseline`` is the CPU oracle on a bounded sample of the same layer.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT8 TOPS & ms/layer of W8A8 CausalConv3d (% MFMA peak); quant-pass HBM GB/s"
PEAK_INT8_TOPS = 5000.0       # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, 8 TB/s
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, 2.5 PFLOP/s


def layer_counts(spec, cache: bool):
    """Algorithmic work of one layer (conv ops exclude structurally zero taps)."""
    kt, kh, kw = spec.k
    valid = 0
    for t in range(spec.T):
        valid += kt if cache else min(kt, t + 1)
    hw = spec.H * spec.W
    ops = 2 * spec.N * spec.Cout * spec.Cin * kh * kw * hw * valid
    nominal = 2 * spec.N * spec.Cout * spec.Cin * kt * kh * kw * hw * spec.T
    numel = spec.numel
    conv_bytes = (numel + (spec.N * (kt - 1) * hw * spec.Cin if cache else 0)
                  + spec.Cout * spec.Cin * kt * kh * kw + 8 * spec.Cout
                  + 2 * spec.Cout * spec.N * spec.T * hw)
    return dict(ops=ops, nominal_ops=nominal, numel=numel, conv_bytes=conv_bytes,
                absmax_bytes=2 * numel, quant_bytes=3 * numel)


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(workload_key, conv_src):
    """HBM bytes per conv launch from the committed rocprofv3 counter summary,
    valid only while the kernel source is the one the counters were taken on."""
    p = os.path.join(ROOT, "profiles", f"traffic_conv_{workload_key}.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_s = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m_b or not m_s or m_s.group(1) != source_sha(conv_src):
        return None
    return float(m_b.group(1))


def cpu_baseline(ci, cache_np, budget_s=12.0, clip=1.0):
    """The CPU oracle (as it stands) on a bounded sample of the same layer:
    absmax + quantize over the whole input, the conv + epilogue over a random
    sample of output positions; scaled to the whole layer in TOPS."""
    import numpy as np
    import oracle

    spec = ci.spec
    wq, ws = oracle.quantize_weights(ci.w, clip)
    t0 = time.perf_counter()
    a, s, xq = oracle.act_absmax_quant(ci.x, clip)
    t_quant = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    total = spec.positions
    npos = 64
    t_conv = 0.0
    used = 0
    while True:
        pos = rng.integers(0, total, npos).astype(np.int64)
        t0 = time.perf_counter()
        acc = oracle.conv_acc(xq, wq, cache_np, positions=pos)
        oracle.epilogue(acc, s, ws, ci.b)
        dt = time.perf_counter() - t0
        t_conv += dt
        used += npos
        if t_conv + t_quant > budget_s or used >= total:
            break
        npos = int(min(total - used, max(64, npos * 2, (budget_s - t_conv - t_quant) / max(dt, 1e-6) * npos * 0.8)))
    per_pos = t_conv / used
    t_layer = t_quant + per_pos * total
    cnt = layer_counts(spec, cache_np is not None)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": cnt["ops"] / t_layer / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": (f"absmax+quantize over all {spec.numel} elements ({t_quant:.2f} s) + conv/epilogue "
                       f"at {used} random output positions of {total} ({t_conv:.2f} s), scaled to the "
                       f"whole layer: {t_layer:.1f} s/layer")}


def first_calls(with_init: bool = False):
    """First-call latency at each new resolution, in one process: every layer
    of the two level sweeps (new shapes, new tile configurations) runs its
    step (absmax + quantize + conv) once from a cold start at that shape, then
    again; host wall clock around each call with a device synchronize on both
    sides.  Nothing is compiled or tuned at run time: every kernel is built
    ahead of time for gfx950.  With `with_init`, qvae_init (which loads the
    library's GPU code) runs first and is timed on its own."""
    import numpy as np
    import torch
    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl
    dev = "cuda:0"
    t0 = time.perf_counter()
    ops.lib()
    torch.zeros(1, device=dev)
    torch.cuda.synchronize()
    out = {"probe": "first call per resolution", "library_and_context_ms": round((time.perf_counter() - t0) * 1e3, 2),
           "layers": []}
    if with_init:
        t1 = time.perf_counter()
        ops.init()
        out["qvae_init_ms"] = round((time.perf_counter() - t1) * 1e3, 3)
    for key in ("sweep_1024", "sweep_840x1256"):
        for ci in wl.draw_workload(key):
            spec = ci.spec
            x = torch.from_numpy(ci.x.view(np.int16)).to(dev).view(torch.bfloat16)
            wq, ws = ops.quantize_weights(torch.from_numpy(ci.w).to(dev))
            b = torch.from_numpy(ci.b).to(dev)
            torch.cuda.synchronize()
            ts = []
            for _ in range(2):
                t1 = time.perf_counter()
                ops.layer_forward(x, wq, ws, b)
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t1) * 1e3)
            out["layers"].append({"layer": f"{key} {spec.Cin}->{spec.Cout} @{spec.H}x{spec.W}",
                                  "first_ms": round(ts[0], 3), "second_ms": round(ts[1], 3)})
    print(json.dumps(out))


def zero_share_of_k(T: int, kt: int, zero_cache: bool) -> float:
    """Share of a layer's contraction (summed over its T frames) that reads an
    all-zero cache: frame t takes max(0, kt-1-t) of its kt temporal taps from
    the cache.  Without a cache those taps are front padding and skipped, so
    they are not part of K at all."""
    if not zero_cache:
        return 0.0
    return sum(max(0, kt - 1 - t) for t in range(T)) / (T * kt)


def mfma_probe():
    """The matrix cores' sustained rate per instruction shape and operand
    distribution (qvae_probe_mfma: nothing but matrix instructions on operands
    held in registers, one wave per SIMD on every CU): the power-limited
    ceiling the convolution's rate is bounded by.  Median of 5 launches of
    ~2 ms after a warm-up; 256 and 512 workgroups."""
    import torch
    from w8a8_int8_quantized_act_amd import ops
    dev = "cuda:0"
    g = torch.Generator().manual_seed(12)

    def table(kind):
        n = 14 * 4096 * 16
        if kind == "zero":
            b = torch.zeros(n, dtype=torch.int8)
        elif kind == "small":
            b = torch.randint(-5, 6, (n,), generator=g, dtype=torch.int8)
        elif kind == "full":
            b = torch.randint(-127, 128, (n,), generator=g, dtype=torch.int8)
        else:   # bf16 values uniform in [-2, 2)
            v = (torch.rand(n // 2, generator=g) * 4 - 2).to(torch.bfloat16)
            b = v.view(torch.int8)
        return b.view(torch.int32).reshape(14, 4096, 4).to(dev)

    out = {"probe": "matrix-core rate by instruction shape and operand values", "peaks": {
        "int8_TOPS": 5000.0, "bf16_TFLOPS": 2500.0}, "results": {}}
    stream = torch.cuda.current_stream()
    cases = [("i8_32x32x32", k) for k in ("zero", "small", "full")] + \
            [("i8_16x16x64", k) for k in ("zero", "small", "full")] + \
            [("bf16_32x32x16", k) for k in ("zero", "bf16")] + [("bf16_16x16x32", k) for k in ("zero", "bf16")]
    for name, kind in cases:
        shape = ops.PROBE_SHAPES[name]
        tab = table(kind)
        for blocks in (256, 512):
            target = 8e12 if shape < 2 else 4e12            # ~2 ms of work per launch
            iters = max(1, round(target / (blocks * 4 * ops.PROBE_WORK[shape])))
            ops.probe_mfma(shape, tab, 100, blocks)
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                ops.probe_mfma(shape, tab, iters, blocks)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ms = sorted(ts)[2]
            rate = blocks * 4 * iters * ops.PROBE_WORK[shape] / (ms * 1e-3) / 1e12
            out["results"][f"{name}/{kind}/{blocks}"] = {"ms": round(ms, 3), "rate_T_per_s": round(rate, 1)}
    print(json.dumps(out))


def operand_probe(args):
    """The workload's conv (same packed weights, scale and bias) timed on int8
    inputs and caches drawn from different value distributions: the matrix
    cores' throughput depends on the operand values (power), not only on the
    instruction count.  Inputs are seeded draws; nothing is checked against the
    oracle here (the kernels' parity is the tests' job)."""
    import torch
    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl
    dev = "cuda:0"
    ci = wl.draw_workload(args.workload, only=args.level)[-1]
    spec = ci.spec
    kt = spec.k[0]
    wq, ws = ops.quantize_weights(torch.from_numpy(ci.w).to(dev))
    b = torch.from_numpy(ci.b).to(dev)
    xs = torch.tensor([0.01], dtype=torch.float32, device=dev)
    y = torch.empty((spec.N, spec.T, spec.H, spec.W, spec.Cout), dtype=torch.bfloat16, device=dev)
    g = torch.Generator().manual_seed(11)
    shape = (spec.N, spec.T, spec.H, spec.W, spec.Cin)
    cshape = (spec.N, kt - 1, spec.H, spec.W, spec.Cin)

    def codes(kind, shp):
        if kind == "zero":
            return torch.zeros(shp, dtype=torch.int8)
        if kind == "small":
            return torch.randint(-5, 6, shp, generator=g, dtype=torch.int8)
        if kind == "silu":
            z = torch.randn(shp, generator=g)
            v = z * torch.sigmoid(z)
            return torch.round(v / (v.abs().max() / 127)).clamp(-127, 127).to(torch.int8)
        return torch.randint(-127, 128, shp, generator=g, dtype=torch.int8)

    cnt = layer_counts(spec, True)
    out = {"probe": "conv time by operand distribution", "workload": args.workload, "level": args.level,
           "algorithmic_ops": cnt["ops"], "note": "input and 2-frame cache drawn from the same distribution; "
           "median of 5 runs of 20 back-to-back launches (HIP events)", "results": {}}
    stream = torch.cuda.current_stream()
    for kind in ("zero", "small", "silu", "full"):
        xq = codes(kind, shape).to(dev)
        cache = codes(kind, cshape).to(dev) if kt > 1 else None
        run = lambda: ops.causalconv3d_w8a8(xq, xs, wq, ws, b, cache, out=y)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        meds = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            meds.append(e0.elapsed_time(e1) / 20)
        ms = sorted(meds)[2]
        out["results"][kind] = {"conv_us": round(ms * 1e3, 2), "tops": round(cnt["ops"] / (ms * 1e-3) / 1e12, 1)}
    print(json.dumps(out))


def decoder_cpu_baseline(data, budget_s=12.0):
    """The oracle (as it stands) on the native residual branches of the stack:
    RMSNorm + SiLU over one layer's whole input and the exact bf16 conv at a
    random sample of output positions, per distinct layer shape, scaled to all
    28 layers (ms per stack)."""
    import numpy as np
    import torch

    import oracle

    shapes = {}
    for d in data:
        s = d["spec"]
        shapes.setdefault((s.Cin, s.Cout, s.H, s.W), []).append(d)
    per_shape_budget = budget_s / len(shapes)
    total_s = 0.0
    notes = []
    rng = np.random.default_rng(0)
    for (cin, cout, h, w), ds in shapes.items():
        d = ds[0]
        xb = d["x"].view(torch.int16).cpu().numpy().view(np.uint16)
        gam = d["gam"].cpu().numpy()
        wb = d["w"].view(torch.int16).cpu().numpy().view(np.uint16)
        b = d["b"].cpu().numpy()
        t0 = time.perf_counter()
        hb = oracle.rmsnorm_silu(xb, gam, 1e-6)
        t_norm = time.perf_counter() - t0
        npos, t_conv, used = 16, 0.0, 0
        while t_conv < per_shape_budget * 0.8 and used < h * w:
            pos = rng.integers(0, h * w, npos).astype(np.int64)
            t0 = time.perf_counter()
            oracle.conv_bf16(hb, wb, b, positions=pos)
            t_conv += time.perf_counter() - t0
            used += npos
            npos *= 2
        layer_s = t_norm + t_conv / used * h * w
        total_s += layer_s * len(ds)
        notes.append(f"{cin}->{cout} @{h}x{w}: norm {t_norm:.2f} s + conv at {used} of {h * w} positions "
                     f"{t_conv:.2f} s -> {layer_s:.1f} s/layer x {len(ds)}")
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    return {"value": round(total_s * 1e3, 1), "unit": "ms per stack (native residual branches)", "cores": threads,
            "kind": "oracle", "sample": "; ".join(notes)}


def decoder_stack(args):
    """The 28 residual-block convs of the decoder at one output size, run as
    each preset says (W8A8 layer step = absmax + quantize + INT8 conv, native =
    bf16 conv), timed as one stack per preset."""
    import numpy as np
    import torch

    from w8a8_int8_quantized_act_amd import decoder, ops

    dev = "cuda:0"
    L = ops.lib()
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream()
    sp = P(stream.cuda_stream)
    layers = decoder.residual_convs(args.out_h, args.out_w)
    g = torch.Generator(device=dev).manual_seed(7)
    data = []
    for spec in layers:
        w = (torch.randn(spec.Cout, spec.Cin, 3, 3, 3, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        b = torch.randn(spec.Cout, generator=g, device=dev) * 0.01
        x = torch.randn(1, 1, spec.H, spec.W, spec.Cin, generator=g, device=dev)
        x = (x * torch.sigmoid(x)).to(torch.bfloat16)
        wq, ws = ops.quantize_weights(w.float())
        wp = ops.pack_weights_bf16(w)
        gam = (1.0 + 0.1 * torch.randn(spec.Cin, generator=g, device=dev)).float()
        d = dict(spec=spec, x=x, b=b, w=w, wq=wq, ws=ws, wp=wp, gam=gam,
                 hb=torch.empty(x.shape, dtype=torch.bfloat16, device=dev),
                 xq=torch.empty(x.shape, dtype=torch.int8, device=dev),
                 xs=torch.empty((1,), dtype=torch.float32, device=dev),
                 am=torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=dev),
                 y=torch.empty((1, 1, spec.H, spec.W, spec.Cout), dtype=torch.bfloat16, device=dev))
        dims = (1, 1, spec.H, spec.W, spec.Cin, spec.Cout, 3, 3, 3)
        d["w8a8"] = [(L.qvae_act_absmax, (P(x.data_ptr()), x.numel(), P(d["am"].data_ptr()), sp)),
                     (L.qvae_act_quantize, (P(x.data_ptr()), x.numel(), ctypes.c_float(1.0), P(d["am"].data_ptr()),
                                            P(d["xs"].data_ptr()), P(d["xq"].data_ptr()), sp)),
                     (L.qvae_causalconv3d_w8a8, (P(d["xq"].data_ptr()), P(d["xs"].data_ptr()), None,
                                                 P(wq.data_ptr()), P(ws.data_ptr()), P(b.data_ptr()), *dims,
                                                 P(d["y"].data_ptr()), sp))]
        d["native"] = [(L.qvae_causalconv3d_bf16, (P(x.data_ptr()), None, P(wp.data_ptr()), P(b.data_ptr()), *dims,
                                                   P(d["y"].data_ptr()), sp))]
        # the residual branch: RMSNorm + SiLU of x into h, then the conv on h
        npix, hp = spec.H * spec.W, P(d["hb"].data_ptr())
        eps = ctypes.c_float(1e-6)
        d["br_native"] = [(L.qvae_rmsnorm_silu, (P(x.data_ptr()), npix, spec.Cin, P(gam.data_ptr()), eps, hp, sp)),
                          (L.qvae_causalconv3d_bf16, (hp, None, P(wp.data_ptr()), P(b.data_ptr()), *dims,
                                                      P(d["y"].data_ptr()), sp))]
        d["br_w8a8"] = [(L.qvae_rmsnorm_silu_absmax, (P(x.data_ptr()), npix, spec.Cin, P(gam.data_ptr()), eps, hp,
                                                      P(d["am"].data_ptr()), sp)),
                        (L.qvae_act_quantize, (hp, x.numel(), ctypes.c_float(1.0), P(d["am"].data_ptr()),
                                               P(d["xs"].data_ptr()), P(d["xq"].data_ptr()), sp)),
                        (L.qvae_causalconv3d_w8a8, (P(d["xq"].data_ptr()), P(d["xs"].data_ptr()), None,
                                                    P(wq.data_ptr()), P(ws.data_ptr()), P(b.data_ptr()), *dims,
                                                    P(d["y"].data_ptr()), sp))]
        # the branch with the quantize pass absorbed into the conv (it reads bf16 h)
        d["br_w8a8_qin"] = [d["br_w8a8"][0],
                            (L.qvae_causalconv3d_w8a8_qin, (hp, None, P(d["am"].data_ptr()), ctypes.c_float(1.0),
                                                            P(wq.data_ptr()), P(ws.data_ptr()), P(b.data_ptr()),
                                                            *dims, P(d["xs"].data_ptr()), P(d["y"].data_ptr()), sp))]
        d["qin_ok"] = spec.H * spec.W >= decoder.QIN_MIN_PIXELS
        # the same branch without the fused maximum: norm + SiLU, then both quantizer passes
        d["br_w8a8_unfused"] = [d["br_native"][0]] + [
            (f, (hp,) + a[1:]) for f, a in d["w8a8"][:2]] + d["br_w8a8"][2:]
        d["ops"] = 2 * spec.Cout * spec.Cin * 9 * spec.H * spec.W      # T = 1: the two front frames are padding
        data.append(d)

    def timed(calls, k):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        rc = 0
        for _ in range(k):
            for f, a in calls:
                rc |= f(*a)
        e1.record(stream)
        torch.cuda.synchronize()
        assert rc == 0
        return e0.elapsed_time(e1) / k

    total_ops = sum(d["ops"] for d in data)
    presets = {}
    for preset in ("native", "conservative", "balanced", "aggressive"):
        pl = decoder.plan(preset, layers)
        calls = [c for d in data for c in (d["w8a8"] if pl[d["spec"].name] else d["native"])]
        timed(calls, 2)
        ms = float(np.median([timed(calls, args.steps) for _ in range(3)]))
        presets[preset] = {"w8a8_layers": sum(pl.values()), "ms_per_stack": round(ms, 4),
                           "TOPS": round(total_ops / (ms * 1e-3) / 1e12, 1)}
    base = presets["native"]["ms_per_stack"]
    for v in presets.values():
        v["speedup_vs_native"] = round(base / v["ms_per_stack"], 3)
    # whole residual branches (norm + SiLU + conv) per preset; W8A8 layers with
    # the maximum fused into the norm pass, and (for Aggressive) without it
    branches = {}
    def branch(d, key):
        if key == "qin":   # the input-quantizing conv where the runner's rule picks it
            return d["br_w8a8_qin"] if d["qin_ok"] else d["br_w8a8"]
        return d[key]

    for preset, key in (("native", "br_w8a8"), ("conservative", "br_w8a8"), ("balanced", "br_w8a8"),
                        ("aggressive", "br_w8a8"), ("aggressive_unfused_absmax", "br_w8a8_unfused"),
                        ("conservative_quantize_in_conv", "qin"), ("balanced_quantize_in_conv", "qin"),
                        ("aggressive_quantize_in_conv", "qin")):
        pl = decoder.plan(preset.split("_")[0], layers)
        calls = [c for d in data for c in (branch(d, key) if pl[d["spec"].name] else d["br_native"])]
        timed(calls, 2)
        ms = float(np.median([timed(calls, args.steps) for _ in range(3)]))
        branches[preset] = {"w8a8_layers": sum(pl.values()), "ms_per_stack": round(ms, 4)}
    base_b = branches["native"]["ms_per_stack"]
    for v in branches.values():
        v["speedup_vs_native"] = round(base_b / v["ms_per_stack"], 3)
    # each distinct layer shape alone: native bf16 conv and the W8A8 step / conv
    shapes = {}
    for d in data:
        s = d["spec"]
        key = f"{s.Cin}->{s.Cout} @{s.H}x{s.W}"
        if key in shapes:
            continue
        nat = timed(d["native"], args.steps)
        step = timed(d["w8a8"], args.steps)
        conv = timed(d["w8a8"][2:], args.steps)
        qin = timed(d["br_w8a8_qin"][1:], args.steps)
        norm = timed(d["br_native"][:1], args.steps)
        norm_mx = timed(d["br_w8a8"][:1], args.steps)
        quant = timed(d["br_w8a8"][1:2], args.steps)
        nbytes = 4 * s.H * s.W * s.Cin
        shapes[key] = {"alg_GOP": round(d["ops"] / 1e9, 2),
                       "native_conv_ms": round(nat, 5),
                       "native_TFLOPs": round(d["ops"] / (nat * 1e-3) / 1e12, 1),
                       "native_frac_of_bf16_peak": round(d["ops"] / (nat * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "w8a8_step_ms": round(step, 5), "w8a8_conv_ms": round(conv, 5),
                       "w8a8_conv_frac_of_int8_peak": round(d["ops"] / (conv * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                       "norm_silu_ms": round(norm, 5), "norm_silu_GBs": round(nbytes / (norm * 1e-3) / 1e9, 1),
                       "norm_silu_absmax_ms": round(norm_mx, 5), "quantize_ms": round(quant, 5),
                       "branch_native_ms": round(norm + nat, 5), "branch_w8a8_ms": round(norm_mx + quant + conv, 5),
                       "conv_quantize_in_ms": round(qin, 5), "branch_w8a8_qin_ms": round(norm_mx + qin, 5)}
    cpu = None if args.no_cpu else decoder_cpu_baseline(data, args.cpu_budget)
    print(json.dumps({"probe": "decoder conv stack by preset", "output": f"{args.out_h}x{args.out_w}",
                      "cpu_baseline": cpu,
                      "layers": len(layers), "alg_GOP_per_stack": round(total_ops / 1e9, 1),
                      "steps": args.steps, "presets": presets, "residual_branches": branches, "per_shape": shapes,
                      "note": "presets: W8A8 layer = absmax + quantize + INT8 conv, native layer = bf16 conv "
                              "(FP32 accumulation); residual_branches: each conv preceded by its RMSNorm + SiLU "
                              "pass (native: norm + SiLU -> bf16 conv; W8A8: norm + SiLU with the fused maximum -> "
                              "quantize -> INT8 conv; *_quantize_in_conv: the conv quantizes h itself on frames of "
                              f"at least {decoder.QIN_MIN_PIXELS} pixels); each layer has its own resident input; HIP events around "
                              "K back-to-back stacks, median of 3"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="latent_384_128_cache")
    ap.add_argument("--level", type=int, default=0, help="layer index inside a level sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--first-calls", action="store_true",
                    help="only time the first and second layer step at each resolution of the level sweeps")
    ap.add_argument("--init", action="store_true", help="with --first-calls: call qvae_init first")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="sustained matrix-core rate per instruction shape and operand distribution")
    ap.add_argument("--operand-probe", action="store_true",
                    help="only time the workload's conv on int8 inputs of different value distributions")
    ap.add_argument("--frames", type=int, default=0,
                    help="a multi-frame variant: the layer's shape with T frames (redrawn, same recipe)")
    ap.add_argument("--clip", type=float, default=1.0,
                    help="activation and weight clip ratio in (0, 1] (the page fixes 1.0)")
    ap.add_argument("--decoder", action="store_true",
                    help="only time the decoder's 28 residual-block convs per preset (W8A8 vs native bf16)")
    ap.add_argument("--out-h", type=int, default=1024)
    ap.add_argument("--out-w", type=int, default=1024)
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))
        return

    if args.mfma_probe:
        mfma_probe()
        return
    if args.operand_probe:
        operand_probe(args)
        return
    if args.first_calls:
        first_calls(with_init=args.init)
        return
    if args.decoder:
        decoder_stack(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the W8A8 CausalConv3d path here runs on a single MI355X "
              "(multi-GPU sharding is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.lib()
    dev = "cuda:0"

    ci = wl.draw_workload(args.workload, only=args.level)[-1]
    if args.frames and args.frames != ci.spec.T:
        spec_t = dataclasses.replace(ci.spec, T=args.frames, name=f"{ci.spec.name}_t{args.frames}")
        ci = wl.draw_conv(spec_t, torch.Generator().manual_seed(
            1000 * wl.WORKLOADS[args.workload].seed + 10 * args.level + args.frames))
    variant = ci.spec.T != wl.WORKLOADS[args.workload].convs[args.level].T or args.clip != 1.0
    spec = ci.spec
    kt = spec.k[0]
    use_cache = spec.zero_cache
    cnt = layer_counts(spec, use_cache)

    x = torch.from_numpy(ci.x.view(np.int16)).to(dev).view(torch.bfloat16)
    wq, ws = ops.quantize_weights(torch.from_numpy(ci.w).to(dev), args.clip)
    b = torch.from_numpy(ci.b).to(dev)
    cache = (torch.zeros((spec.N, kt - 1, spec.H, spec.W, spec.Cin), dtype=torch.int8, device=dev)
             if use_cache else None)
    absmax = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=dev)
    xs = torch.empty((1,), dtype=torch.float32, device=dev)
    xq = torch.empty(x.shape, dtype=torch.int8, device=dev)
    y = torch.empty((spec.N, spec.T, spec.H, spec.W, spec.Cout), dtype=torch.bfloat16, device=dev)
    y_absmax = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    # Launch arguments marshalled once; the timed loops call the C entry
    # points directly (the same calls ops.* makes, without its per-call checks).
    L = ops.lib()
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    a_absmax = (P(x.data_ptr()), x.numel(), P(absmax.data_ptr()), sp)
    a_quant = (P(x.data_ptr()), x.numel(), ctypes.c_float(args.clip), P(absmax.data_ptr()), P(xs.data_ptr()),
               P(xq.data_ptr()), sp)
    a_conv = (P(xq.data_ptr()), P(xs.data_ptr()), P(cache.data_ptr()) if cache is not None else None,
              P(wq.data_ptr()), P(ws.data_ptr()), P(b.data_ptr()), spec.N, spec.T, spec.H, spec.W, spec.Cin,
              spec.Cout, kt, spec.k[1], spec.k[2], P(y.data_ptr()), sp)

    def absmax_pass():
        return L.qvae_act_absmax(*a_absmax)

    def quant_pass():
        return L.qvae_act_quantize(*a_quant)

    def conv_pass():
        return L.qvae_causalconv3d_w8a8(*a_conv)

    a_conv_mx = a_conv[:-1] + (P(y_absmax.data_ptr()), sp)

    def conv_absmax_pass():
        return L.qvae_causalconv3d_w8a8_absmax(*a_conv_mx)

    def step_chained():
        # a decoder chain with the absmax pass folded into the producing conv:
        # this layer quantizes with the partial maxima its producer left (here
        # the absmax pass's, filled in the warm-up) and emits its own output's
        return quant_pass() | conv_absmax_pass()

    def step():
        return absmax_pass() | quant_pass() | conv_pass()

    # first call in this process (cold code object, cold caches)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert step() == 0
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(fn, k):
        """k back-to-back launches on the stream, bracketed by synchronize and
        by two HIP events on that stream -> (wall ms, event ms) per launch."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        rc = 0
        for _ in range(k):
            rc |= fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        assert rc == 0
        return wall * 1e3 / k, e0.elapsed_time(e1) / k

    # timed region: exactly K steps
    ms_per_step, ev_ms_per_step = timed(step, args.steps)
    value = cnt["ops"] / (ms_per_step * 1e-3) / 1e12

    # per kernel: K back-to-back launches each, on the launch stream
    _, conv_avg = timed(conv_pass, args.steps)
    # the conv again in 5 groups of K/5 launches: median and min of the group averages
    conv_groups = sorted(timed(conv_pass, max(1, args.steps // 5))[1] for _ in range(5))
    _, absmax_avg = timed(absmax_pass, args.steps)
    _, quant_avg = timed(quant_pass, args.steps)
    _, conv_mx_avg = timed(conv_absmax_pass, args.steps)
    ms_chained, _ = timed(step_chained, args.steps)
    conv_tops = cnt["ops"] / (conv_avg * 1e-3) / 1e12

    # quant passes with a cold last-level cache: before each rep a 1 GiB
    # scratch buffer is written on the same stream (evicting the 256 MB
    # Infinity Cache), then one launch is bracketed by two events (the
    # first fires when the fill has finished); median over the reps
    def cold(fn, reps=10):
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(reps):
            scratch.fill_(i & 0xFF)
            e0.record(stream)
            assert fn() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        del scratch
        return float(np.median(ts))

    absmax_cold = cold(absmax_pass)
    quant_cold = cold(quant_pass)

    # the same step replayed from a HIP graph (launch overhead removed)
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs = torch.cuda.current_stream()
            ga = (a_absmax[:-1] + (P(gs.cuda_stream),), a_quant[:-1] + (P(gs.cuda_stream),),
                  a_conv[:-1] + (P(gs.cuda_stream),))
            L.qvae_act_absmax(*ga[0])
            L.qvae_act_quantize(*ga[1])
            L.qvae_causalconv3d_w8a8(*ga[2])
        g.replay()
        torch.cuda.synchronize()
        _, graph_ms = timed(lambda: (g.replay(), 0)[1], args.steps)
    except Exception as exc:  # graphs are an extra figure, never the headline
        print(f"graph replay skipped: {exc}", file=sys.stderr)

    # The matrix cores' power-limited ceiling for this layer (after the timed
    # region): the rate of the instruction the conv uses on random full-range
    # codes and on zeros (qvae_probe_mfma), weighted by the share of K that
    # reads the zero cache.  The frac against it says how close the conv is
    # to what the chip sustains on these operands, not only to the nominal peak.
    ceiling = None
    try:
        shape16 = spec.k[1] == 3 and (spec.Cin // 32) % 2 == 0 and spec.Cout % 192 == 0
        pshape = 1 if shape16 else 0
        gp = torch.Generator().manual_seed(13)
        tabs = {"data": torch.randint(-127, 128, (14 * 4096 * 16,), generator=gp, dtype=torch.int8)
                .view(torch.int32).reshape(14, 4096, 4).to(dev)}
        tabs["zero"] = torch.zeros_like(tabs["data"])
        iters = max(1, round(8e12 / (256 * 4 * ops.PROBE_WORK[pshape])))
        rates = {}
        for nm, tab in tabs.items():
            ops.probe_mfma(pshape, tab, 50, 256)
            torch.cuda.synchronize()
            pts = []
            for _ in range(5):
                q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                q0.record(stream)
                ops.probe_mfma(pshape, tab, iters, 256)
                q1.record(stream)
                torch.cuda.synchronize()
                pts.append(q0.elapsed_time(q1))
            rates[nm] = 256 * 4 * iters * ops.PROBE_WORK[pshape] / (sorted(pts)[2] * 1e-3) / 1e12
        f_zero = zero_share_of_k(spec.T, spec.k[0], use_cache)
        cap = 1.0 / ((1.0 - f_zero) / rates["data"] + f_zero / rates["zero"])
        ceiling = {"instruction": "v_mfma_i32_16x16x64_i8" if shape16 else "v_mfma_i32_32x32x32_i8",
                   "data_TOPS": round(rates["data"], 1), "zero_TOPS": round(rates["zero"], 1),
                   "zero_share_of_K": round(f_zero, 4), "ceiling_TOPS": round(cap, 1),
                   "frac_of_ceiling": round(conv_tops / cap, 4)}
    except Exception as exc:  # an extra figure, never the headline
        print(f"matrix-core ceiling probe skipped: {exc}", file=sys.stderr)

    # output sanity after the timed loop (no stale-output speedups)
    ref_y = ops.causalconv3d_w8a8(xq, xs, wq, ws, b, cache)
    torch.cuda.synchronize()
    assert torch.equal(ref_y.view(torch.int16), y.view(torch.int16))

    conv_src = os.path.join(ROOT, "w8a8_int8_quantized_act_amd", "csrc", "qvae_conv.hip")
    traffic = None if variant else read_traffic(
        args.workload if args.level == 0 else f"{args.workload}_l{args.level}", conv_src)
    wl_name = (args.workload if args.level == 0 and len(wl.WORKLOADS[args.workload].convs) == 1
               else f"{args.workload}[{args.level}]")
    if ci.spec.T != wl.WORKLOADS[args.workload].convs[args.level].T:
        wl_name += f" T={ci.spec.T}"
    if args.clip != 1.0:
        wl_name += f" clip={args.clip:g}"
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wl_name,
            "layer": f"CausalConv3d {spec.k[0]}x{spec.k[1]}x{spec.k[2]} Cin={spec.Cin} Cout={spec.Cout} "
                     f"input [{spec.N},{spec.Cin},{spec.T},{spec.H},{spec.W}] bf16 channels-last"
                     + (", explicit 2-frame zero cache" if use_cache else ", causal front padding"),
            "global_batch": spec.N,
            "parallelism": "single GPU",
            "step": "absmax + quantize + implicit-GEMM conv (fused FP32 rescale, bias, bf16 store)",
        },
        "roofline": {
            "kernel": "k_conv_igemm",
            "bound": "mfma",
            "achieved": round(conv_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "op_kind": "INT8 ops (TOPS), algorithmic count",
            "frac": round(conv_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_launch": cnt["ops"],
            "avg_launch_ms": round(conv_avg, 5),
            "median_launch_ms": round(conv_groups[2], 5),
            "min_launch_ms": round(conv_groups[0], 5),
            "algorithmic_bytes_per_launch": cnt["conv_bytes"],
            "ai_ops_per_byte": round(cnt["ops"] / cnt["conv_bytes"], 1),
            # the attainable roofline min(MFMA peak, AI x HBM bandwidth) for this layer
            "attainable_peak": round(min(PEAK_INT8_TOPS, cnt["ops"] / cnt["conv_bytes"] * PEAK_HBM_GBS / 1e3), 1),
            "frac_of_attainable": round(conv_tops / min(PEAK_INT8_TOPS,
                                                        cnt["ops"] / cnt["conv_bytes"] * PEAK_HBM_GBS / 1e3), 4),
            "power_limited_ceiling": ceiling,
        },
        "ms_per_step_gpu_events": round(ev_ms_per_step, 5),
        "ms_per_step_hip_graph": None if graph_ms is None else round(graph_ms, 5),
        "conv_ms": round(conv_avg, 5),
        "conv_tops": round(conv_tops, 2),
        "nominal_ops": cnt["nominal_ops"],
        "quant_pass": {
            "absmax_ms": round(absmax_avg, 5),
            "absmax_GBs": round(cnt["absmax_bytes"] / (absmax_avg * 1e-3) / 1e9, 1),
            "quantize_ms": round(quant_avg, 5),
            "quantize_GBs": round(cnt["quant_bytes"] / (quant_avg * 1e-3) / 1e9, 1),
            "absmax_cold_ms": round(absmax_cold, 5),
            "absmax_cold_GBs": round(cnt["absmax_bytes"] / (absmax_cold * 1e-3) / 1e9, 1),
            "quantize_cold_ms": round(quant_cold, 5),
            "quantize_cold_GBs": round(cnt["quant_bytes"] / (quant_cold * 1e-3) / 1e9, 1),
            "hbm_peak_GBs": PEAK_HBM_GBS,
            "note": "absmax_/quantize_ms: back-to-back launches, warm (a tensor under 256 MB may be partly "
                    "resident in the last-level cache); *_cold: one launch between two events after a 1 GiB "
                    "write evicted the last-level cache, median of 10 (dispatch latency included)",
        },
        "first_call_ms": round(first_ms, 3),
        "chained_step": {
            "ms_per_step": round(ms_chained, 5),
            "value": round(cnt["ops"] / (ms_chained * 1e-3) / 1e12, 3),
            "conv_absmax_ms": round(conv_mx_avg, 5),
            "note": "quantize + a conv that also emits the partial maxima of its output, so the next layer "
                    "needs no absmax pass (the input's maxima come from the producing layer)",
        },
    }
    if not args.no_cpu:
        cache_np = (np.zeros((spec.N, kt - 1, spec.H, spec.W, spec.Cin), np.int8) if use_cache else None)
        out["cpu_baseline"] = cpu_baseline(ci, cache_np, args.cpu_budget, args.clip)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
