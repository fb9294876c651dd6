#!/usr/bin/env python3
"""Benchmark of the W8A8 INT8 CausalConv3d hot path on one MI355X.

Default workload: the video-style chunked causal decode, input
[1,384,8,90,160] bf16 ~N(0,1).  One step, with every input resident in HBM:
    absmax + quantize over all 8 frames (one scale for every chunk),
    4 chunk convs 3x3x3 384->384 of 2 frames each (chunk 0 with causal front
    padding, chunks 1-3 with the previous chunk's 2 int8 frames as cache),
    the 1x1x1 384->192 projection over the same int8 input,
each conv with its fused FP32 rescale + bias + bf16 store.  Weight
quantization happens once at load, outside the timed region.
``--workload`` picks a single layer instead (absmax + quantize + conv).

Prints ONE JSON line.  ``value`` is INT8 TOPS of the whole step (algorithmic
conv ops / step time); the ``roofline`` object covers the dominant kernel
(the 3x3x3 conv: the four chunk launches), timed with HIP events around its
launches inside K steps run right after the timed ones, on the stream it runs
on; ``cpu_baseline`` is the CPU oracle on a bounded sample of the same
workload.

Order of the chunked run: the first call, the step untimed for 150 ms, the
per-kernel figures (each kernel on its own, warm and cold, a plain copy, the
captured step), then the W warm-up steps and the K timed steps, K steps with
events around the chunk convs, and K more steps after one second idle.  The
chip's power management needs a few tens of milliseconds of sustained load to
settle after any idle period (the steps right after it run up to ~35 %
slower), so everything timed follows that settling load without a pause, and
the after-idle figure is reported beside the headline.
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


def chunk_launches(spec):
    """The convs of one chunked-decode step, in launch order, with their
    algorithmic work: chunk c covers frames [c*F, (c+1)*F) (F = T / chunks) and
    reads the previous F frames of the same int8 input as its cache (chunk 0:
    causal front padding), then the 1x1x1 projection runs over all T frames."""
    fpc = spec.T // spec.chunks
    out = []
    for c in range(spec.chunks):
        cs = dataclasses.replace(spec, T=fpc, chunks=1, proj_cout=0, zero_cache=False, name=f"{spec.name}_chunk{c}")
        out.append(dict(name=f"chunk{c}", spec=cs, frame0=c * fpc, cache_frame0=(c - 1) * fpc if c else None,
                        **layer_counts(cs, c > 0)))
    if spec.proj_cout:
        ps = dataclasses.replace(spec, Cout=spec.proj_cout, k=(1, 1, 1), chunks=1, proj_cout=0, zero_cache=False,
                                 name=f"{spec.name}_proj")
        out.append(dict(name="proj", spec=ps, frame0=0, cache_frame0=None, **layer_counts(ps, False)))
    return out


def _events(k):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(k)]


def _make_timer(stream):
    import torch

    def timed(fn, k):
        """k back-to-back calls on the stream, bracketed by synchronize and by
        two HIP events on that stream -> (wall ms, event ms) per call."""
        e0, e1 = _events(2)
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

    def per_launch(fns, k):
        """Each of k rounds of the launches in fns between its own pair of
        events -> per-launch durations in ms (one list per launch of fns)."""
        evs = [[_events(2) for _ in fns] for _ in range(k)]
        torch.cuda.synchronize()
        for r in range(k):
            for (e0, e1), fn in zip(evs[r], fns):
                e0.record(stream)
                assert fn() == 0
                e1.record(stream)
        torch.cuda.synchronize()
        return [[evs[r][i][0].elapsed_time(evs[r][i][1]) for r in range(k)] for i in range(len(fns))]

    def cold(fn, reps=10):
        """One launch after a 1 GiB write on the same stream evicted the 256 MB
        last-level cache, between two events; median of reps."""
        import numpy as np
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        e0, e1 = _events(2)
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

    return timed, per_launch, cold


def copy_reference(timed, cold, dev, nbytes=1 << 28):
    """Read+write rate of a plain device-to-device copy of nbytes on this machine
    (torch's copy kernel), warm (back-to-back) and cold: the practical ceiling
    for a pass that both reads and writes HBM."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    def cp():
        dst.copy_(src)
        return 0
    cp()
    _, warm = timed(cp, 20)
    c = cold(cp)
    del src, dst
    return {"bytes_read_plus_written": 2 * nbytes, "warm_GBs": round(2 * nbytes / (warm * 1e-3) / 1e9, 1),
            "cold_GBs": round(2 * nbytes / (c * 1e-3) / 1e9, 1)}


def _median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def cpu_baseline_chunked(ci, budget_s=12.0):
    """The CPU oracle (as it stands) on a bounded sample of the chunked step:
    absmax + quantize over the whole input, then each chunk conv and the
    projection (conv + epilogue) at a random sample of their output positions,
    each timed and scaled to all of its positions; TOPS of the whole step."""
    import numpy as np
    import oracle

    spec = ci.spec
    wq, ws = oracle.quantize_weights(ci.w)
    wp, wps = oracle.quantize_weights(ci.w_proj)
    t0 = time.perf_counter()
    _, s, xq = oracle.act_absmax_quant(ci.x)
    t_quant = time.perf_counter() - t0
    launches = chunk_launches(spec)
    total_ops = sum(L["ops"] for L in launches)
    rng = np.random.default_rng(0)
    per_budget = max(0.5, budget_s - t_quant) / len(launches)
    t_total = t_quant
    notes = []
    for L in launches:
        ls = L["spec"]
        f0 = L["frame0"]
        x_c = np.ascontiguousarray(xq[:, f0:f0 + ls.T])
        cache = None if L["cache_frame0"] is None else np.ascontiguousarray(
            xq[:, L["cache_frame0"]:L["cache_frame0"] + ls.k[0] - 1])
        w_c, s_c, b_c = (wq, ws, ci.b) if L["name"] != "proj" else (wp, wps, ci.b_proj)
        total = ls.positions
        npos, used, t_conv = 32, 0, 0.0
        while used < total and t_conv < per_budget:
            pos = rng.integers(0, total, npos).astype(np.int64)
            t1 = time.perf_counter()
            acc = oracle.conv_acc(x_c, w_c, cache, positions=pos)
            oracle.epilogue(acc, s, s_c, b_c)
            t_conv += time.perf_counter() - t1
            used += npos
            npos = min(total - used, npos * 2) if used < total else 0
            if npos <= 0:
                break
        t_total += t_conv / used * total
        notes.append(f"{L['name']} {used} of {total} positions {t_conv:.2f} s")
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(total_ops / t_total / 1e12, 5), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "cpu_model": model, "s_per_step": round(t_total, 2),
            "sample": (f"absmax+quantize over all {spec.numel} elements ({t_quant:.2f} s); conv + epilogue at "
                       f"random output positions of each launch, scaled to all of them: " + "; ".join(notes))}


def step_series(step, stream, n):
    """Durations of n consecutive steps (an event pair around each, on the
    stream), right after the first call, then again after 1 s and after 5 s
    with the GPU idle: means over windows of 100 steps and the first 10."""
    import numpy as np
    import torch
    out = {"steps_per_phase": n}
    for phase, gap in (("from_first_call", 0.0), ("after_1s_idle", 1.0), ("after_5s_idle", 5.0)):
        time.sleep(gap)
        ev = _events(n + 1)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(n):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)]) * 1e3
        out[phase] = {"us_per_step_100_step_windows": [round(float(d[i:i + 100].mean()), 1) for i in range(0, n, 100)],
                      "us_first_10_steps": [round(float(v), 1) for v in d[:10]],
                      "us_median_last_half": round(float(np.median(d[n // 2:])), 1)}
    return out


def bench_chunked(args):
    """The chunked causal decode step (see the module docstring)."""
    import numpy as np
    import torch

    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl

    dev = "cuda:0"
    ci = wl.draw_workload(args.workload)[0]
    spec = ci.spec
    launches = chunk_launches(spec)
    step_ops = sum(L["ops"] for L in launches)
    conv3 = [L for L in launches if L["name"] != "proj"]
    proj = [L for L in launches if L["name"] == "proj"]

    x = torch.from_numpy(ci.x.view(np.int16)).to(dev).view(torch.bfloat16)
    wq, ws = ops.quantize_weights(torch.from_numpy(ci.w).to(dev))
    b = torch.from_numpy(ci.b).to(dev)
    wp, wps = ops.quantize_weights(torch.from_numpy(ci.w_proj).to(dev))
    bp = torch.from_numpy(ci.b_proj).to(dev)
    absmax = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=dev)
    xs = torch.empty((1,), dtype=torch.float32, device=dev)
    xq = torch.empty(x.shape, dtype=torch.int8, device=dev)
    y = torch.empty((spec.N, spec.T, spec.H, spec.W, spec.Cout), dtype=torch.bfloat16, device=dev)
    yp = torch.empty((spec.N, spec.T, spec.H, spec.W, spec.proj_cout), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    timed, per_launch, cold = _make_timer(stream)

    # launch arguments marshalled once; the timed loops call the C entry points
    # directly (the calls ops.* makes, without its per-call checks)
    L = ops.lib()
    P = ctypes.c_void_p
    sp = P(stream.cuda_stream)
    fx = spec.H * spec.W * spec.Cin            # int8 bytes per input frame (N = 1)
    fy = spec.H * spec.W * spec.Cout * 2       # bf16 bytes per output frame
    assert spec.N == 1
    a_absmax = (P(x.data_ptr()), x.numel(), P(absmax.data_ptr()), sp)
    a_quant = (P(x.data_ptr()), x.numel(), ctypes.c_float(1.0), P(absmax.data_ptr()), P(xs.data_ptr()),
               P(xq.data_ptr()), sp)
    conv_args = []
    for Lc in conv3:
        cs = Lc["spec"]
        cache = None if Lc["cache_frame0"] is None else P(xq.data_ptr() + Lc["cache_frame0"] * fx)
        conv_args.append((P(xq.data_ptr() + Lc["frame0"] * fx), P(xs.data_ptr()), cache, P(wq.data_ptr()),
                          P(ws.data_ptr()), P(b.data_ptr()), cs.N, cs.T, cs.H, cs.W, cs.Cin, cs.Cout, 3, 3, 3,
                          P(y.data_ptr() + Lc["frame0"] * fy), sp))
    ps = proj[0]["spec"]
    a_proj = (P(xq.data_ptr()), P(xs.data_ptr()), None, P(wp.data_ptr()), P(wps.data_ptr()), P(bp.data_ptr()),
              ps.N, ps.T, ps.H, ps.W, ps.Cin, ps.Cout, 1, 1, 1, P(yp.data_ptr()), sp)
    conv_fns = [(lambda a=a: L.qvae_causalconv3d_w8a8(*a)) for a in conv_args]

    def absmax_pass():
        return L.qvae_act_absmax(*a_absmax)

    def quant_pass():
        return L.qvae_act_quantize(*a_quant)

    def chunk_convs():
        rc = 0
        for f in conv_fns:
            rc |= f()
        return rc

    def proj_pass():
        return L.qvae_causalconv3d_w8a8(*a_proj)

    def step():
        return absmax_pass() | quant_pass() | chunk_convs() | proj_pass()

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert step() == 0
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    if args.series:
        return step_series(step, stream, args.series)

    # the step, untimed, for at least 150 ms: the clock settles under sustained
    # load after the idle start.  Then the per-kernel figures (each kernel on
    # its own, warm and cold, a plain device copy, the captured step), which
    # keep the load on until the timed steps.
    t_end = time.perf_counter() + 0.15
    settle_steps = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    pl = per_launch(conv_fns, max(5, args.steps // 4))
    per_chunk = {}
    for Lc, d in zip(conv3, pl):
        per_chunk[Lc["name"]] = {"alg_GOP": round(Lc["ops"] / 1e9, 2), "median_ms": round(_median(d), 5),
                                 "min_ms": round(min(d), 5),
                                 "TOPS_at_median": round(Lc["ops"] / (_median(d) * 1e-3) / 1e12, 1)}
    _, loop_ms = timed(chunk_convs, max(args.steps, 50))       # the 4 chunk convs back to back
    _, proj_ms = timed(proj_pass, args.steps)
    _, absmax_ms = timed(absmax_pass, args.steps)
    _, quant_ms = timed(quant_pass, args.steps)
    absmax_cold = cold(absmax_pass)
    quant_cold = cold(quant_pass)
    copy_ref = copy_reference(timed, cold, dev)

    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs = P(torch.cuda.current_stream().cuda_stream)
            L.qvae_act_absmax(*(a_absmax[:-1] + (gs,)))
            L.qvae_act_quantize(*(a_quant[:-1] + (gs,)))
            for a in conv_args:
                L.qvae_causalconv3d_w8a8(*(a[:-1] + (gs,)))
            L.qvae_causalconv3d_w8a8(*(a_proj[:-1] + (gs,)))
        g.replay()
        torch.cuda.synchronize()
        _, graph_ms = timed(lambda: (g.replay(), 0)[1], args.steps)
    except Exception as exc:  # an extra figure, never the headline
        print(f"graph replay skipped: {exc}", file=sys.stderr)

    # the headline: W warm-up steps, then exactly K timed steps
    for _ in range(args.warmup):
        step()
    ms_per_step, ev_ms_per_step = timed(step, args.steps)
    value = step_ops / (ms_per_step * 1e-3) / 1e12

    # right after them, K more steps, each with an event pair around its four
    # chunk convs (same stream): the dominant kernel's average launch inside
    # the steps.  (An event record between two kernels costs the queue a few
    # microseconds, so the headline steps above carry none.)
    chunk_ev = [_events(2) for _ in range(args.steps)]
    torch.cuda.synchronize()
    rc = 0
    for k in range(args.steps):
        rc |= absmax_pass() | quant_pass()
        chunk_ev[k][0].record(stream)
        rc |= chunk_convs()
        chunk_ev[k][1].record(stream)
        rc |= proj_pass()
    torch.cuda.synchronize()
    assert rc == 0
    chunks_ms = sum(a.elapsed_time(b) for a, b in chunk_ev) / args.steps
    conv_avg = chunks_ms / len(conv_fns)                       # average launch inside the timed steps
    ops_avg = sum(Lc["ops"] for Lc in conv3) / len(conv3)      # average algorithmic ops per launch
    bytes_avg = sum(Lc["conv_bytes"] for Lc in conv3) / len(conv3)
    conv_tops = ops_avg / (conv_avg * 1e-3) / 1e12

    # the same K steps after one second with the GPU idle (the clock's transient)
    time.sleep(1.0)
    idle_ms, _ = timed(step, args.steps)

    # output check after the timed loops: the chunked output equals one
    # unchunked pass over all frames (no stale outputs counted)
    ref_y = ops.causalconv3d_w8a8(xq, xs, wq, ws, b)
    ref_p = ops.causalconv3d_w8a8(xq, xs, wp, wps, bp)
    torch.cuda.synchronize()
    assert torch.equal(ref_y.view(torch.int16), y.view(torch.int16))
    assert torch.equal(ref_p.view(torch.int16), yp.view(torch.int16))

    conv_src = os.path.join(ROOT, "w8a8_int8_quantized_act_amd", "csrc", "qvae_conv.hip")
    traffic = read_traffic(args.workload, conv_src)
    numel = spec.numel
    attainable = min(PEAK_INT8_TOPS, ops_avg / bytes_avg * PEAK_HBM_GBS / 1e3)
    pb = proj[0]["conv_bytes"]
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
            "workload": args.workload,
            "layer": (f"CausalConv3d 3x3x3 Cin=Cout={spec.Cin} input [{spec.N},{spec.Cin},{spec.T},{spec.H},"
                      f"{spec.W}] bf16 channels-last as {spec.chunks} chunks of {spec.T // spec.chunks} frames "
                      f"(chunks 1-{spec.chunks - 1} with the previous chunk's int8 frames as cache) + 1x1x1 "
                      f"{spec.Cin}->{spec.proj_cout} projection on the same int8 input"),
            "global_batch": spec.N,
            "parallelism": "single GPU",
            "step": ("absmax + quantize over all frames (one scale), 4 chunk convs, projection conv; each conv "
                     "with fused FP32 rescale, bias, bf16 store"),
            "alg_GOP_per_step": round(step_ops / 1e9, 2),
        },
        "roofline": {
            "kernel": "k_conv_igemm 3x3x3 (the 4 chunk-conv launches of a step)",
            "bound": "mfma",
            "achieved": round(conv_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS",
            "op_kind": "INT8 ops, algorithmic count (structurally zero front-pad taps excluded)",
            "frac": round(conv_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_launch": ops_avg,
            "avg_launch_ms": round(conv_avg, 5),
            "per_launch": per_chunk,
            "algorithmic_bytes_per_launch": bytes_avg,
            "ai_ops_per_byte": round(ops_avg / bytes_avg, 1),
            "attainable_peak": round(attainable, 1),
            "frac_of_attainable": round(conv_tops / attainable, 4),
            "note": ("achieved = average algorithmic ops per chunk launch / average launch time of the 4 chunk "
                     "convs inside K steps run right after the timed ones (one HIP event pair around the 4 "
                     "launches of each step, on the launch stream); per_launch: one event pair around each "
                     "launch, run before the timed steps, median and min over the rounds; chunk_loop_ms: the 4 "
                     "launches back to back, before the timed steps"),
            "chunk_loop_ms": round(loop_ms, 5),
        },
        "ms_per_step_gpu_events": round(ev_ms_per_step, 5),
        "ms_per_step_hip_graph": None if graph_ms is None else round(graph_ms, 5),
        "ms_per_step_after_1s_idle": round(idle_ms, 5),
        "settle_steps": settle_steps,
        "chunk_convs_ms": round(chunks_ms, 5),
        "projection": {"ms": round(proj_ms, 5), "alg_GOP": round(proj[0]["ops"] / 1e9, 2),
                       "TOPS": round(proj[0]["ops"] / (proj_ms * 1e-3) / 1e12, 1),
                       "GBs": round(pb / (proj_ms * 1e-3) / 1e9, 1),
                       "frac_of_hbm": round(pb / (proj_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "quant_pass": {
            "elements": numel,
            "absmax_ms": round(absmax_ms, 5),
            "absmax_GBs": round(2 * numel / (absmax_ms * 1e-3) / 1e9, 1),
            "quantize_ms": round(quant_ms, 5),
            "quantize_GBs": round(3 * numel / (quant_ms * 1e-3) / 1e9, 1),
            "absmax_cold_ms": round(absmax_cold, 5),
            "absmax_cold_GBs": round(2 * numel / (absmax_cold * 1e-3) / 1e9, 1),
            "quantize_cold_ms": round(quant_cold, 5),
            "quantize_cold_GBs": round(3 * numel / (quant_cold * 1e-3) / 1e9, 1),
            "hbm_peak_GBs": PEAK_HBM_GBS,
            "reference_copy_256MiB": copy_ref,
            "note": "absmax 2 B and quantize 3 B per element; *_ms: back-to-back launches (warm); *_cold: one "
                    "launch after a 1 GiB write evicted the last-level cache, median of 10; reference_copy: a "
                    "plain device copy on the same box (read + written bytes), the ceiling for a read+write pass",
        },
        "first_call_ms": round(first_ms, 3),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_chunked(ci, args.cpu_budget)
    return out


def bench_layer(args):
    """One layer (``--workload``, ``--level``): absmax + quantize + conv."""
    import numpy as np
    import torch

    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl

    dev = "cuda:0"
    ci = wl.draw_workload(args.workload, only=args.level)[-1]
    if args.frames and args.frames != ci.spec.T:
        spec_t = dataclasses.replace(ci.spec, T=args.frames, name=f"{ci.spec.name}_t{args.frames}")
        ci = wl.draw_conv(spec_t, torch.Generator().manual_seed(
            1000 * wl.WORKLOADS[args.workload].seed + 10 * args.level + args.frames))
    spec = ci.spec
    kt = spec.k[0]
    use_cache = spec.zero_cache
    variant = (ci.spec.T != wl.WORKLOADS[args.workload].convs[args.level].T or args.clip != 1.0
               or (use_cache and args.cache == "data"))
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
    timed, per_launch, cold = _make_timer(stream)

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

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    assert step() == 0
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    if cache is not None and args.cache == "data":
        # a cache of data instead of zeros: both cache frames hold the layer's
        # own int8 codes (the distribution a real previous chunk would have)
        cache.copy_(xq.expand(spec.N, kt - 1, spec.H, spec.W, spec.Cin) if spec.T == 1
                    else xq[:, :1].expand(spec.N, kt - 1, spec.H, spec.W, spec.Cin))
    # the conv back to back in rounds of K launches until at least 150 ms of
    # sustained load have passed (the clock settles after the idle start); the
    # last round is the conv's figure.  The other per-kernel figures follow,
    # then the W warm-up and K timed steps.
    t_end = time.perf_counter() + 0.15
    rounds = 0
    while True:
        _, conv_avg = timed(conv_pass, args.steps)
        rounds += 1
        if time.perf_counter() >= t_end:
            break
    pl = per_launch([conv_pass], max(5, args.steps // 4))[0]
    _, absmax_avg = timed(absmax_pass, args.steps)
    _, quant_avg = timed(quant_pass, args.steps)
    _, conv_mx_avg = timed(conv_absmax_pass, args.steps)
    ms_chained, _ = timed(step_chained, args.steps)
    conv_tops = cnt["ops"] / (conv_avg * 1e-3) / 1e12
    absmax_cold = cold(absmax_pass)
    quant_cold = cold(quant_pass)

    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gs = P(torch.cuda.current_stream().cuda_stream)
            L.qvae_act_absmax(*(a_absmax[:-1] + (gs,)))
            L.qvae_act_quantize(*(a_quant[:-1] + (gs,)))
            L.qvae_causalconv3d_w8a8(*(a_conv[:-1] + (gs,)))
        g.replay()
        torch.cuda.synchronize()
        _, graph_ms = timed(lambda: (g.replay(), 0)[1], args.steps)
    except Exception as exc:  # graphs are an extra figure, never the headline
        print(f"graph replay skipped: {exc}", file=sys.stderr)

    for _ in range(args.warmup):
        step()
    ms_per_step, ev_ms_per_step = timed(step, args.steps)
    value = cnt["ops"] / (ms_per_step * 1e-3) / 1e12

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
    if use_cache and args.cache == "data":
        wl_name += " cache=data"
    attainable = min(PEAK_INT8_TOPS, cnt["ops"] / cnt["conv_bytes"] * PEAK_HBM_GBS / 1e3)
    cache_txt = ""
    if use_cache:
        cache_txt = ", explicit 2-frame cache of " + ("the layer's own int8 codes" if args.cache == "data"
                                                      else "zeros")
    else:
        cache_txt = ", causal front padding"
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
                     f"input [{spec.N},{spec.Cin},{spec.T},{spec.H},{spec.W}] bf16 channels-last" + cache_txt,
            "global_batch": spec.N,
            "parallelism": "single GPU",
            "step": "absmax + quantize + implicit-GEMM conv (fused FP32 rescale, bias, bf16 store)",
            "zero_share_of_K": round(zero_share_of_k(spec.T, kt, use_cache and args.cache == "zero"), 4),
        },
        "roofline": {
            "kernel": "k_conv_igemm",
            "bound": "mfma" if attainable >= PEAK_INT8_TOPS else "hbm",
            "achieved": round(conv_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS",
            "op_kind": "INT8 ops, algorithmic count (structurally zero front-pad taps excluded)",
            "frac": round(conv_tops / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "algorithmic_ops_per_launch": cnt["ops"],
            "avg_launch_ms": round(conv_avg, 5),
            "per_launch_median_ms": round(_median(pl), 5),
            "per_launch_min_ms": round(min(pl), 5),
            "algorithmic_bytes_per_launch": cnt["conv_bytes"],
            "ai_ops_per_byte": round(cnt["ops"] / cnt["conv_bytes"], 1),
            "attainable_peak": round(attainable, 1),
            "frac_of_attainable": round(conv_tops / attainable, 4),
            "note": ("achieved = algorithmic ops / average launch time of K back-to-back launches (HIP events on "
                     "the launch stream), the last of settle_rounds such rounds run for at least 150 ms from the "
                     "start; per_launch_*: one event pair around each launch"),
            "settle_rounds": rounds,
        },
        "ms_per_step_gpu_events": round(ev_ms_per_step, 5),
        "ms_per_step_hip_graph": None if graph_ms is None else round(graph_ms, 5),
        "conv_ms": round(conv_avg, 5),
        "conv_tops": round(conv_tops, 2),
        "nominal_ops": cnt["nominal_ops"],
        "quant_pass": {
            "elements": spec.numel,
            "absmax_ms": round(absmax_avg, 5),
            "absmax_GBs": round(cnt["absmax_bytes"] / (absmax_avg * 1e-3) / 1e9, 1),
            "quantize_ms": round(quant_avg, 5),
            "quantize_GBs": round(cnt["quant_bytes"] / (quant_avg * 1e-3) / 1e9, 1),
            "absmax_cold_ms": round(absmax_cold, 5),
            "absmax_cold_GBs": round(cnt["absmax_bytes"] / (absmax_cold * 1e-3) / 1e9, 1),
            "quantize_cold_ms": round(quant_cold, 5),
            "quantize_cold_GBs": round(cnt["quant_bytes"] / (quant_cold * 1e-3) / 1e9, 1),
            "hbm_peak_GBs": PEAK_HBM_GBS,
            "note": "*_ms: back-to-back launches, warm (a tensor under 256 MB may be partly resident in the "
                    "last-level cache); *_cold: one launch after a 1 GiB write evicted the last-level cache, "
                    "median of 10 (dispatch latency included)",
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
        cache_np = None
        if use_cache:
            cache_np = (np.zeros((spec.N, kt - 1, spec.H, spec.W, spec.Cin), np.int8) if args.cache == "zero"
                        else cache.cpu().numpy())
        out["cpu_baseline"] = cpu_baseline(ci, cache_np, args.cpu_budget, args.clip)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="video_384_t8_chunked")
    ap.add_argument("--level", type=int, default=0, help="layer index inside a level sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cache", choices=("zero", "data"), default="zero",
                    help="layers with an explicit cache: all-zero codes (the workload) or the layer's own codes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--first-calls", action="store_true",
                    help="only time the first and second layer step at each resolution of the level sweeps")
    ap.add_argument("--init", action="store_true", help="with --first-calls: call qvae_init first")
    ap.add_argument("--frames", type=int, default=0,
                    help="a multi-frame variant: the layer's shape with T frames (redrawn, same recipe)")
    ap.add_argument("--clip", type=float, default=1.0,
                    help="activation and weight clip ratio in (0, 1] (the page fixes 1.0)")
    ap.add_argument("--decoder", action="store_true",
                    help="only time the decoder's 28 residual-block convs per preset (W8A8 vs native bf16)")
    ap.add_argument("--out-h", type=int, default=1024)
    ap.add_argument("--out-w", type=int, default=1024)
    ap.add_argument("--series", type=int, default=0,
                    help="chunked workload only: the duration of each of N steps from the first call on, then of "
                         "N more after 1 s and after 5 s idle (the clock's transient), instead of the bench line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the W8A8 CausalConv3d path here runs on a single MI355X "
              "(multi-GPU sharding is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
    if args.first_calls:
        first_calls(with_init=args.init)
        return
    if args.decoder:
        decoder_stack(args)
        return

    import torch

    from w8a8_int8_quantized_act_amd import ops
    from w8a8_int8_quantized_act_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ops.lib()
    chunked = wl.WORKLOADS[args.workload].convs[0].chunks > 1
    if chunked and (args.frames or args.clip != 1.0 or args.level):
        print("--frames, --clip and --level apply to single-layer workloads", file=sys.stderr)
        sys.exit(2)
    if args.series and not chunked:
        print("--series applies to the chunked workload", file=sys.stderr)
        sys.exit(2)
    out = bench_chunked(args) if chunked else bench_layer(args)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
