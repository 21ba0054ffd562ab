#!/usr/bin/env python3
"""Benchmark of the routed-expert FFN (qwen3_5-MoE 35B-A3B shapes) on one MI355X.

Headline workload: decode, 8 independent rows through 40 distinct MoE layer
weight sets (hidden 2048, 256 experts, top-8, expert intermediate 512, shared
expert 512), 4-bit affine g64 weights everywhere (~18 GB packed, so the ~4 GB
of expert bytes a step touches cannot stay in cache). One step is one pass of
the whole hot path over one batch: for each of the 40 layers, route (logits,
top-8, weights, shared gate) then the decode experts (gate/up + SwiGLU, down,
combine). Inputs are resident in HBM before the timed region; each step takes
a fresh set of activations (4 sets rotate).

Prints ONE JSON line. `value` is MoE-layer tokens/s: rows x layers per
second. `roofline` is the dominant kernel (decode gate/up) timed live with
HIP events on its stream: algorithmic bytes per launch (the packed gate/up
bytes of the unique experts the launch reads, plus x in and h out) over its
mean duration. `workloads` holds the other shapes on their own binding
rooflines: one decode row and the mixed 3-bit layers (1 and 8 rows), both
over 40 distinct layers, and the two prompt chunks (512 rows 4-bit against
HBM, 2048 rows W4A16 Zipf against MFMA), each chunk timed over 4 rotating
weight sets. `cpu_baseline` is the FP64 oracle timed on bounded samples on
the host cores (all of them, and one thread).

Per-kernel times come from HIP events recorded inside the library's launches
on the bench stream; the launches of a timed pass are queued behind a GPU-side
sleep so that the kernels run back to back (host launch gaps do not count).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
METRIC = "MoE-layer tokens/s; decode HBM GB/s and prefill MFMA TFLOPS as % of peak"
N_PREFILL_SETS = 4     # weight sets a prompt-chunk timing rotates through


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scale_entry_bytes(fmt):
    """Packed bytes per group: affine scale + bias 4, symmetric 2, MXFP4 1."""
    return {0: 4, 1: 2, 3: 1}[fmt.mode]


def expert_bytes(spec, fmt, inter):
    """Packed bytes of one expert: gate/up and down (codes + scale words)."""
    scb = scale_entry_bytes(fmt)
    gu = 2 * inter * spec.hidden * fmt.bits // 8 + 2 * inter * (spec.hidden // fmt.group) * scb
    dn = spec.hidden * inter * fmt.bits // 8 + spec.hidden * (inter // fmt.group) * scb
    return gu, dn


def fmt_name(f):
    """Short text name of a weight format, e.g. 'affine 4-bit g64 bf16 scale/bias'."""
    dt = "bf16" if f.scale_dtype == 0 else "fp16"
    if f.mode == 3:
        return f"mxfp4 e2m1 g{f.group} e8m0 scale"
    if f.mode == 2:
        return f"dense {dt}"
    if f.mode == 1:
        return f"symmetric {f.bits}-bit g{f.group} {dt} scale"
    return f"affine {f.bits}-bit g{f.group} {dt} scale/bias"


def router_bytes(spec):
    f, g = spec.router, spec.gate_row
    scb = scale_entry_bytes(f)
    r = spec.n_experts * spec.hidden * f.bits // 8 + spec.n_experts * (spec.hidden // f.group) * scb
    if g.mode == 2:
        gr = spec.hidden * 2
    else:
        gr = spec.hidden * g.bits // 8 + (spec.hidden // g.group) * (4 if g.mode == 0 else 2)
    return r + gr


def build_layers(spec, n_layers, B, to_abi, synth, keep_host=0):
    desc = B.layer_desc(*to_abi.desc_args(spec))
    layers = [None] * n_layers
    host_keep = {}
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=6) as ex:
        futs = {ex.submit(synth.make_layer, spec, l): l for l in range(n_layers)}
        done = 0
        for fut in list(futs):
            l = futs[fut]
            Lh = fut.result()
            layers[l] = B.pack_layer(desc, to_abi.tensors(Lh))
            if l < keep_host:
                host_keep[l] = Lh
            del Lh
            done += 1
            if done % 10 == 0 or done == n_layers:
                log(f"[bench] packed {done}/{n_layers} layers ({time.time() - t0:.1f}s)")
    return layers, host_keep


def cpu_model():
    """The host CPU's model name (the first `model name` of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads():
    """Threads the oracle's BLAS may use on this host: the CPUs this process
    may run on, capped by OMP_NUM_THREADS when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _blas_threads(n):
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:  # pragma: no cover
        return contextlib.nullcontext()


def cpu_decode_baseline(spec, Lh, rows, threads, budget_s=12.0):
    """The FP64 oracle (as it stands), per-row form, on one layer x up to
    `rows` rows, numpy's BLAS on `threads` threads; experts are dequantised
    on first use inside the timed region (part of the oracle's work)."""
    import oracle.moe_oracle as O
    import synth
    xb = synth.make_x(spec, 0, rows, rep=0)
    with _blas_threads(threads):
        t0 = time.perf_counter()
        done = 0
        dense = O.DenseExperts(Lh, cache=True)
        for r in range(rows):
            O.moe_forward(Lh, xb[r:r + 1], dense)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{done} decode rows through the first layer of {spec.name}, per-row fp64 "
                       f"form, experts dequantised on first use, {dt:.1f} s")


def cpu_prefill_baseline(spec, Lh, xb, threads):
    """The FP64 oracle's expert-major form (each expert's rows as one matrix
    product) on a whole prompt chunk, BLAS on `threads` threads; the timed
    region includes dequantising every touched expert."""
    import oracle.moe_oracle as O
    with _blas_threads(threads):
        t0 = time.perf_counter()
        O.moe_forward(Lh, xb, form="expert_major")
        dt = time.perf_counter() - t0
    return dict(value=xb.shape[0] / dt, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"one {xb.shape[0]}-row chunk of {spec.name}, expert-major fp64 form, {dt:.1f} s")


class GpuSleep:
    """Queues a GPU-side wait (torch.cuda._sleep) long enough for the host to
    enqueue a timed pass behind it, so the pass's kernels run back to back."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 20_000_000
        with torch.cuda.stream(stream):
            torch.cuda._sleep(n // 10)
            e0.record(stream)
            torch.cuda._sleep(n)
            e1.record(stream)
            torch.cuda.synchronize()
        self.cycles_per_ms = n / max(e0.elapsed_time(e1), 1e-3)

    def __call__(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


def event_pass(torch, stream, sleeper, n_passes, n_ev, enqueue):
    """Runs `enqueue(events)` n_passes times, each queued behind a GPU sleep of
    twice the host's measured enqueue time, with n_ev timing events per pass.
    Returns the events and the host enqueue time of one pass (ms)."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n_passes)]
    with torch.cuda.stream(stream):
        for es in evs:              # torch creates the HIP event on first record
            for e in es:
                e.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        enqueue(None)
        t_enq = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        for es in evs:
            sleeper(2.0 * t_enq + 0.5)
            enqueue(es)
        torch.cuda.synchronize()
    return evs, t_enq


def prefill_algorithmic(spec, ids):
    """Algorithmic bytes and flops of one prompt chunk: the packed bytes of
    the unique routed experts its ids select plus the shared expert, router
    and gate row, x in and y out (fp32); flops 2*3*H*I per (row, slot), the
    shared expert's per row, and the router's 2*(E+1)*H per row."""
    R, k = ids.shape
    H, E = spec.hidden, spec.n_experts
    uniq = len(np.unique(ids[(ids >= 0) & (ids < E)]))
    gu_b, dn_b = expert_bytes(spec, spec.routed, spec.inter)
    sgu_b, sdn_b = expert_bytes(spec, spec.shared, spec.shared_inter)
    act_b = 2
    nbytes = uniq * (gu_b + dn_b) + sgu_b + sdn_b + router_bytes(spec) + R * H * act_b + R * H * 4
    f_routed = 2.0 * 3 * H * spec.inter * R * k
    f_shared = 2.0 * 3 * H * spec.shared_inter * R
    f_router = 2.0 * (E + 1) * H * R
    return dict(bytes=nbytes, unique_experts=uniq, flop_routed=f_routed, flop_shared=f_shared,
                flop_router=f_router)


def bench_prefill(cfg, steps, warmup, B, to_abi, synth, torch, dev, stream, sleeper,
                  n_sets=N_PREFILL_SETS, windows=False, keep_host=False):
    """One prompt chunk through one layer: route + grouped experts. The timed
    replays rotate through n_sets distinct weight sets (each with its own
    activations), so the touched experts come from HBM, not the MALL. Whole
    chunks are timed as HIP graph replays; per-phase times from events inside
    the library's launches, queued behind a GPU sleep. cfg: a config id or a
    ConfigSpec."""
    spec = synth.CONFIGS[cfg] if isinstance(cfg, int) else cfg
    R, k, H, E = spec.rows[0], spec.top_k, spec.hidden, spec.n_experts
    desc = B.layer_desc(*to_abi.desc_args(spec))
    layers, biases, xs, host = [], [], [], None
    for l in range(n_sets):
        Lh = synth.make_layer(spec, l)
        layers.append(B.pack_layer(desc, to_abi.tensors(Lh)))
        biases.append(torch.from_numpy(Lh.logit_bias).to(dev) if Lh.logit_bias is not None else None)
        xs.append(torch.from_numpy(synth.make_x(spec, l, R, rep=0).view(np.int16)).to(dev))
        if keep_host and l == 0:
            host = Lh
        del Lh
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    p = torch.empty((R, k), dtype=torch.float32, device=dev)
    sg = torch.empty((R,), dtype=torch.float32, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = B.new_workspace(layers[0], R, True, dev, stream=stream)

    def chunk(l, events=None):
        B.route(layers[l], xs[l], biases[l], taps=dict(events=events[:2]) if events else None,
                out=(ids, p, sg), ws=ws, stream=stream)
        B.experts(layers[l], xs[l], ids, p, sg, True, ws=ws, y=y,
                  taps=dict(events=events[2:]) if events else None, stream=stream)

    # algorithmic work of each weight set's chunk
    alg = []
    with torch.cuda.stream(stream):
        for l in range(n_sets):
            chunk(l)
            stream.synchronize()
            alg.append(prefill_algorithmic(spec, ids.cpu().numpy()))
        graphs = []
        for l in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                chunk(l)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            graphs[i % n_sets].replay()
        t1.record(stream)
        torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    mean = lambda key: float(np.mean([alg[i % n_sets][key] for i in range(steps)]))
    nbytes = mean("bytes")
    f_rt, f_sh, f_ro = mean("flop_routed"), mean("flop_shared"), mean("flop_router")
    # per phase: route | sort | gate/up GEMMs | down GEMMs | combine
    evs, _ = event_pass(torch, stream, sleeper, steps, 10,
                        lambda es, c=[0]: (chunk(c[0] % n_sets, es), c.__setitem__(0, c[0] + 1)))
    ph = np.zeros(5)
    for es in evs:
        for i in range(5):
            ph[i] += es[2 * i].elapsed_time(es[2 * i + 1])
    ph = ph / steps * 1e3
    tf = lambda f, t: f / (t * 1e-6) / 1e12
    cnt = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    res = {
        "workload": spec.name, "rows": R, "weight_sets": n_sets, "us_per_chunk": us,
        "tokens_per_s": R / (us * 1e-6),
        "algorithmic_bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9,
        "frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "flop": f_rt + f_sh + f_ro, "tflops": tf(f_rt + f_sh + f_ro, us),
        "frac_mfma": tf(f_rt + f_sh + f_ro, us) / MFMA_F16_PEAK_TFLOPS,
        "tflops_without_shared_flops": tf(f_rt + f_ro, us),
        "phase_us": {"route": ph[0], "sort": ph[1], "gate_up": ph[2], "down": ph[3], "combine": ph[4]},
        "gate_up_tflops": tf(2 * (f_rt + f_sh) / 3, ph[2]), "down_tflops": tf((f_rt + f_sh) / 3, ph[3]),
        "mean_unique_experts": mean("unique_experts"),
        "rows_per_expert": {"max": int(cnt.max()), "mean": float(cnt.mean()),
                            "empty": int((cnt == 0).sum())},
    }
    # the exact chunk form (moe_forward_exact: every row with its one-row
    # decode step's bits), timed as graph replays over the same weight sets
    xws = B.new_workspace(layers[0], R, B.MOE_WS_EXACT, dev, stream=stream)
    y2 = torch.empty_like(y)
    with torch.cuda.stream(stream):
        B.forward_exact(layers[0], xs[0], biases[0], ws=xws, out=(ids, p, sg), y=y2, stream=stream)
        torch.cuda.synchronize()
        xgraphs = []
        for l in range(n_sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                B.forward_exact(layers[l], xs[l], biases[l], ws=xws, out=(ids, p, sg), y=y2, stream=stream)
            xgraphs.append(g)
        for i in range(warmup):
            xgraphs[i % n_sets].replay()
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(steps):
            xgraphs[i % n_sets].replay()
        t1.record(stream)
        torch.cuda.synchronize()
    res["exact_us_per_chunk"] = t0.elapsed_time(t1) / steps * 1e3
    res["exact_over_grouped"] = res["exact_us_per_chunk"] / us
    del xgraphs, xws
    if windows:
        # the same chunk through the decode step's arithmetic in 16-row windows
        # (moe_forward_windows: same bits however the prompt is cut), eager
        wws = B.new_workspace(layers[0], 16, False, dev, stream=stream)
        with torch.cuda.stream(stream):
            B.forward_windows(layers[0], xs[0], biases[0], ws=wws, out=(ids, p, sg), y=y, stream=stream)
            torch.cuda.synchronize()
            t0.record(stream)
            for i in range(3):
                B.forward_windows(layers[i % n_sets], xs[i % n_sets], biases[i % n_sets], ws=wws,
                                  out=(ids, p, sg), y=y, stream=stream)
            t1.record(stream)
            torch.cuda.synchronize()
        res["windows_us_per_chunk"] = t0.elapsed_time(t1) / 3 * 1e3
    log(f"[bench] prefill {spec.name} ({n_sets} weight sets): {us:.1f} us/chunk, "
        f"{res['tokens_per_s']:.0f} tokens/s, {res['gbs']:.0f} GB/s ({100 * res['frac_hbm']:.1f}% of HBM), "
        f"{res['tflops']:.1f} TFLOP/s ({100 * res['frac_mfma']:.1f}% of f16 MFMA); "
        + ", ".join(f"{k_} {v:.1f}" for k_, v in res["phase_us"].items())
        + f"; exact form {res['exact_us_per_chunk']:.1f} us/chunk ({res['exact_over_grouped']:.2f}x grouped)"
        + (f"; 16-row windows {res['windows_us_per_chunk']:.1f} us/chunk" if windows else ""))
    del graphs, ws
    return res, host


def bench_decode(spec, layers, R, steps, warmup, B, synth, torch, dev, stream, sleeper,
                 graph=True, tag="", sample_clock=False):
    """Decode: R rows through every layer of `layers` (route, then the decode
    experts), 4 activation sets rotating. Whole steps are timed as HIP graph
    replays; per-kernel times from events inside the library's launches."""
    L, k, H = len(layers), spec.top_k, spec.hidden
    NX = 4
    xs = [[torch.from_numpy(synth.make_x(spec, l, R, rep=s).view(np.int16)).to(dev)
           for s in range(NX)] for l in range(L)]
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    p = torch.empty((R, k), dtype=torch.float32, device=dev)
    sg = torch.empty((R,), dtype=torch.float32, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = B.new_workspace(layers[0], R, False, dev, stream=stream)

    def step(s, events=None):
        for l in range(L):
            x = xs[l][s % NX]
            rt = dict(events=events[6 * l:6 * l + 2]) if events is not None else None
            B.route(layers[l], x, taps=rt, out=(ids, p, sg), ws=ws, stream=stream)
            tp = dict(events=events[6 * l + 2:6 * l + 6]) if events is not None else None
            B.experts(layers[l], x, ids, p, sg, False, ws=ws, y=y, taps=tp, stream=stream)

    # unique experts per (layer, x set): algorithmic bytes
    uniq = np.zeros((L, NX), np.int64)
    with torch.cuda.stream(stream):
        for l in range(L):
            for s in range(NX):
                B.route(layers[l], xs[l][s], out=(ids, p, sg), ws=ws, stream=stream)
                stream.synchronize()
                uniq[l, s] = len(np.unique(ids.cpu().numpy()))
    gu_b, dn_b = expert_bytes(spec, spec.routed, spec.inter)
    sgu_b, sdn_b = expert_bytes(spec, spec.shared, spec.shared_inter)
    x_b, y_b = R * H * 2, R * H * 4
    h_b = R * (k + 1) * max(spec.inter, spec.shared_inter) * 4
    gu_launch_bytes = uniq * gu_b + sgu_b + x_b + h_b            # per gate/up launch
    step_bytes = (uniq * (gu_b + dn_b) + sgu_b + sdn_b + router_bytes(spec) + x_b + y_b).sum(0)

    graphs = None
    if graph:
        try:
            graphs = []
            for s in range(NX):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(s)
                graphs.append(g)
        except Exception as e:  # graph capture unavailable: time eager launches
            log(f"[bench] graph capture failed ({e}); timing eager launches")
            graphs = None
    run = (lambda s: graphs[s % NX].replay()) if graphs else (lambda s: step(s))
    with torch.cuda.stream(stream):
        for s in range(warmup):
            run(s)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for s in range(steps):
            run(s)
        t1.record(stream)
        torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    mean_step_bytes = float(np.mean([step_bytes[s % NX] for s in range(steps)]))
    # per-step spread, from a separate pass with an event between steps
    with torch.cuda.stream(stream):
        se = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        se[0].record(stream)
        for s in range(steps):
            run(s)
            se[s + 1].record(stream)
        torch.cuda.synchronize()
    per_step = np.array([se[i].elapsed_time(se[i + 1]) for i in range(steps)])
    spread = {q: float(np.percentile(per_step, v)) * 1e3 / L for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}
    clock = None
    if sample_clock:
        # shader clock sampled from sysfs while ~0.2 s of steps replay
        reps = max(1, int(200.0 / max(ms_step, 1e-3)))
        clock = sampled_sclk(lambda: [run(s) for s in range(reps)], torch, stream)

    # per kernel: events around route, gate/up, down + combine of every layer
    nk = max(1, min(steps, 20))
    evs, t_enq = event_pass(torch, stream, sleeper, nk, 6 * L,
                            lambda es, c=[0]: (step(c[0], es), c.__setitem__(0, c[0] + 1)))
    dur = np.zeros(3)
    gu_bytes_sum = 0.0
    for s in range(nk):
        e = evs[s]
        for l in range(L):
            for i in range(3):
                dur[i] += e[6 * l + 2 * i].elapsed_time(e[6 * l + 2 * i + 1])
            gu_bytes_sum += gu_launch_bytes[l, (s + 1) % NX]
    n_launch = nk * L
    kus = dur / n_launch * 1e3
    gu_bytes = gu_bytes_sum / n_launch
    achieved = gu_bytes / (kus[1] * 1e-6) / 1e9
    res = {
        "workload": spec.name, "rows": R, "layers": L, "ms_per_step": ms_step,
        "us_per_layer": ms_step * 1e3 / L, "us_per_layer_spread": spread,
        "tokens_per_s": R * L / (ms_step / 1e3),
        "algorithmic_bytes_per_step": mean_step_bytes,
        "gbs": mean_step_bytes / ms_step / 1e6, "frac_hbm": mean_step_bytes / ms_step / 1e6 / HBM_PEAK_GBS,
        "kernel_us": {"route": kus[0], "decode_gateup": kus[1], "decode_down_combine": kus[2]},
        "gateup_bytes_per_launch": gu_bytes, "gateup_gbs": achieved,
        "mean_unique_experts": float(uniq.mean()),
        "timing": "hip graph replay" if graphs else "eager",
    }
    if clock is not None:
        res["sclk_mhz"] = clock
    log(f"[bench] decode {tag or spec.name} rows={R} layers={L}: {res['us_per_layer']:.2f} us/layer, "
        f"{res['tokens_per_s']:.0f} tokens/s, step HBM {res['gbs']:.0f} GB/s "
        f"({100 * res['frac_hbm']:.1f}%); route {kus[0]:.2f}, gate/up {kus[1]:.2f} ({achieved:.0f} GB/s), "
        f"down+combine {kus[2]:.2f} us")
    del graphs, ws
    return res


def kernel_source_hash():
    """sha256 over the decode kernel sources: a stored counter figure applies
    only to the kernel it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "moe_kernels.h", "moe_launch.h"):
        with open(os.path.join(ROOT, "quantized_routed_expert_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE passes, scaled by the copy-kernel factors),
    or None when the summary is absent or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_decode-8rows-40layers_pmc.md")
    try:
        with open(path) as fh:
            kv = dict(l.strip("- \n").split(": ", 1) for l in fh if l.startswith("- ") and ": " in l)
        if kv.get("source_sha256") != kernel_source_hash():
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration():
    """A plain copy of known size (3 x 1 GiB), for scaling the HBM counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n}), flush=True)


def read_sclk():
    """Current shader clock in MHz from the amdgpu sysfs table (the level
    marked '*'), or None where no table is readable."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if "*" in line:
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
    return None


def sampled_sclk(work, torch, stream):
    """Samples read_sclk() every ~2 ms on a host thread while `work` enqueues
    and the GPU runs it; min / median / max MHz, or the reason there is none."""
    import threading
    vals, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_sclk()
            if v is None:
                return
            vals.append(v)
            time.sleep(0.002)

    th = threading.Thread(target=sampler)
    th.start()
    with torch.cuda.stream(stream):
        work()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return {"note": "no readable pp_dpm_sclk on this host"}
    return {"min": min(vals), "median": float(np.median(vals)), "max": max(vals), "samples": len(vals)}


def mfma_ceiling(torch, dev, stream):
    """Dense fp16 MFMA rate measured with back-to-back 32x32x16 MFMAs on every
    SIMD (libmoe_ceilings.so, built beside libmoe.so), TFLOP/s."""
    import ctypes as C
    path = os.path.join(ROOT, "quantized_routed_expert_fp32_amd", "libmoe_ceilings.so")
    if not os.path.exists(path):
        return None
    lib = C.CDLL(path)
    lib.moe_ceiling_mfma_f16.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                         C.POINTER(C.c_double)]
    lib.moe_ceiling_mfma_f16.restype = C.c_int
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 8 * n_cu                    # 8 waves per CU: two per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    tf = C.c_double(0.0)
    st = lib.moe_ceiling_mfma_f16(blocks, 2000, 10, C.c_void_p(out.data_ptr()),
                                  C.c_void_p(stream.cuda_stream), C.byref(tf))
    if st != 0:
        raise RuntimeError(f"moe_ceiling_mfma_f16 failed: hipError {st}")
    return tf.value


def measured_ceilings(torch, dev, stream):
    """A practical HBM ceiling beside the published peak: a plain 1 GiB device
    copy (read + write bytes over its time), timed with events on the bench
    stream after warm-up. Context for the roofline fractions, not their
    denominator."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    with torch.cuda.stream(stream):
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        e0.record(stream)
        for _ in range(10):
            b.copy_(a)
        e1.record(stream)
        torch.cuda.synchronize()
        out["copy_1GiB_gbs"] = 2 * n * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    out["mfma_f16_32x32x16_tflops"] = mfma_ceiling(torch, dev, stream)
    return out


def grouped_source_hash():
    """sha256 over the grouped-path kernel sources (what an MFMA counter
    figure of the grouped GEMMs applies to)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("grouped.hip", "moe_kernels.h", "moe_launch.h"):
        with open(os.path.join(ROOT, "quantized_routed_expert_fp32_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def mfma_summary(pmc_csv, trace_csv, commands, n_cu=256, simd_per_cu=4, n_xcd=8):
    """Markdown summary of the grouped GEMMs' MFMA counters: per kernel, the
    mean per dispatch of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F16,
    GRBM_GUI_ACTIVE and the other SQ counters of the pass, with
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x SIMDs)
    (GRBM_GUI_ACTIVE reads the sum over the 8 XCDs of their active cycles)
    and the counted f16 MFMA flops (512 per MOPS unit) over the mean duration
    from the kernel trace, against 2,516.6 TFLOP/s."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(pmc_csv)):
        if "k_grp_" not in r["Kernel_Name"]:
            continue
        vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    dur = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if "k_grp_" in r["Kernel_Name"]:
            dur[r["Kernel_Name"]].append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3)
    lines = ["# MFMA counters of the grouped GEMMs, prompt chunks of 512 rows (4-bit g64) and 2048 rows (W4A16 Zipf)",
             "", "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", f"- source_sha256: {grouped_source_hash()}",
              f"- mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {n_xcd} XCDs x {n_cu} CUs x "
              f"{simd_per_cu} SIMDs); GRBM_GUI_ACTIVE sums the XCDs' active cycles",
              "- mfma_tflops = 512 x SQ_INSTS_VALU_MFMA_MOPS_F16 / mean duration (kernel trace)", ""]
    names = sorted(vals)
    cols = sorted({c for n in names for c in vals[n]})
    lines.append("| kernel | dispatches | mean us | " + " | ".join(cols) + " | mfma_busy | mfma_tflops | of peak |")
    lines.append("|---" * (len(cols) + 6) + "|")
    for n in names:
        m = {c: float(np.mean(v)) for c, v in vals[n].items()}
        nd = max(len(v) for v in vals[n].values())
        us = float(np.mean(dur[n])) if dur.get(n) else float("nan")
        busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (
            m.get("GRBM_GUI_ACTIVE", float("nan")) / n_xcd * n_cu * simd_per_cu)
        tfl = 512.0 * m.get("SQ_INSTS_VALU_MFMA_MOPS_F16", float("nan")) / (us * 1e-6) / 1e12
        lines.append(f"| `{n}` | {nd} | {us:.1f} | " + " | ".join(f"{m[c]:.4g}" for c in cols)
                     + f" | {busy:.3f} | {tfl:.1f} | {tfl / MFMA_F16_PEAK_TFLOPS:.3f} |")
    return "\n".join(lines) + "\n"


def counter_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, kernel, commands):
    """Markdown summary of the HBM byte counters of `kernel`: mean FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) scaled by what the same counters read
    for a plain copy of 1 GiB."""
    import csv

    def mean_kib(path, name):
        v = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
             if name in r["Kernel_Name"]]
        return sum(v) / len(v), len(v)

    f_kib, nf = mean_kib(fetch_csv, kernel)
    w_kib, nw = mean_kib(write_csv, kernel)
    cf_kib, _ = mean_kib(copy_fetch_csv, "copyBuffer")
    cw_kib, _ = mean_kib(copy_write_csv, "copyBuffer")
    gib_kib = float(1 << 20)
    f_scale, w_scale = gib_kib / cf_kib, gib_kib / cw_kib
    total = (f_kib * f_scale + w_kib * w_scale) * 1024
    lines = [f"# HBM traffic of {kernel}, decode 8 rows x 40 layers (4-bit g64)", "",
             "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Figures:", "",
              f"- kernel: {kernel}",
              f"- dispatches: {nf} (FETCH_SIZE pass), {nw} (WRITE_SIZE pass)",
              f"- fetch_kib_per_dispatch: {f_kib:.1f}",
              f"- write_kib_per_dispatch: {w_kib:.1f}",
              f"- copy_1GiB_fetch_kib: {cf_kib:.1f}",
              f"- copy_1GiB_write_kib: {cw_kib:.1f}",
              f"- fetch_scale: {f_scale:.4f}",
              f"- write_scale: {w_scale:.4f}",
              f"- hbm_bytes_per_launch: {total:.0f}",
              f"- source_sha256: {kernel_source_hash()}"]
    return "\n".join(lines) + "\n"


def counter_table(csvs, title, commands, fetch_scale=2.0):
    """Markdown table of the mean of every counter per kernel over the given
    rocprofv3 --pmc CSVs (one pass each); FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch) also as MB, FETCH_SIZE scaled by the plain copy's factor."""
    import collections
    import csv
    d = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csvs:
        for r in csv.DictReader(open(path)):
            d[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for v in d.values() for c in v})
    out = [f"# {title}", "", "Commands (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", ""]
    out += [f"    {c}" for c in commands]
    out += ["", f"Mean per dispatch; FETCH_SIZE and WRITE_SIZE in KiB as counted, `fetch MB` = FETCH_SIZE x "
            f"{fetch_scale} (the factor a plain 1 GiB copy reads for the counter) / 1e6.", "",
            "| kernel | dispatches | " + " | ".join(names) + (" | fetch MB |" if "FETCH_SIZE" in names else " |"),
            "|---" * (2 + len(names) + ("FETCH_SIZE" in names)) + "|"]
    for k in sorted(d):
        v = d[k]
        n = max(len(x) for x in v.values())
        cells = [f"{np.mean(v[c]):.4g}" if c in v else "-" for c in names]
        row = f"| `{k}` | {n} | " + " | ".join(cells)
        if "FETCH_SIZE" in names:
            row += f" | {np.mean(v['FETCH_SIZE']) * 1024 * fetch_scale / 1e6:.1f}" if "FETCH_SIZE" in v else " | -"
        out.append(row + " |")
    return "\n".join(out) + "\n"


def trace_summary(stats_csv, title, command, render, top=16):
    """Markdown table of a rocprofv3 kernel-stats CSV: per kernel the calls
    and the average, min and max duration in microseconds, and its share."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (from the repository root, `cd /tmp && export TMPDIR=/tmp` first):", "",
             f"    {command}", f"    {render}", "",
             "Durations in microseconds:", "",
             "| kernel | calls | average | min | max | share |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=None, help="override the 40 layers (debug)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="only the prompt-chunk lines (debug)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline decode workload and the prompt chunks (no 1-row and 3-bit lines)")
    ap.add_argument("--windows", action="store_true",
                    help="also time each prompt chunk through moe_forward_windows (16-row decode windows)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB copy (scales the HBM byte counters)")
    ap.add_argument("--counter-summary", nargs=4, metavar="CSV",
                    help="print the counter summary of k_dec_gateup from the FETCH_SIZE, "
                         "WRITE_SIZE, copy FETCH_SIZE and copy WRITE_SIZE counter CSVs")
    ap.add_argument("--trace-summary", nargs=3, metavar=("CSV", "PROGRAM", "TITLE"),
                    help="print a markdown table of a kernel-stats CSV written by rocprofv3 "
                         "--kernel-trace --stats around PROGRAM")
    ap.add_argument("--counter-table", nargs="+", metavar="ARG",
                    help="TITLE PROGRAM CSV...: a markdown table of per-kernel counter means from "
                         "rocprofv3 --pmc CSVs taken around PROGRAM (one pass per CSV)")
    ap.add_argument("--mfma-summary", nargs=2, metavar="CSV",
                    help="print the MFMA counter summary of the grouped GEMMs from a counter CSV "
                         "and a kernel-trace CSV of `bench.py --prefill-only`")
    args = ap.parse_args()
    if args.copy_calib:
        copy_calibration()
        return

    def run_of(path):
        folder = os.path.dirname(path)
        return folder, os.path.basename(path).split("_counter_collection")[0].split("_kernel_trace")[0]

    if args.counter_summary:
        # the commands that wrote the four CSVs: each pass's output folder and
        # file prefix are read back from the CSV path it was given
        dec = "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-prefill --no-extra --no-graph"
        passes = [("FETCH_SIZE", dec), ("WRITE_SIZE", dec), ("FETCH_SIZE", "python3 bench.py --copy-calib"),
                  ("WRITE_SIZE", "python3 bench.py --copy-calib")]
        cmds = []
        for (counter, prog), path in zip(passes, args.counter_summary):
            folder, prefix = run_of(path)
            cmds.append(f"rocprofv3 --pmc {counter} --output-format csv -d {folder} -o {prefix} -- {prog}")
        cmds.append("python3 bench.py --counter-summary " + " ".join(args.counter_summary))
        sys.stdout.write(counter_summary(*args.counter_summary, "k_dec_gateup", cmds))
        return
    if args.trace_summary:
        path, prog, title = args.trace_summary
        folder, prefix = run_of(path)
        prefix = prefix.split("_kernel_stats")[0]
        sys.stdout.write(trace_summary(path, title, f"rocprofv3 --kernel-trace --stats --output-format csv "
                                                    f"-d {folder} -o {prefix} -- {prog}",
                                       f'python3 bench.py --trace-summary {path} "{prog}" "{title}"'))
        return
    if args.counter_table:
        import csv
        title, prog, *paths = args.counter_table
        cmds = []
        for path in paths:
            folder, prefix = run_of(path)
            counters = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
            cmds.append(f"rocprofv3 --pmc {' '.join(counters)} --output-format csv -d {folder} -o {prefix} -- {prog}")
        cmds.append("python3 bench.py --counter-table " + " ".join(f'"{a_}"' if " " in a_ else a_
                                                                 for a_ in args.counter_table))
        sys.stdout.write(counter_table(paths, title, cmds))
        return
    if args.mfma_summary:
        import csv
        pmc, trace = args.mfma_summary
        counters = sorted({r["Counter_Name"] for r in csv.DictReader(open(pmc))})
        prog = "python3 bench.py --prefill-only --steps 5 --warmup 1"
        fp, pp = run_of(pmc)
        ft, pt = run_of(trace)
        cmds = [f"rocprofv3 --pmc {' '.join(counters)} --output-format csv -d {fp} -o {pp} -- {prog}",
                f"rocprofv3 --kernel-trace --output-format csv -d {ft} -o {pt} -- {prog}",
                "python3 bench.py --mfma-summary " + " ".join(args.mfma_summary)]
        sys.stdout.write(mfma_summary(pmc, trace, cmds))
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not run "
              "(the routed-expert FFN is benchmarked on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from synth import to_abi
    import quantized_routed_expert_fp32_amd as qr
    B = qr.binding
    B.lib()
    torch.cuda.init()
    dev = torch.device("cuda:0")

    stream = torch.cuda.Stream()
    sleeper = GpuSleep(torch, stream)
    prefill, host_prefill = {}, {}
    if not args.no_prefill:
        for c in (3, 4):
            r, h = bench_prefill(c, args.steps, args.warmup, B, to_abi, synth, torch, dev, stream, sleeper,
                                 windows=args.windows, keep_host=not args.no_cpu_baseline)
            prefill[f"c{c}"] = r
            host_prefill[c] = h
            torch.cuda.empty_cache()
        if not args.no_extra:
            # MXFP4 routed and shared experts at the 512-row chunk's shapes
            spec_mx = dataclasses.replace(synth.CONFIGS[3], cfg_id=346, name="prefill-512rows-mxfp4-experts",
                                          routed=synth.MX4G32, shared=synth.MX4G32)
            prefill["f4_mxfp4_512rows"], _ = bench_prefill(spec_mx, args.steps, args.warmup, B, to_abi, synth,
                                                           torch, dev, stream, sleeper)
            torch.cuda.empty_cache()
        if args.prefill_only:
            print(json.dumps({"prefill": prefill}), flush=True)
            return

    spec = synth.CONFIGS[1]
    L = args.layers or spec.layers
    R, k, H = spec.rows[-1], spec.top_k, spec.hidden
    default_workload = L == spec.layers
    layers, host = build_layers(spec, L, B, to_abi, synth, keep_host=1)
    head = bench_decode(spec, layers, R, args.steps, args.warmup, B, synth, torch, dev, stream, sleeper,
                        graph=not args.no_graph, sample_clock=True)
    workloads = {}
    if not args.no_extra:
        # one row through the same 40 layers (the one-row workload's shapes
        # and formats, rotated over distinct weights so it is not cache-resident)
        workloads["c0_1row_40layers"] = bench_decode(spec, layers, 1, args.steps, args.warmup, B, synth, torch,
                                                    dev, stream, sleeper, graph=not args.no_graph,
                                                    tag="decode-1row-q4g64 over 40 layers")
    del layers
    torch.cuda.empty_cache()
    if not args.no_extra:
        spec2 = synth.CONFIGS[2]
        layers2, _ = build_layers(spec2, args.layers or spec2.layers, B, to_abi, synth)
        for r2 in spec2.rows:
            workloads[f"c2_{r2}rows"] = bench_decode(spec2, layers2, r2, args.steps, args.warmup, B, synth,
                                                    torch, dev, stream, sleeper, graph=not args.no_graph)
        del layers2
        torch.cuda.empty_cache()
        # MXFP4 routed and shared experts, the headline shapes and router, over
        # 10 distinct layers (4 GB of weights: not cache-resident)
        spec_mx = dataclasses.replace(spec, cfg_id=340, name="decode-8rows-mxfp4-experts",
                                      routed=synth.MX4G32, shared=synth.MX4G32)
        layers_mx, _ = build_layers(spec_mx, args.layers or 10, B, to_abi, synth)
        workloads["f4_mxfp4_8rows"] = bench_decode(spec_mx, layers_mx, R, args.steps, args.warmup, B, synth,
                                                   torch, dev, stream, sleeper, graph=not args.no_graph,
                                                   tag="decode-8rows-mxfp4-experts over 10 layers")
        del layers_mx
        torch.cuda.empty_cache()
    for name, r in prefill.items():
        workloads[name] = r

    ceilings = measured_ceilings(torch, dev, stream)
    mf = ceilings.get("mfma_f16_32x32x16_tflops")
    log(f"[bench] measured ceilings: copy {ceilings['copy_1GiB_gbs']:.0f} GB/s, 32x32x16 f16 MFMA loop "
        + (f"{mf:.0f} TFLOP/s" if mf else "not built") + f"; sclk during the headline steps {head.get('sclk_mhz')}")

    cpu = None
    if not args.no_cpu_baseline:
        nt = host_threads()
        log(f"[bench] cpu baseline (fp64 oracle) on {nt} threads and on 1 thread")
        cpu = cpu_decode_baseline(spec, host[0], 64, nt)
        cpu["cpu_model"] = cpu_model()
        cpu["one_thread"] = cpu_decode_baseline(spec, host[0], 64, 1)
        pre = {}
        for c, Lh in host_prefill.items():
            if Lh is None:
                continue
            sp = synth.CONFIGS[c]
            xb = synth.make_x(sp, 0, sp.rows[0], rep=0)
            pre[f"c{c}"] = cpu_prefill_baseline(sp, Lh, xb, nt)
        cpu["prefill"] = pre
        log(f"[bench] cpu baseline: decode {cpu['value']:.2f} tokens/s ({nt} threads), "
            f"{cpu['one_thread']['value']:.2f} (1 thread); "
            + ", ".join(f"{k_} {v['value']:.1f} tokens/s" for k_, v in pre.items()))

    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "rows": R, "layers": L, "hidden": H,
                   "experts": spec.n_experts, "top_k": k, "inter": spec.inter,
                   "shared_inter": spec.shared_inter, "weights": fmt_name(spec.routed),
                   "shared_weights": fmt_name(spec.shared), "router_weights": fmt_name(spec.router),
                   "timing": head["timing"]},
        "roofline": {"bound": "hbm", "kernel": "k_dec_gateup", "achieved": head["gateup_gbs"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["gateup_gbs"] / HBM_PEAK_GBS,
                     "traffic": stored_traffic("k_dec_gateup") if default_workload else None,
                     "mean_us": head["kernel_us"]["decode_gateup"],
                     "bytes_per_launch": head["gateup_bytes_per_launch"]},
        "us_per_layer_spread": head["us_per_layer_spread"],
        "sclk_mhz": head.get("sclk_mhz"),
        "step_hbm": {"algorithmic_bytes": head["algorithmic_bytes_per_step"], "gbs": head["gbs"],
                     "frac": head["frac_hbm"], "us_per_layer": head["us_per_layer"],
                     "kernel_us": head["kernel_us"],
                     "mean_unique_experts": head["mean_unique_experts"]},
        "workloads": workloads,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
