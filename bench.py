#!/usr/bin/env python3
"""Benchmark of the routed-expert FFN (qwen3_5-MoE 35B-A3B shapes) on one MI355X.

Workload (the headline): decode, 8 independent rows through 40 distinct MoE
layer weight sets (hidden 2048, 256 experts, top-8, expert intermediate 512,
shared expert 512), 4-bit affine g64 weights everywhere (~18 GB packed, so
the ~4 GB of expert bytes a step touches cannot stay in cache). One step is
one pass of the whole hot path over one batch: for each of the 40 layers,
route (logits, top-8, weights, shared gate) then the decode experts
(gate/up + SwiGLU, down, combine). Inputs are resident in HBM before the
timed region; each step takes a fresh set of activations (4 sets rotate).

Prints ONE JSON line. `value` is MoE-layer tokens/s: rows x layers per
second. `roofline` is the dominant kernel (decode gate/up) timed live with
HIP events on its stream: algorithmic bytes per launch (the packed gate/up
bytes of the unique experts the launch reads, plus x in and h out) over its
mean duration. `cpu_baseline` is the FP64 oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(spec, fmt, inter):
    """Packed bytes of one expert: gate/up and down (codes + scale words)."""
    scb = 4 if fmt.mode == 0 else 2
    gu = 2 * inter * spec.hidden * fmt.bits // 8 + 2 * inter * (spec.hidden // fmt.group) * scb
    dn = spec.hidden * inter * fmt.bits // 8 + spec.hidden * (inter // fmt.group) * scb
    return gu, dn


def fmt_name(f):
    """Short text name of a weight format, e.g. 'affine 4-bit g64 bf16 scale/bias'."""
    dt = "bf16" if f.scale_dtype == 0 else "fp16"
    if f.mode == 2:
        return f"dense {dt}"
    if f.mode == 1:
        return f"symmetric {f.bits}-bit g{f.group} {dt} scale"
    return f"affine {f.bits}-bit g{f.group} {dt} scale/bias"


def router_bytes(spec):
    f, g = spec.router, spec.gate_row
    scb = 4 if f.mode == 0 else 2
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


def cpu_baseline(spec, Lh, rows, budget_s=15.0):
    """The FP64 oracle (as it stands) on one layer x `rows` rows, BLAS on 1 thread."""
    import contextlib

    import oracle.moe_oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        ctx = contextlib.nullcontext()
    xb = synth.make_x(spec, 0, rows, rep=0)
    with ctx:
        t0 = time.perf_counter()
        done = 0
        dense = O.DenseExperts(Lh, cache=True)
        for r in range(rows):
            O.moe_forward(Lh, xb[r:r + 1], dense)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{done} decode rows (x of the workload's first layer) through that "
                       f"layer, per-row fp64 form, experts dequantised on first use, {dt:.1f} s")


def bench_prefill(cfg_id, steps, warmup, B, to_abi, synth, torch, dev, stream, windows=False):
    """One prompt chunk through one layer: route + grouped experts, timed as a
    HIP graph; per-phase times from events inside the library's launches."""
    spec = synth.CONFIGS[cfg_id]
    R, k, H, E = spec.rows[0], spec.top_k, spec.hidden, spec.n_experts
    I, Is = spec.inter, spec.shared_inter
    Lh = synth.make_layer(spec, 0)
    layer = B.pack_layer(B.layer_desc(*to_abi.desc_args(spec)), to_abi.tensors(Lh))
    bias = torch.from_numpy(Lh.logit_bias).to(dev) if Lh.logit_bias is not None else None
    del Lh
    x = torch.from_numpy(synth.make_x(spec, 0, R, rep=0).view(np.int16)).to(dev)
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    p = torch.empty((R, k), dtype=torch.float32, device=dev)
    sg = torch.empty((R,), dtype=torch.float32, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = B.new_workspace(layer, R, True, dev)

    def chunk(events=None):
        B.route(layer, x, bias, taps=dict(events=events[:2]) if events else None,
                out=(ids, p, sg), ws=ws, stream=stream)
        B.experts(layer, x, ids, p, sg, True, ws=ws, y=y,
                  taps=dict(events=events[2:]) if events else None, stream=stream)

    with torch.cuda.stream(stream):
        chunk()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            chunk()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
    us = t0.elapsed_time(t1) / steps * 1e3
    # per phase: route | sort | gate/up GEMMs | down GEMMs | combine
    n_ev = 10
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    with torch.cuda.stream(stream):
        for es in evs:
            for e in es:
                e.record(stream)
        for es in evs:
            chunk(events=es)
        torch.cuda.synchronize()
    ph = np.zeros(5)
    for es in evs:
        for i in range(5):
            ph[i] += es[2 * i].elapsed_time(es[2 * i + 1])
    ph = ph / steps * 1e3
    slots = R * k
    f_gu = 2.0 * (slots * 2 * I + R * 2 * Is) * H
    f_dn = 2.0 * (slots * I + R * Is) * H
    f_rt = 2.0 * R * H * (E + 1)
    ids_h = ids.cpu().numpy()
    cnt = np.bincount(ids_h.reshape(-1), minlength=E)
    tf = lambda f, t: f / (t * 1e-6) / 1e12
    res = {
        "workload": spec.name, "rows": R, "us_per_chunk": us, "tokens_per_s": R / (us * 1e-6),
        "flop": f_gu + f_dn + f_rt, "tflops": tf(f_gu + f_dn + f_rt, us),
        "frac_mfma_peak": tf(f_gu + f_dn + f_rt, us) / MFMA_F16_PEAK_TFLOPS,
        "phase_us": {"route": ph[0], "sort": ph[1], "gate_up": ph[2], "down": ph[3],
                     "combine": ph[4]},
        "gate_up_tflops": tf(f_gu, ph[2]), "down_tflops": tf(f_dn, ph[3]),
        "rows_per_expert": {"max": int(cnt.max()), "mean": float(cnt.mean()),
                            "empty": int((cnt == 0).sum())},
    }
    if windows:
        # the same chunk through the decode step's arithmetic in 16-row windows
        # (moe_forward_windows: same bits however the prompt is cut), eager;
        # off by default so that the decode kernels' traced averages stay the
        # 8-row workload's
        wws = B.new_workspace(layer, 16, False, dev)
        with torch.cuda.stream(stream):
            B.forward_windows(layer, x, bias, ws=wws, out=(ids, p, sg), y=y, stream=stream)
            torch.cuda.synchronize()
            t0.record(stream)
            for _ in range(3):
                B.forward_windows(layer, x, bias, ws=wws, out=(ids, p, sg), y=y, stream=stream)
            t1.record(stream)
            torch.cuda.synchronize()
        res["windows_us_per_chunk"] = t0.elapsed_time(t1) / 3 * 1e3
    log(f"[bench] prefill {spec.name}: {us:.1f} us/chunk, {res['tokens_per_s']:.0f} tokens/s, "
        f"{res['tflops']:.1f} TFLOP/s ({100 * res['frac_mfma_peak']:.1f}% of f16 MFMA); "
        + ", ".join(f"{k_} {v:.1f}" for k_, v in res["phase_us"].items())
        + (f"; 16-row windows {res['windows_us_per_chunk']:.1f} us/chunk" if windows else ""))
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


def measured_ceilings(torch, dev, stream):
    """Practical ceilings beside the published peaks: a plain 1 GiB device
    copy (read + write bytes over its time) and a square fp16 GEMM of 8192
    through torch's BLAS, each timed with events on the bench stream after
    warm-up. Context for the roofline fractions, not their denominators."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    m = 8192
    A = torch.randn(m, m, dtype=torch.float16, device=dev)
    Bm = torch.randn(m, m, dtype=torch.float16, device=dev)
    C = torch.empty(m, m, dtype=torch.float16, device=dev)
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
        for _ in range(3):
            torch.mm(A, Bm, out=C)
        e0.record(stream)
        for _ in range(10):
            torch.mm(A, Bm, out=C)
        e1.record(stream)
        torch.cuda.synchronize()
        out["gemm_fp16_8192_tflops"] = 2 * m ** 3 * 10 / (e0.elapsed_time(e1) / 1e3) / 1e12
    del a, b, A, Bm, C
    torch.cuda.empty_cache()
    return out


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None, help="override the 40 layers (debug)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="only the prompt-chunk lines (debug)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--decode-config", type=int, default=1, choices=(0, 1, 2),
                    help="decode workload (default 1, the 8-row 40-layer 4-bit one; 2 is the mixed "
                         "3-bit one, 0 the one-row one)")
    ap.add_argument("--rows", type=int, default=None, help="decode rows (default: the workload's)")
    ap.add_argument("--windows", action="store_true",
                    help="also time each prompt chunk through moe_forward_windows (16-row decode windows)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB copy (scales the HBM byte counters)")
    ap.add_argument("--counter-summary", nargs=4, metavar="CSV",
                    help="print the counter summary of k_dec_gateup from the FETCH_SIZE, "
                         "WRITE_SIZE, copy FETCH_SIZE and copy WRITE_SIZE counter CSVs")
    args = ap.parse_args()
    if args.copy_calib:
        copy_calibration()
        return
    if args.counter_summary:
        # the commands that wrote the four CSVs: each pass's output folder and
        # file prefix are read back from the CSV path it was given
        def run_of(path):
            folder = os.path.dirname(path)
            return folder, os.path.basename(path).split("_counter_collection")[0]
        dec = "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --no-prefill --no-graph"
        passes = [("FETCH_SIZE", dec), ("WRITE_SIZE", dec), ("FETCH_SIZE", "python3 bench.py --copy-calib"),
                  ("WRITE_SIZE", "python3 bench.py --copy-calib")]
        cmds = []
        for (counter, prog), path in zip(passes, args.counter_summary):
            folder, prefix = run_of(path)
            cmds.append(f"rocprofv3 --pmc {counter} --output-format csv -d {folder} -o {prefix} -- {prog}")
        cmds.append("python3 bench.py --counter-summary " + " ".join(args.counter_summary))
        sys.stdout.write(counter_summary(*args.counter_summary, "k_dec_gateup", cmds))
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
    prefill = None
    if not args.no_prefill:
        prefill = [bench_prefill(c, 20, 3, B, to_abi, synth, torch, dev, stream, args.windows) for c in (3, 4)]
        if args.prefill_only:
            print(json.dumps({"prefill": prefill}), flush=True)
            return

    spec = synth.CONFIGS[args.decode_config]
    L = args.layers or spec.layers
    R, k, H = args.rows or spec.rows[-1], spec.top_k, spec.hidden
    NX = 4
    # the stored counter summary covers the default decode workload only
    default_workload = args.decode_config == 1 and R == spec.rows[-1] and L == spec.layers
    log(f"[bench] workload {spec.name}: rows={R} layers={L}")
    layers, host = build_layers(spec, L, B, to_abi, synth, keep_host=1)
    xs = [[torch.from_numpy(synth.make_x(spec, l, R, rep=s).view(np.int16)).to(dev)
           for s in range(NX)] for l in range(L)]
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    p = torch.empty((R, k), dtype=torch.float32, device=dev)
    sg = torch.empty((R,), dtype=torch.float32, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = B.new_workspace(layers[0], R, False, dev)

    def step(s, events=None):
        for l in range(L):
            x = xs[l][s % NX]
            rt = dict(events=events[l][:2]) if events is not None else None
            B.route(layers[l], x, taps=rt, out=(ids, p, sg), ws=ws, stream=stream)
            tp = dict(events=events[l][2:]) if events is not None else None
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

    # ---- timed region: whole steps
    graphs = None
    if not args.no_graph:
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
        for s in range(args.warmup):
            run(s)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for s in range(args.steps):
            run(s)
        t1.record(stream)
        torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    tokens_per_s = R * L / (ms_step / 1e3)
    mean_step_bytes = float(np.mean([step_bytes[s % NX] for s in range(args.steps)]))
    log(f"[bench] {ms_step * 1e3:.1f} us/step, {ms_step * 1e3 / L:.2f} us/layer, "
        f"{tokens_per_s:.0f} tokens/s, step HBM {mean_step_bytes / ms_step / 1e6:.0f} GB/s")

    # ---- dominant kernel: events around each kernel of the decode call
    nk = max(1, min(args.steps, 50))
    # events bracket each kernel: route, gate/up, down + combine
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)]
           for _ in range(nk)]
    with torch.cuda.stream(stream):
        for es in evs:              # torch creates the HIP event on first record
            for el in es:
                for e in el:
                    e.record(stream)
        step(0)
        torch.cuda.synchronize()
        for s in range(nk):
            step(s, events=evs[s])
        torch.cuda.synchronize()
    dur = np.zeros((3,))  # route, gate/up, down+combine
    gu_bytes_sum = 0.0
    for s in range(nk):
        for l in range(L):
            e = evs[s][l]
            for i in range(3):
                dur[i] += e[2 * i].elapsed_time(e[2 * i + 1])
            gu_bytes_sum += gu_launch_bytes[l, s % NX]
    n_launch = nk * L
    gu_ms = dur[1] / n_launch
    gu_bytes = gu_bytes_sum / n_launch
    achieved = gu_bytes / (gu_ms / 1e3) / 1e9
    kus = dur / n_launch * 1e3
    log(f"[bench] route {kus[0]:.2f} us, gate/up {kus[1]:.2f} us ({achieved:.0f} GB/s), "
        f"down+combine {kus[2]:.2f} us")

    ceilings = measured_ceilings(torch, dev, stream)
    log(f"[bench] measured ceilings: copy {ceilings['copy_1GiB_gbs']:.0f} GB/s, "
        f"fp16 GEMM {ceilings['gemm_fp16_8192_tflops']:.0f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(spec, host[0], 64)
        log(f"[bench] cpu baseline {cpu['value']:.3f} tokens/s")

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "rows": R, "layers": L, "hidden": H,
                   "experts": spec.n_experts, "top_k": k, "inter": spec.inter,
                   "shared_inter": spec.shared_inter, "weights": fmt_name(spec.routed),
                   "shared_weights": fmt_name(spec.shared), "router_weights": fmt_name(spec.router),
                   "timing": "hip graph replay" if graphs else "eager"},
        "roofline": {"bound": "hbm", "kernel": "k_dec_gateup", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic("k_dec_gateup") if default_workload else None, "mean_us": gu_ms * 1e3,
                     "bytes_per_launch": gu_bytes},
        "step_hbm": {"algorithmic_bytes": mean_step_bytes,
                     "gbs": mean_step_bytes / ms_step / 1e6,
                     "frac": mean_step_bytes / ms_step / 1e6 / HBM_PEAK_GBS,
                     "us_per_layer": ms_step * 1e3 / L,
                     "kernel_us": {"route": kus[0], "decode_gateup": kus[1],
                                   "decode_down_combine": kus[2]},
                     "mean_unique_experts": float(uniq.mean())},
        "prefill": prefill,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
