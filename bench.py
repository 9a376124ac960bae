#!/usr/bin/env python3
"""Benchmark of the MoE decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one moe_decode_step call on one layer: for the default batch-1
dense workload that is three kernels (the router GEMV's row-slice partials,
the routing expert kernel that takes the top-k itself and streams the
experts' gate/up/down rows, and the fixed-order combine).  The default
workload is the Qwen3-30B-A3B-shaped batch-1 layer (H=2048, I=768, E=128,
top-8): 48 independent layers are resident in HBM and step i runs on layer
i mod 48, so every step streams its routed weights cold from HBM (47 x 75.5 MB
are read between two visits of a layer, far beyond the 256 MB Infinity
Cache).

Timing: the steps are captured in HIP graphs (the library never allocates or
synchronises inside a call) of at most one 48-layer cycle each; the timed
region is exactly K steps after W warm-up steps, every graph replay bracketed
by HIP events.  A statistics pass then replays the 48-step cycle at least 7
times and reports the median and min-max of the per-step time; eager
(uncaptured) timing is reported beside it.

Printed: one JSON line with the metric, the per-kernel roofline of the
dominant kernel (durations from HIP events recorded by the library on its
launch stream) and the fp64 oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE layer decode step + routed-weight HBM GB/s (% of 8 TB/s peak)"
HBM_PEAK_GBS = 8000.0
LAYERS = 48


def routed_bytes_per_step(wl, n_experts: int) -> int:
    """Routed expert bytes of one step (each distinct expert read once); the
    VQ format adds its layer-shared basis and code books, read once per step."""
    shared = 2 * (wl.H * wl.lr_r * 2 + wl.vq_K * wl.vq_d * 2) if wl.vq else 0
    return n_experts * wl.routed_bytes_per_expert + shared


def reader_screen_bytes(wl, M: int) -> int:
    """Sketch bytes the screening reads per step: for every routed (token,
    slot) and projection, the rows of the 80 scanned coordinates of every
    128-block (ceil(I/5) padded to 16 bytes each) and the blocks' scales,
    plus the routed experts' down-column norms."""
    nb = wl.H // 128
    rowb = ((wl.I + 4) // 5 + 15) // 16 * 16
    return M * wl.k * (2 * nb * (80 * rowb + 4 * wl.I) + 4 * wl.I)


def reader_bytes_per_step(wl, M: int) -> int:
    """Weight bytes of one reader step: screening, the kept channels' gate,
    up and down rows, and the recovery map's coefficients and basis."""
    rec = M * wl.k * wl.I * wl.rec_rank * 2 + wl.H * wl.rec_rank * 4 if wl.rec_rank else 0
    return reader_screen_bytes(wl, M) + wl.keep * M * 3 * wl.H * 2 + rec


def step_weight_bytes(wl, n_experts: int, M: int) -> int:
    if wl.reader:
        return reader_bytes_per_step(wl, M)
    if wl.keep:
        return wl.keep * 3 * wl.H * 2 * M
    return routed_bytes_per_step(wl, n_experts)


def kernel_algorithmic_bytes(wl, kernel: str, n_experts: int, M: int, K: int = 0) -> int:
    """Bytes a kernel must move by definition (weights it streams once plus
    its small activation inputs/outputs)."""
    H, I = wl.H, wl.I
    if kernel == "reader_screen":
        return reader_screen_bytes(wl, M)
    if kernel == "reader_recover":
        return M * wl.k * I * wl.rec_rank * 2
    if kernel in ("expert_fused", "decode_fused"):
        return n_experts * 3 * I * H * 2
    if kernel == "gateup":
        return n_experts * 2 * I * H * 2
    if kernel == "down":
        return n_experts * I * H * 2
    if kernel == "gateup_vqlr":
        return n_experts * 2 * (I * (H // wl.vq_d) + I * wl.lr_r * 2)
    if kernel == "chan_gather":
        return K * 3 * H * 2
    return 0


def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "expert_fused": ["memory_bound_routed_amd/csrc/dense.hip", "memory_bound_routed_amd/csrc/device_common.h",
                     "memory_bound_routed_amd/csrc/topk_device.h"],
    "decode_fused": ["memory_bound_routed_amd/csrc/dense.hip", "memory_bound_routed_amd/csrc/device_common.h",
                     "memory_bound_routed_amd/csrc/topk_device.h"],
    "gateup": ["memory_bound_routed_amd/csrc/dense.hip", "memory_bound_routed_amd/csrc/device_common.h"],
    "down": ["memory_bound_routed_amd/csrc/dense.hip", "memory_bound_routed_amd/csrc/device_common.h"],
    "gateup_vqlr": ["memory_bound_routed_amd/csrc/vqlr.hip", "memory_bound_routed_amd/csrc/device_common.h"],
    "chan_gather": ["memory_bound_routed_amd/csrc/chansparse.hip", "memory_bound_routed_amd/csrc/device_common.h",
                    "memory_bound_routed_amd/csrc/select_device.h", "memory_bound_routed_amd/csrc/reader_device.h",
                    "memory_bound_routed_amd/csrc/topk_device.h"],
    "reader_screen": ["memory_bound_routed_amd/csrc/reader.hip", "memory_bound_routed_amd/csrc/device_common.h",
                      "memory_bound_routed_amd/csrc/topk_device.h"],
}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


def _pmc_rows(path, counter):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc counter CSV."""
    import csv
    out = []
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                out.append((row["Kernel_Name"], float(row["Counter_Value"])))
    return out


# rocprofv3 kernel-name fragment of each library kernel whose traffic is taken
# (decode_fused is the routing instance of the fused expert kernel).
ROCPROF_NAME = {"expert_fused": "expert_fused_kernel", "decode_fused": "expert_fused_kernel",
                "gateup": "gateup_dense_kernel", "down": "down_kernel", "gateup_vqlr": "gateup_vqt_kernel",
                "chan_gather": "chan_topk_gather_kernel", "reader_screen": "reader_screen_kernel"}


def traffic_from_counters(fetch_csv, write_csv, workload, kernel="decode_fused"):
    """HBM bytes per launch of `kernel` from two rocprofv3 --pmc runs of
    `bench.py --counter-pass` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by what it reads for the calibration copy (a
    256 MiB fp32 negation: 256 MiB read, 256 MiB written), so the result is
    in bytes of the same kind as the algorithmic count."""
    copy_bytes = 64 * 2 ** 20 * 4
    res = {"workload": workload, "kernel": kernel, "source_digest": source_digest(KERNEL_SOURCES[kernel])}
    total = 0.0
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, name)
        cal = [v for k, v in rows if "neg" in k and "elementwise" in k]
        ker = [v for k, v in rows if ROCPROF_NAME[kernel] in k]
        if not cal or not ker:
            raise SystemExit("%s: no calibration (%d) or %s (%d) dispatches" % (path, len(cal), kernel, len(ker)))
        cal_kib = float(np.median(cal))
        factor = copy_bytes / (cal_kib * 1024.0)
        per = float(np.mean(ker)) * 1024.0 * factor
        res[name] = {"calibration_kib": cal_kib, "factor": round(factor, 4), "dispatches": len(ker),
                     "kib_per_dispatch_mean": round(float(np.mean(ker)), 1),
                     "kib_per_dispatch_min": round(float(np.min(ker)), 1),
                     "kib_per_dispatch_max": round(float(np.max(ker)), 1), "bytes_per_launch": round(per)}
        total += per
    res["hbm_bytes_per_launch"] = round(total)
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


# ----------------------------------------------------------------------------

def build_layers(wl, n_layers, M, keep=0):
    """Layer 0 from the seeded host generator, the rest drawn on the device."""
    import torch
    import synth
    import memory_bound_routed_amd as mb

    def dev_bf16(shape, gen):
        x = torch.empty(shape, dtype=torch.float32, device="cuda")
        x.normal_(0.0, synth.SIGMA_W, generator=gen)
        return x.to(torch.bfloat16).view(torch.int16)

    layers = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(wl.seed)
    for L in range(n_layers):
        if L == 0:
            inp = synth.layer_inputs(wl, 0)
            t = {k: torch.from_numpy(v.view(np.int16) if v.dtype == np.uint16 else v).cuda()
                 for k, v in inp.items() if v is not None and k != "h"}
        else:
            t = {"router_w": dev_bf16((wl.H, wl.E), gen)}
            if wl.hot_experts:
                t["router_bias"] = torch.from_numpy(synth.router_bias(wl, L)).cuda()
            # one allocation per layer for the three expert matrices
            big = dev_bf16((3, wl.E, wl.I, wl.H), gen) if not wl.vq else None
            if wl.vq:
                t["w_down"] = dev_bf16((wl.E, wl.I, wl.H), gen)
                for P in ("gate", "up"):
                    t["lr_basis_" + P] = dev_bf16((wl.H, wl.lr_r), gen)
                    t["lr_coef_" + P] = dev_bf16((wl.E, wl.I, wl.lr_r), gen)
                    t["vq_book_" + P] = dev_bf16((wl.vq_K, wl.vq_d), gen)
                    t["vq_idx_" + P] = torch.randint(0, 256, (wl.E, wl.I, wl.H // wl.vq_d), dtype=torch.uint8,
                                                     device="cuda", generator=gen)
            else:
                t["w_gate"], t["w_up"], t["w_down"] = big[0], big[1], big[2]
        if wl.vq:
            cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, M, mb.MOE_WFORMAT_VQLR, wl.vq_d, wl.vq_K,
                                 wl.lr_r)
        else:
            cfg = mb.make_config(wl.H, wl.I, wl.E, wl.k, wl.block_b, M, max_keep=keep, reader=int(wl.reader),
                                 rec_rank=wl.rec_rank)
        if wl.reader:
            reader_tables(mb, cfg, t, synth.rotation_signs(wl, L))
        elif keep:
            norms = torch.empty((wl.E, wl.I), dtype=torch.float32, device="cuda")
            mb.moe_channel_norms(cfg, t["w_gate"], t["w_up"], t["w_down"], norms)
            t["chan_norm"] = norms
        layers.append(mb.Layer(cfg, t))
    torch.cuda.synchronize()
    return layers


def reader_tables(mb, cfg, t, signs, iters=8):
    """The reader's load-time arrays of one layer, built on the device."""
    import torch
    E, I, H = cfg.E, cfg.I, cfg.H
    t["rot_signs"] = torch.from_numpy(np.ascontiguousarray(signs, np.int8).reshape(-1)).cuda()
    t["sketch"] = torch.empty(E * 2 * H * mb.moe_sketch_row_bytes(I), dtype=torch.uint8, device="cuda")
    t["sketch_scale"] = torch.empty((E, 2, H // 128, I), dtype=torch.float32, device="cuda")
    t["down_norm"] = torch.empty((E, I), dtype=torch.float32, device="cuda")
    mb.moe_reader_sketch(cfg, t["w_gate"], t["w_up"], t["rot_signs"], t["sketch"], t["sketch_scale"])
    mb.moe_down_norms(cfg, t["w_down"], t["down_norm"])
    if cfg.rec_rank:
        t["rec_basis"] = torch.empty((H, cfg.rec_rank), dtype=torch.float32, device="cuda")
        t["rec_coef"] = torch.empty((E, I, cfg.rec_rank), dtype=torch.int16, device="cuda")
        mb.moe_recovery_basis(cfg, t["w_down"], cfg.rec_rank, iters, t["rec_basis"])
        mb.moe_recovery_coefs(cfg, t["rec_basis"], cfg.rec_rank, t["w_down"], t["rec_coef"])


def run_steps(layers, hs, M, keep, order):
    for i in order:
        L = layers[i % len(layers)]
        L.decode_step(hs[i % len(hs)], M, keep=keep)


def host_info():
    """Host CPU model and the cores this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = int(cores or 1)
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:  # the host share this process is given
        cores = min(cores, int(omp))
    return model, cores


def cpu_baseline(wl, budget_s=10.0, max_steps=40):
    """The fp64 oracle timed on the host on a bounded sample: steps over the
    first 4 layers, each layer's routed experts drawn from the seeded
    generator beforehand (generation is not timed); once with one BLAS
    thread, once with a thread per usable host core."""
    import synth
    import oracle as O
    from threadpoolctl import threadpool_limits
    model, cores = host_info()
    sample = _cpu_sample(wl, synth, O)
    with threadpool_limits(limits=1):
        one = _cpu_time(wl, sample, budget_s, max_steps, O)
    with threadpool_limits(limits=cores):
        allc = _cpu_time(wl, sample, budget_s, max_steps, O)
    # the faster of the two thread counts is the reported value (small GEMVs
    # can run slower on many BLAS threads than on one)
    best, nthreads = (allc, cores) if allc["value"] >= one["value"] else (one, 1)
    return {"value": best["value"], "unit": "GB/s", "us_per_step": best["us_per_step"], "cores": nthreads,
            "kind": "oracle", "cpu_model": model, "nproc": cores,
            "single_core": {"value": one["value"], "us_per_step": one["us_per_step"], "steps": one["steps"]},
            "all_cores": {"value": allc["value"], "us_per_step": allc["us_per_step"], "steps": allc["steps"],
                          "threads": cores},
            "sample": "%d steps of %s cycling over %d host-resident layers (only routed experts drawn%s); fp64 numpy, "
                      "timed with 1 and with %d BLAS threads"
                      % (best["steps"], wl.name, len(sample),
                         "; sketches precomputed, recovery basis of the routed experts' down columns"
                         if wl.reader else "", cores)}


def _cpu_sample(wl, synth, O):
    keep = wl.keep
    layers = []
    for L in range(min(4, wl.layers if not wl.reader else 4)):
        inp = {"h": synth.hidden(wl, L), "router_w": synth.router_weight(wl, L),
               "router_bias": synth.router_bias(wl, L)}
        ids, _, _ = O.route_topk(inp["h"], inp["router_w"], wl.k, inp["router_bias"])
        ex = sorted(set(ids.ravel().tolist()))
        full = synth.layer_inputs(wl, L, experts=ex)
        extra = None
        if wl.reader:
            # load-time arrays of the routed experts (not timed): sketches,
            # down norms and -- standing in for the whole layer's -- a recovery
            # basis of the routed experts' down columns
            signs = synth.rotation_signs(wl, L)
            sk = {}
            for e in ex:
                cg, sg = O.reader.sketch_expert(full["w_gate"][e], signs)
                cu, su = O.reader.sketch_expert(full["w_up"][e], signs)
                sk[e] = (cg, sg, cu, su, O.reader.down_norms(full["w_down"][e]))
            rec = None
            if wl.rec_rank:
                U = O.reader.recovery_basis(full["w_down"][ex], wl.rec_rank)
                b = np.zeros((wl.E, wl.I, wl.rec_rank), np.uint16)
                for e in ex:
                    b[e] = O.reader.recovery_coefs(U, full["w_down"][e])
                rec = (U, b)
            extra = (signs, sk, rec)
            norms = None
        else:
            norms = O.channel_norms(full["w_gate"], full["w_up"], full["w_down"], experts=ex) if keep else None
        layers.append((full, norms, len(ex), extra))
    return layers


def _cpu_time(wl, layers, budget_s, max_steps, O):
    keep = wl.keep
    t_total, n, bytes_total = 0.0, 0, 0
    while n < max_steps and t_total < budget_s:
        full, norms, nex, extra = layers[n % len(layers)]
        t0 = time.perf_counter()
        if wl.reader:
            signs, sk, rec = extra
            ids, aff, _ = O.route_topk(full["h"], full["router_w"], wl.k, full.get("router_bias"))
            for t in range(wl.M):
                O.reader.reader_step(full["h"][t], ids[t], aff[t].astype(np.float32), full["w_gate"], full["w_up"],
                                     full["w_down"], signs, keep, recovery=rec, sketches=sk)
        else:
            O.moe_step(full, wl.k, keep=keep, norms=norms)
        t_total += time.perf_counter() - t0
        bytes_total += step_weight_bytes(wl, nex, wl.M)
        n += 1
    return {"value": round(bytes_total / t_total / 1e9, 4), "us_per_step": round(t_total / n * 1e6, 1), "steps": n}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=960)
    ap.add_argument("--warmup", type=int, default=96)
    ap.add_argument("--workload", default="dense_h2048_i768_e128_k8_m1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="short run for rocprofv3 --pmc: a 256 MiB elementwise copy (calibration) then 96 steps")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: turn two rocprofv3 --pmc counter CSVs of --counter-pass into "
                         "profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--traffic-kernel", default="decode_fused", choices=sorted(ROCPROF_NAME),
                    help="the kernel whose dispatches --traffic-from reads")
    args = ap.parse_args()

    if args.traffic_from:
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload, args.traffic_kernel)
        return

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode step is measured on a single MI355X "
              "(multi-GPU sharding is a design note, not built); got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import memory_bound_routed_amd as mb

    wl = synth.WORKLOADS[args.workload]
    M, keep = wl.M, wl.keep
    n_layers = LAYERS if wl.layers > 1 else 1
    if wl.layers == 1 and args.workload != "tiny_h256_i128_e16_k2":
        n_layers = LAYERS  # rotate layers for cold reads on every full-size workload
    layers = build_layers(wl, n_layers, M, keep)

    n_h = max(n_layers, 48)
    hs = torch.from_numpy(np.stack([synth.hidden(wl, 0, step=i) for i in range(n_h)])).cuda()

    if args.counter_pass:
        x = torch.empty(64 * 2 ** 20, dtype=torch.float32, device="cuda").normal_()
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        run_steps(layers, hs, M, keep, range(96))
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": True, "copy_bytes": x.numel() * 4, "workload": wl.name}))
        return

    cycle = list(range(n_h))
    K = max(1, args.steps)
    W = max(0, args.warmup)

    # distinct routed experts per layer for the byte count: route every layer once (eager)
    n_ex = []
    for i in cycle:
        L = layers[i % n_layers]
        L.route(hs[i], M)
        n_ex.append(len(set(L.ids[:M].flatten().tolist())))
    torch.cuda.synchronize()
    step_bytes = [step_weight_bytes(wl, n, M) for n in n_ex]

    # ---- graph-captured steps: graphs of one 48-step cycle (and a shorter
    # one for a remainder), step i of a run on layer i mod 48
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_steps(layers, hs, M, keep, cycle)  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = {}

    def graph_of(n):
        if n not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_steps(layers, hs, M, keep, range(n))
            torch.cuda.synchronize()
            graphs[n] = g
        return graphs[n]

    def blocks_of(n):
        return [len(cycle)] * (n // len(cycle)) + ([n % len(cycle)] if n % len(cycle) else [])

    def timed_replays(sizes):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sizes]
        gs = [graph_of(n) for n in sizes]
        torch.cuda.synchronize()
        for (a, b), g in zip(ev, gs):
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    for n in blocks_of(W):
        graph_of(n).replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    sizes = blocks_of(K)
    gs = [graph_of(n) for n in sizes]
    torch.cuda.synchronize()
    t0.record()
    for g in gs:
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_graph = t0.elapsed_time(t1)
    ms_per_step = ms_graph / K
    bytes_timed = sum(step_bytes[i % len(cycle)] for i in range(K))

    # statistics: at least 7 replays of the 48-step cycle, each timed
    n_stat = max(7, K // len(cycle))
    per_step = sorted(t / len(cycle) * 1e3 for t in timed_replays([len(cycle)] * n_stat))
    stats = {"replays": n_stat, "steps_per_replay": len(cycle),
             "median_us_per_step": round(float(np.median(per_step)), 3),
             "min_us_per_step": round(per_step[0], 3), "max_us_per_step": round(per_step[-1], 3)}
    reps = max(1, round(K / len(cycle)))

    # ---- eager steps (no graph)
    run_steps(layers, hs, M, keep, cycle)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run_steps(layers, hs, M, keep, cycle)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / K

    # ---- per-kernel durations: the library attaches a pair of HIP events to
    # every launch (stamped by the kernel's own dispatch on its stream) while
    # profiling is enabled; same steps, eager, right after the timed region
    for L in layers:
        mb.moe_profile_enable(L.ctx, True)
    for _ in range(reps):
        run_steps(layers, hs, M, keep, cycle)
    torch.cuda.synchronize()
    kern = {}
    for L in layers:
        for name, (ms, n) in mb.moe_profile_read(L.ctx).items():
            a = kern.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
        mb.moe_profile_enable(L.ctx, False)
    kernels = {k: {"avg_us": round(v[0] / v[1] * 1e3, 3), "launches": v[1]} for k, v in kern.items()}
    # the roofline is that of the dominant kernel among those streaming routed
    # weights (routing, selection and combines are latency-bound and listed
    # in "kernels" with their durations)
    streaming = [k for k in kern if kernel_algorithmic_bytes(wl, k, 1, M, max(keep * M, 1)) > 0]
    dominant = max(streaming or list(kern), key=lambda k: kern[k][0])
    avg_ex = float(np.mean(n_ex))
    alg = kernel_algorithmic_bytes(wl, dominant, round(avg_ex), M, keep * M)
    dur_s = kernels[dominant]["avg_us"] / 1e6
    achieved = alg / dur_s / 1e9 if alg else None
    expert_kernels = [k for k in kern if k not in ("router", "align", "router_align", "router_gemv")]
    expert_us = sum(kernels[k]["avg_us"] * kernels[k]["launches"] for k in expert_kernels) / K

    us_step = ms_per_step * 1e3
    gbs = bytes_timed / (ms_graph / 1e3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(us_step, 3),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "us_per_step_eager": round(ms_eager * 1e3, 3),
        "expert_path_us_sum_of_kernels": round(expert_us, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 weights, fp32 activations and accumulation",
        "data": "synthetic: layer 0 from the seeded host generator, layers 1..%d drawn on the device; "
                "N(0,0.02) bf16 weights, N(0,1) fp32 hidden states" % (n_layers - 1),
        "config": {"workload": wl.name, "H": wl.H, "I": wl.I, "E": wl.E, "top_k": wl.k, "tokens": M,
                   "block_b": wl.block_b, "layers_rotated": n_layers, "keep_channels": keep or None,
                   "selection": ("ternary-sketch reader" + (", rank-%d recovery map" % wl.rec_rank
                                                           if wl.rec_rank else "")) if wl.reader else
                   ("static channel norms" if keep else None),
                   "routed_bytes_per_step": int(sum(step_bytes) / len(cycle)),
                   "avg_distinct_experts": round(avg_ex, 2), "timing": "exactly %d steps as HIP-graph replays of <= %d steps "
                   "between two HIP events after %d warm-up steps" % (K, len(cycle), W)},
        "timing_stats": stats,
        "kernels": kernels,
        "roofline": {
            "kernel": dominant,
            "duration_us": kernels[dominant]["avg_us"],
            "bound": "hbm",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
            "algorithmic_bytes_per_launch": alg,
            "traffic": measured_traffic(dominant, wl.name),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
