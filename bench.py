"""Benchmark of the MoE layer on one MI355X.

A step is one moe_forward over one batch of synthetic tokens: router, group-limited
top-k, permutation, grouped SwiGLU experts, weighted combine.  The default workload
is the Ling-3.0-tiny-shaped decode layer (T=4, H=1536, I=512, E=128 in 8 groups of
16 keeping 4, top-8, bf16).  Expert weights rotate over several copies placed at
different addresses so that every step streams them from HBM rather than from the
256 MiB Infinity Cache (a model runs a different layer's weights each time).

Prints ONE JSON line (stdout) with the throughput, a roofline entry for the
dominant kernel (timed with HIP events on the library's stream) and the float64
oracle timed on the host cores as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 MI355X; decode HBM GB/s and prefill MFMA % of peak"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2         # MI355X dense fp8 MFMA
WEIGHT_KEYS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up",
               "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")
NV_KEYS = ("b_gate", "b_up", "b_down", "g_gate", "g_up", "g_down")
# weight copies rotated per step so that the weight stream comes from HBM, not from
# the 256 MB last-level cache (one NVFP4 copy of the decode layer is ~170 MB)
DEFAULT_SETS = {"tiny": 1, "decode": 8, "prefill": 2, "fp8": 4, "inkling": 1, "decode_nvfp4": 16,
                "prefill_nvfp4": 4, "decode_stack": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "fp8", "inkling", "decode_nvfp4",
                             "prefill_nvfp4", "decode_stack"])
    ap.add_argument("--sets", type=int, default=0, help="weight copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget for the oracle baseline (0 = skip)")
    ap.add_argument("--event-every", type=int, default=8,
                    help="attach kernel start/stop events to every n-th timed step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (a known byte "
                         "count for scaling the profiler's FETCH_SIZE / WRITE_SIZE) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)      # one elementwise kernel: reads n bytes, writes n
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "repeats": 5}),
          flush=True)


def measured_traffic(workload, which):
    """HBM bytes per launch of kernel `which` from the committed counter summary
    (profiles/<workload>_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by a
    copy-kernel calibration).  None when there is none, or when the kernel sources have
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    src = os.path.join(ROOT, "mixture_experts_layer_route_amd", "csrc")
    for name in sorted(os.listdir(src)):
        h.update(name.encode())
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    if rec.get("sources_sha256") != h.hexdigest() or which not in rec.get("kernels", {}):
        return None
    return rec["kernels"][which]["hbm_bytes_per_launch"]


def kernel_roofline(shape, which, ms, U):
    """Roofline entry of one expert kernel ("gateup" or "down") from its measured
    average duration `ms`: weight-stream bytes for few rows per expert, matrix-core
    flops for large batches."""
    T, H, I, k, S = shape.T, shape.H, shape.I, shape.k, shape.S
    R = T * (k + S)
    mats = 2 if which == "gateup" else 1          # gate+up, or down
    name = ("gate/up expert kernel (SwiGLU fused)" if which == "gateup"
            else "down expert kernel (routing weight applied)")
    if shape.name in ("prefill", "prefill_nvfp4"):
        flops = 2.0 * R * H * I * mats
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(shape.name, which),
                "kernel": name, "kernel_us": round(ms * 1e3, 2),
                "per_launch": f"{flops / 1e9:.2f} GFLOP = 2*R*H*I*{mats}, R={R} rows"}
    wbytes = {"e4m3": 1, "f32": 4, "bf16": 2, "nvfp4": 0.5}[shape.wt]
    if shape.wt == "e4m3":
        scales = mats * (I // 128) * (H // 128) * 4
    elif shape.wt == "nvfp4":
        scales = mats * (I * H // 16 + 4)          # e4m3 per 16 inputs + fp32 per matrix
    else:
        scales = 0
    per_expert = int(mats * I * H * wbytes) + scales
    abytes = U * per_expert
    achieved = abytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(shape.name, which), "kernel": name,
            "kernel_us": round(ms * 1e3, 2),
            "per_launch": f"{abytes} B = {U} touched experts x {per_expert} B of weights"}


def step_roofline(shape, ms, U):
    """The whole step against the same peak (the way the scope table prices a config):
    prefill-sized bf16 work by all expert and router flops, everything else by the
    bytes the method must move (each touched expert's weights once, the router, x, y)."""
    T, H, I, E, k, S = shape.T, shape.H, shape.I, shape.E, shape.k, shape.S
    act = 4 if shape.act == "f32" else 2
    if shape.name in ("prefill", "prefill_nvfp4"):
        flops = 2.0 * T * (k + S) * H * I * 3 + 2.0 * T * E * H
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "per_step": f"{flops / 1e9:.2f} GFLOP (experts 2*R*H*I*3 + router 2*T*E*H)"}
    wbytes = {"e4m3": 1, "f32": 4, "bf16": 2, "nvfp4": 0.5}[shape.wt]
    if shape.wt == "e4m3":
        scales = 3 * (I // 128) * (H // 128) * 4
    elif shape.wt == "nvfp4":
        scales = 3 * (I * H // 16 + 4)
    else:
        scales = 0
    per_expert = int(3 * I * H * wbytes) + scales
    nbytes = U * per_expert + E * H * act + 2 * T * H * act
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "per_step": f"{nbytes} B = {U} touched experts x {per_expert} B + router, x and y"}


def oracle_experts(mo, cpu, f):
    """The oracle's expert set over the synthetic layer's stored weights."""
    nv = sh_nv = None
    if cpu.get("b_gate") is not None:
        nv = tuple(f(cpu[n]) for n in NV_KEYS)
        if cpu.get("sh_b_gate") is not None:
            sh_nv = tuple(f(cpu["sh_" + n]) for n in NV_KEYS)
    return mo.Experts(*(f(cpu[n]) for n in WEIGHT_KEYS), nv=nv, sh_nv=sh_nv)


def blas_threads():
    """Threads numpy's BLAS runs the oracle with."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(shape, cpu, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import moe_oracle as mo
    threads = blas_threads()
    f = lambda t: None if t is None else (t.numpy() if t.dtype.itemsize == 1 else t.float().numpy())
    ex = oracle_experts(mo, cpu, f)
    x, wr, b = f(cpu["x"]), f(cpu["w_router"]), f(cpu["router_bias"])
    n_tok = min(shape.T, 64)
    xs = x[:n_tok]
    t0 = time.perf_counter()
    reps = 0
    while True:
        mo.forward(xs, wr, b, ex, shape.G, shape.Gk, shape.k)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(reps * n_tok / el, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{reps} x oracle forward of the first {n_tok} of {shape.T} tokens "
                      f"(full routing + experts + combine, float64 numpy), {el:.1f} s"}


def run_stack(args):
    """The decoder step's 23 MoE blocks (x_{l+1} = x_l + MoE_l(RMSNorm_l(x_l))) for a
    decode batch, captured in one HIP graph and replayed; the same chain launched eagerly
    beside it.  Each block streams its own copy of the experts from HBM."""
    import torch
    import mixture_experts_layer_route_amd as moe
    import synth
    from oracle import moe_oracle as mo

    shape = synth.WORKLOADS["decode_stack"]
    L = synth.STACK_BLOCKS
    eps = 1e-6
    log(f"workload {shape}; {L} blocks")
    cpu = synth.make_layer(shape)
    base = {k: (None if v is None else v.cuda()) for k, v in cpu.items()}
    blocks = []
    for l in range(L):
        d = {k: (v.clone() if k in WEIGHT_KEYS and v is not None else v) for k, v in base.items()}
        router = synth.make_router(shape.E, shape.H, shape.act, 10_000 + l)
        gamma = synth.make_norm_weight(shape.H, shape.act, 20_000 + l)
        d["w_router"] = router.cuda()
        blocks.append((d, moe.weights_struct(d), gamma.cuda(), router, gamma))
    cfg = moe.make_config(shape.T, shape.H, shape.I, shape.E, shape.G, shape.Gk, shape.k,
                          shape.S, shape.act, shape.wt)
    ws = moe.alloc_workspace(cfg)
    xs = [base["x"].clone()] + [torch.empty_like(base["x"]) for _ in range(L)]
    ids = [torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda") for _ in range(L)]

    def chain():
        for l, (d, wst, g, _, _) in enumerate(blocks):
            moe.forward_residual(cfg, xs[l], g, d, ws, x_out=xs[l + 1], eps=eps, ids=ids[l],
                                 wst=wst)

    chain()
    torch.cuda.synchronize()
    # parity per block on the GPU's own trajectory (oracle forced onto the GPU's ids)
    f = lambda t: t.float().cpu().numpy()
    ex = oracle_experts(mo, cpu, lambda t: None if t is None else
                        (t.numpy() if t.dtype.itemsize == 1 else t.float().numpy()))
    worst, U_tot = 0.0, 0
    for l, (_, _, _, router, gamma) in enumerate(blocks):
        g_ids = ids[l].cpu().numpy()
        U_tot += int(np.unique(g_ids).size)
        ref = mo.residual_layer(f(xs[l]), gamma.float().numpy(), router.float().numpy(), None, ex,
                                shape.G, shape.Gk, shape.k, eps=eps, ids=g_ids)
        e = np.abs(f(xs[l + 1]).astype(np.float64) - f(xs[l]) - ref["y"])
        a = np.abs(ref["x_out"])
        half_step = 0.5 * 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
        worst = max(worst, float(np.linalg.norm(np.maximum(e - half_step, 0.0))
                                 / np.linalg.norm(ref["y"])))
    log(f"parity over {L} blocks: worst rel_l2 of y beyond the bf16 store's rounding "
        f"{worst:.3e}; touched experts {U_tot}")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    for _ in range(W):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(end) / K
    start.record()
    for _ in range(K):
        chain()
    end.record()
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / K
    log(f"stack step {ms_graph * 1e3:.1f} us in one graph ({ms_graph * 1e3 / L:.2f} us per "
        f"block); eager launches {ms_eager * 1e3:.1f} us")
    per_expert = 3 * shape.I * shape.H * 2
    abytes = U_tot * per_expert + L * (shape.E * shape.H * 2 + shape.H * 2 + 2 * shape.T * shape.H * 2)
    achieved = abytes / (ms_graph * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(shape.T / (ms_graph * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_graph, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_stack", "blocks": L, "T": shape.T, "H": shape.H,
                   "I": shape.I, "E": shape.E, "G": shape.G, "Gk": shape.Gk, "k": shape.k,
                   "touched_experts": U_tot},
        "us_per_block": round(ms_graph * 1e3 / L, 2),
        "ms_per_step_eager_launches": round(ms_eager, 5),
        "parity_rel_l2_worst_block": float(f"{worst:.3e}"),   # beyond the bf16 store rounding
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": f"whole step: {L} blocks x (norm+logits, gate/up, down+combine+"
                               "residual) in one graph",
                     "per_launch": f"{abytes} B = {U_tot} touched experts x {per_expert} B + "
                                   "router, norm weight and rows per block"},
    }
    if args.cpu_seconds > 0:
        t0 = time.perf_counter()
        reps = 0
        xin = f(xs[0])
        while True:
            xc = xin
            for l, (_, _, _, router, gamma) in enumerate(blocks):
                xc = mo.residual_layer(xc, gamma.float().numpy(), router.float().numpy(), None,
                                       ex, shape.G, shape.Gk, shape.k, eps=eps)["x_out"]
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(reps * shape.T / el, 3), "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{reps} x the oracle's {L}-block step on the same "
                                         f"{shape.T} tokens (float64 numpy), {el:.1f} s"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is built "
              "and measured on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.workload == "decode_stack":
        run_stack(args)
        return
    import torch
    import mixture_experts_layer_route_amd as moe
    import synth
    from oracle import moe_oracle as mo

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    shape = synth.WORKLOADS[args.workload]
    nsets = args.sets or DEFAULT_SETS[args.workload]
    log(f"workload {shape}; weight sets {nsets}")
    cpu = synth.make_layer(shape)
    dev = {k: (None if v is None else v.cuda()) for k, v in cpu.items()}
    sets = [dev]
    for _ in range(nsets - 1):
        sets.append({k: (v.clone() if (k in WEIGHT_KEYS + NV_KEYS or k.startswith("sh_"))
                         and v is not None else v)
                     for k, v in dev.items()})
    wsts = [moe.weights_struct(s) for s in sets]
    cfg = moe.make_config(shape.T, shape.H, shape.I, shape.E, shape.G, shape.Gk, shape.k,
                          shape.S, shape.act, shape.wt)
    ws = moe.alloc_workspace(cfg)
    x = dev["x"]
    y = torch.empty((shape.T, shape.H), dtype=x.dtype, device="cuda")
    ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")

    # parity of what is timed: set 0, sampled tokens against the oracle on the GPU's routing
    moe.forward(cfg, x, dev, ws, y=y, ids=ids, wts=wts, wst=wsts[0])
    torch.cuda.synchronize()
    g_ids = ids.cpu().numpy()
    U = int(np.unique(g_ids).size) + shape.S
    rng = np.random.default_rng(0)
    sample = np.arange(shape.T) if shape.T <= 16 else np.unique(
        np.concatenate([[0, shape.T - 1], rng.choice(shape.T, 14, replace=False)]))
    f = lambda t: None if t is None else (t.numpy() if t.dtype.itemsize == 1 else t.float().numpy())
    ex = oracle_experts(mo, cpu, f)
    l64 = mo.router_logits(f(cpu["x"]), f(cpu["w_router"]), f(cpu["router_bias"]))
    w64 = mo.renormalise(mo.gate_scores(l64[sample]), g_ids[sample])
    ref = mo.forward_tokenmajor(f(cpu["x"])[sample], ex, g_ids[sample], w64)
    err = mo.rel_l2(y.float().cpu().numpy()[sample], ref)
    log(f"parity on {len(sample)} tokens: rel_l2 {err:.3e}; unique experts {U}")

    K, W = args.steps, args.warmup
    for i in range(W):
        moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
    # start/stop events attached to the gate/up and down kernel dispatches of every
    # n-th timed step (each attached event costs a few microseconds of queue time)
    every = max(1, args.event_every)
    timed = list(range(0, K, every))
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(moe.TIMED_EVENTS)] for i in timed}
    for row in ev.values():
        for e in row:
            e.record()
    torch.cuda.synchronize()
    arrays = {i: (ctypes.c_void_p * moe.TIMED_EVENTS)(*[e.cuda_event for e in row])
              for i, row in ev.items()}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        if i in arrays:
            moe.forward_timed(cfg, x, wsts[i % nsets], ws, y, arrays[i])
        else:
            moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    samples = {"gateup": [r[0].elapsed_time(r[1]) for r in ev.values()],
               "down": [r[2].elapsed_time(r[3]) for r in ev.values()]}
    kern_ms = {n: float(np.mean(v)) for n, v in samples.items()}
    kern_pct = {n: [round(float(np.percentile(v, q)) * 1e3, 2) for q in (10, 50, 90)]
                for n, v in samples.items()}
    # the same steps with no events at all
    start.record()
    for i in range(K):
        moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
    end.record()
    torch.cuda.synchronize()
    ms_plain = start.elapsed_time(end) / K
    log(f"step {ms_per_step * 1e3:.2f} us (untimed kernels {ms_plain * 1e3:.2f} us); kernels: "
        + ", ".join(f"{n} {v * 1e3:.2f} us" for n, v in kern_ms.items()))
    tokens_per_s = shape.T / (ms_per_step * 1e-3)
    which = max(kern_ms, key=kern_ms.get)
    roof = kernel_roofline(shape, which, kern_ms[which], U)

    res = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3+bf16", "nvfp4": "nvfp4+bf16"}[shape.wt],
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "H": shape.H, "I": shape.I,
                   "E": shape.E, "G": shape.G, "Gk": shape.Gk, "k": shape.k, "S": shape.S,
                   "weight_sets": nsets, "touched_experts": U},
        "kernel_us": {n: round(v * 1e3, 2) for n, v in kern_ms.items()},
        "kernel_us_p10_p50_p90": kern_pct,
        "kernel_events_on_steps": f"every {every}th ({len(timed)} of {K})",
        "ms_per_step_without_kernel_events": round(ms_plain, 5),
        "parity_rel_l2": float(f"{err:.3e}"),
        "roofline": roof,
        "step_roofline": step_roofline(shape, ms_per_step, U),
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(shape, cpu, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
