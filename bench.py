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
                "prefill_nvfp4": 4, "decode_mxfp4": 16, "prefill_mxfp4": 4, "decode_stack": 1}
PREFILL = ("prefill", "prefill_nvfp4", "prefill_mxfp4")


def mfma_peak(shape):
    """Dense matrix-core peak of the workload's contraction: MXFP4 experts multiply fp4
    weights by fp8 activations on the block-scaled MFMA (the fp8 rate); the other prefill
    layers run bf16 MFMAs."""
    return FP8_PEAK_TFLOPS if shape.wt == "mxfp4" else BF16_PEAK_TFLOPS


def weight_bytes(shape, mats):
    """Bytes of `mats` expert matrices of one expert, with their scales."""
    I, H = shape.I, shape.H
    wbytes = {"e4m3": 1, "f32": 4, "bf16": 2, "nvfp4": 0.5, "mxfp4": 0.5}[shape.wt]
    if shape.wt == "e4m3":
        scales = mats * (I // 128) * (H // 128) * 4
    elif shape.wt == "nvfp4":
        scales = mats * (I * H // 16 + 4)          # e4m3 per 16 inputs + fp32 per matrix
    elif shape.wt == "mxfp4":
        scales = mats * (I * H // 32)              # e8m0 per 32 inputs
    else:
        scales = 0
    return int(mats * I * H * wbytes) + scales


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "fp8", "inkling", "decode_nvfp4",
                             "prefill_nvfp4", "decode_mxfp4", "prefill_mxfp4", "decode_stack",
                             "paged"])
    ap.add_argument("--sets", type=int, default=0, help="weight copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host time budget for the oracle baseline (0 = skip)")
    ap.add_argument("--event-every", type=int, default=8,
                    help="attach kernel start/stop events to every n-th timed step")
    ap.add_argument("--no-prefill-leg", action="store_true",
                    help="decode workload only: skip the 8192-token prefill layer that the "
                         "default line carries as its second measurement")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor BLAS (torch.bmm / torch.mm, bf16) on the prefill "
                         "layer's expert-GEMM shapes with equal rows per expert, as a ceiling for "
                         "the grouped kernels, and exit")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure what this GPU achieves on plain work (a 4 GiB streaming "
                         "read, a 4 GiB copy, a large bf16 GEMM through the vendor BLAS), the "
                         "context for the roofline fractions against the published peaks, and exit")
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


def library_gemm(steps=20):
    """The vendor BLAS on the prefill layer's expert GEMMs (bf16, fp32 accumulation) with
    the 65,536 routed rows split evenly over the 128 experts (512 each, no padding, no
    gather, no epilogue): batched gate/up [E,512,H] x [E,H,2I] and down [E,512,I] x
    [E,I,H], and the same flops as one dense GEMM.  A reference point for the grouped
    kernels, which also gather rows, pad ragged tiles and fuse SwiGLU / the weights."""
    import torch
    import synth
    sh = synth.WORKLOADS["prefill"]
    E, H, I, R = sh.E, sh.H, sh.I, sh.T * sh.k
    M = R // E
    g = torch.Generator(device="cuda").manual_seed(7)
    def rnd(*dims):
        return (torch.randn(*dims, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    cases = {
        "gateup_bmm": (lambda a, b: torch.bmm(a, b), rnd(E, M, H), rnd(E, H, 2 * I), 2 * R * H * 2 * I),
        "down_bmm": (lambda a, b: torch.bmm(a, b), rnd(E, M, I), rnd(E, I, H), 2 * R * I * H),
        "gateup_dense_mm": (lambda a, b: torch.mm(a, b), rnd(R, H), rnd(H, 2 * I), 2 * R * H * 2 * I),
        "down_dense_mm": (lambda a, b: torch.mm(a, b), rnd(R, I), rnd(I, H), 2 * R * I * H),
    }
    out = {"library": f"torch {torch.__version__} (hipBLASLt / rocBLAS)", "rows_per_expert": M}
    for name, (fn, a, b, flops) in cases.items():
        for _ in range(5):
            fn(a, b)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn(a, b)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / steps
        tf = flops / us / 1e6
        out[name] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        log(name, out[name])
    print(json.dumps(out), flush=True)


def peaks(steps=10):
    """Achieved rates on plain work, next to the published peaks: HBM read (a sum over a
    4 GiB bf16 tensor), HBM copy (4 GiB read + 4 GiB written), and a 8192^3 bf16 GEMM."""
    import torch
    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / steps       # seconds per call
    n = 4 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    t_read = timed(lambda: torch.sum(src, dim=0, dtype=torch.float32, out=acc))
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    t_mm = timed(lambda: torch.mm(a, b))
    out = {"hbm_read_GBs": round(n / t_read / 1e9, 1), "hbm_copy_GBs": round(2 * n / t_copy / 1e9, 1),
           "bf16_gemm_8192_TFLOPs": round(2 * m ** 3 / t_mm / 1e12, 1),
           "published": {"hbm_GBs": HBM_PEAK_GBS, "bf16_TFLOPs": BF16_PEAK_TFLOPS}}
    print(json.dumps(out), flush=True)


def measured_traffic(workload, which):
    """HBM bytes per launch of kernel `which` from the committed counter summary
    (profiles/<workload>_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE, scaled by a
    copy-kernel calibration).  None when there is none, or when the kernel sources have
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != sources_sha256() or which not in rec.get("kernels", {}):
        return None
    return rec["kernels"][which]["hbm_bytes_per_launch"]


def sources_sha256():
    """SHA-256 over the kernel sources (file names and contents, in name order)."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "mixture_experts_layer_route_amd", "csrc")
    for name in sorted(os.listdir(src)):
        h.update(name.encode())
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_roofline(shape, which, ms, U):
    """Roofline entry of one expert kernel ("gateup" or "down") from its measured
    average duration `ms`: weight-stream bytes for few rows per expert, matrix-core
    flops for large batches."""
    T, H, I, k, S = shape.T, shape.H, shape.I, shape.k, shape.S
    R = T * (k + S)
    mats = 2 if which == "gateup" else 1          # gate+up, or down
    name = ("gate/up expert kernel (SwiGLU fused)" if which == "gateup"
            else "down expert kernel (routing weight applied)")
    if shape.name in PREFILL:
        flops = 2.0 * R * H * I * mats
        achieved = flops / (ms * 1e-3) / 1e12
        peak = mfma_peak(shape)
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(shape.name, which),
                "kernel": name, "kernel_us": round(ms * 1e3, 2),
                "per_launch": f"{flops / 1e9:.2f} GFLOP = 2*R*H*I*{mats}, R={R} rows"}
    per_expert = weight_bytes(shape, mats)
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
    if shape.name in PREFILL:
        flops = 2.0 * T * (k + S) * H * I * 3 + 2.0 * T * E * H
        achieved = flops / (ms * 1e-3) / 1e12
        peak = mfma_peak(shape)
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "per_step": f"{flops / 1e9:.2f} GFLOP (experts 2*R*H*I*3 + router 2*T*E*H)"}
    per_expert = weight_bytes(shape, 3)
    nbytes = U * per_expert + E * H * act + 2 * T * H * act
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "per_step": f"{nbytes} B = {U} touched experts x {per_expert} B + router, x and y"}


def oracle_experts(mo, cpu, f):
    """The oracle's expert set over the synthetic layer's stored weights."""
    nv = sh_nv = mx = sh_mx = None
    if cpu.get("b_gate") is not None and cpu.get("g_gate") is None:        # MXFP4
        mx = tuple(f(cpu[n]) for n in ("b_gate", "b_up", "b_down"))
        if cpu.get("sh_b_gate") is not None:
            sh_mx = tuple(f(cpu["sh_" + n]) for n in ("b_gate", "b_up", "b_down"))
    elif cpu.get("b_gate") is not None:
        nv = tuple(f(cpu[n]) for n in NV_KEYS)
        if cpu.get("sh_b_gate") is not None:
            sh_nv = tuple(f(cpu["sh_" + n]) for n in NV_KEYS)
    return mo.Experts(*(f(cpu[n]) for n in WEIGHT_KEYS), nv=nv, sh_nv=sh_nv, mx=mx, sh_mx=sh_mx)


def blas_info():
    """(library, threads) of the BLAS numpy runs the oracle's matrix products with."""
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            name = f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
            return name, int(i.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", os.cpu_count()


def host_cores():
    return len(os.sched_getaffinity(0))


def baseline_entry(value, sample):
    """cpu_baseline record: `cores` is the threads the oracle ran on (its BLAS threads;
    the rest of the oracle is single-threaded numpy), beside the host's core count."""
    blas, threads = blas_info()
    return {"value": value, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample, "host_cores": host_cores(), "blas": blas,
            "blas_threads": int(threads)}


def cpu_baseline(shape, cpu, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the same workload."""
    from oracle import moe_oracle as mo
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
    return baseline_entry(
        round(reps * n_tok / el, 3),
        f"{reps} x oracle forward of the first {n_tok} of {shape.T} tokens "
        f"(full routing + experts + combine, float64 numpy), {el:.1f} s")


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
        res["cpu_baseline"] = baseline_entry(
            round(reps * shape.T / el, 3),
            f"{reps} x the oracle's {L}-block step on the same {shape.T} tokens "
            f"(float64 numpy), {el:.1f} s")
    print(json.dumps(res), flush=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence
SETTLE_S = 0.25                  # seconds of back-to-back layer runs before the warm-up


class HipTimer:
    """Timing-only HIP events created with hipEventDisableSystemFence: recording one skips
    the system-scope release a default event performs (a cache write-back and invalidate),
    so events attached to the kernels of a timed step cost little and disturb nothing after
    them.  They are read only after a device synchronisation.  Calls go to the HIP runtime
    that torch (and the MoE library) already use in this process."""

    def __init__(self):
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        hip = ctypes.CDLL(path)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip, self.events = hip, []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} returned HIP error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self._check(self.hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")
        self.events.append(e)
        return e

    def record(self, e, stream):
        self._check(self.hip.hipEventRecord(e, ctypes.c_void_p(stream)), "hipEventRecord")

    def ms(self, a, b):
        out = ctypes.c_float()
        self._check(self.hip.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return float(out.value)

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def measure(workload, nsets, K, W, event_every):
    """Time K steps (after W warm-up steps) of one workload's layer, weights rotating over
    `nsets` copies, with kernel events on every `event_every`-th step; parity of what is
    timed on sampled tokens.  Returns (partial JSON record, shape, CPU layer)."""
    import torch
    import mixture_experts_layer_route_amd as moe
    import synth
    from oracle import moe_oracle as mo

    shape = synth.WORKLOADS[workload]
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
    # (the output is kept here and checked on the host after the timed loops, so that no
    # host-only work separates the warm-up from the timed steps)
    moe.forward(cfg, x, dev, ws, y=y, ids=ids, wts=wts, wst=wsts[0])
    torch.cuda.synchronize()
    g_ids = ids.cpu().numpy()
    y_parity = y.float().cpu().numpy()
    U = int(np.unique(g_ids).size) + shape.S

    # The GPU's clocks follow its load: after host-only work it runs the first steps
    # slower for a while (a 20-step prefill timing after 5 warm-up steps read 9% slow).
    # So before the warm-up steps the layer runs back to back for SETTLE_S seconds;
    # these runs are reported ("settle") and are neither warm-up nor timed steps.
    t_settle, n_settle = time.time(), 0
    while time.time() - t_settle < SETTLE_S:
        for i in range(8):
            moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
        torch.cuda.synchronize()
        n_settle += 8
    t_settle = time.time() - t_settle

    for i in range(W):
        moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
    # start/stop events attached to the gate/up and down kernel dispatches of every
    # n-th timed step (each attached event costs a few microseconds of queue time)
    every = max(1, event_every)
    timed = list(range(every - 1, K, every)) or [K - 1]     # the last of every `every` steps
    hipt = HipTimer()
    stream = torch.cuda.current_stream().cuda_stream
    ev = {i: [hipt.event() for _ in range(moe.TIMED_EVENTS)] for i in timed}
    for row in ev.values():
        for e in row:
            hipt.record(e, stream)
    torch.cuda.synchronize()
    arrays = {i: (ctypes.c_void_p * moe.TIMED_EVENTS)(*[e.value for e in row])
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
    samples = {"gateup": [hipt.ms(r[0], r[1]) for r in ev.values()],
               "down": [hipt.ms(r[2], r[3]) for r in ev.values()]}
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
    # the spread over single steps: up to 100 more steps, each between its own event pair
    n1 = min(K, 100)
    pairs = [(hipt.event(), hipt.event()) for _ in range(n1)]
    for i, (a, b) in enumerate(pairs):
        hipt.record(a, stream)
        moe.forward(cfg, x, None, ws, y=y, wst=wsts[i % nsets])
        hipt.record(b, stream)
    torch.cuda.synchronize()
    step_us = [hipt.ms(a, b) * 1e3 for a, b in pairs]
    hipt.close()
    step_pct = [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)]
    log(f"step {ms_per_step * 1e3:.2f} us (untimed kernels {ms_plain * 1e3:.2f} us); kernels: "
        + ", ".join(f"{n} {v * 1e3:.2f} us" for n, v in kern_ms.items()))
    rng = np.random.default_rng(0)
    sample = np.arange(shape.T) if shape.T <= 16 else np.unique(
        np.concatenate([[0, shape.T - 1], rng.choice(shape.T, 14, replace=False)]))
    f = lambda t: None if t is None else (t.numpy() if t.dtype.itemsize == 1 else t.float().numpy())
    ex = oracle_experts(mo, cpu, f)
    l64 = mo.router_logits(f(cpu["x"]), f(cpu["w_router"]), f(cpu["router_bias"]))
    w64 = mo.renormalise(mo.gate_scores(l64[sample]), g_ids[sample])
    ref = mo.forward_tokenmajor(f(cpu["x"])[sample], ex, g_ids[sample], w64)
    err = mo.rel_l2(y_parity[sample], ref)
    log(f"parity on {len(sample)} tokens: rel_l2 {err:.3e}; unique experts {U}")
    tokens_per_s = shape.T / (ms_per_step * 1e-3)
    which = max(kern_ms, key=kern_ms.get)
    roof = kernel_roofline(shape, which, kern_ms[which], U)

    res = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "e4m3": "e4m3+bf16", "nvfp4": "nvfp4+bf16",
                  "mxfp4": "mxfp4+mxfp8"}[shape.wt],
        "data": "synthetic",
        "config": {"workload": shape.name, "T": shape.T, "H": shape.H, "I": shape.I,
                   "E": shape.E, "G": shape.G, "Gk": shape.Gk, "k": shape.k, "S": shape.S,
                   "weight_sets": nsets, "touched_experts": U},
        "kernel_us": {n: round(v * 1e3, 2) for n, v in kern_ms.items()},
        "kernel_us_p10_p50_p90": kern_pct,
        "kernel_events_on_steps": f"every {every}th ({len(timed)} of {K})",
        "settle": {"seconds": round(t_settle, 3), "runs": n_settle},
        "ms_per_step_without_kernel_events": round(ms_plain, 5),
        "step_us_p10_p50_p90": step_pct,
        "step_us_samples": f"{n1} single steps, one event pair each",
        "parity_rel_l2": float(f"{err:.3e}"),
        "roofline": roof,
        "step_roofline": step_roofline(shape, ms_per_step, U),
    }
    return res, shape, cpu


HOST_LINK_PEAK_GBS = 64.0        # PCIe 5.0 x16 between the MI355X and its host, one direction


def run_paged(args):
    """Single-stream decode through the 23 MoE blocks of the stack with every block's
    routed experts in pinned host memory and an HBM arena of N slots per block (the
    HelloSun/ling30tiny RAM-limit table measured on one MI355X): tokens/s, hot rate,
    MiB copied from the host per token and the host-link rate, per arena size."""
    import torch
    import mixture_experts_layer_route_amd as moe
    import synth

    base = synth.WORKLOADS["decode"]
    shape = synth.LayerShape("paged", T=1, H=base.H, I=base.I, E=base.E, G=base.G, Gk=base.Gk,
                             k=base.k, S=0, act="bf16", wt="bf16", x_dist="rms", bias_std=1.0,
                             seed=8)
    L = synth.STACK_BLOCKS
    log(f"workload {shape}; {L} blocks, experts in pinned host memory")
    cpu = synth.make_layer(shape)
    mats = ("w_gate", "w_up", "w_down")
    blocks = []
    for l in range(L):
        store = {k: torch.empty(cpu[k].shape, dtype=cpu[k].dtype, pin_memory=True).copy_(cpu[k])
                 for k in mats}                                    # one store per block
        router = synth.make_router(shape.E, shape.H, shape.act, 10_000 + l).cuda()
        bias = torch.from_numpy(np.random.default_rng(30_000 + l).standard_normal(
            shape.E, dtype=np.float32)).cuda()
        blocks.append((store, moe.weights_struct_host(store), router, bias))
    cfg = moe.make_config(shape.T, shape.H, shape.I, shape.E, shape.G, shape.Gk, shape.k,
                          shape.S, shape.act, shape.wt)
    rng = np.random.default_rng(9)
    pool = torch.from_numpy(rng.standard_normal((256, shape.H), dtype=np.float32))
    pool = (pool / pool.pow(2).mean(dim=1, keepdim=True).sqrt()).to(torch.bfloat16).cuda()
    expert_bytes = 3 * shape.I * shape.H * 2
    K, W = min(args.steps, 64), min(args.warmup, 32)
    sweep = []
    for N in (8, 16, 32, 64, 128):
        arenas, states = [], []
        for l in range(L):
            ar = {"w_gate": torch.empty((N, shape.I, shape.H), dtype=torch.bfloat16, device="cuda"),
                  "w_up": torch.empty((N, shape.I, shape.H), dtype=torch.bfloat16, device="cuda"),
                  "w_down": torch.empty((N, shape.H, shape.I), dtype=torch.bfloat16, device="cuda"),
                  "w_router": blocks[l][2], "router_bias": blocks[l][3]}
            arenas.append((ar, moe.weights_struct(ar)))
            states.append(moe.alloc_pager_state(cfg, N))
        ws = moe.paged_workspace(cfg, N)
        y = torch.empty((1, shape.H), dtype=torch.bfloat16, device="cuda")

        def token(i):
            for l in range(L):
                x = pool[(i * L + l) % pool.shape[0]].view(1, -1)
                moe.forward_paged(cfg, x, blocks[l][1], arenas[l][1], N, states[l], ws, y=y)

        for i in range(W):
            token(i)
        torch.cuda.synchronize()
        before = [moe.pager_tables(cfg, N, st) for st in states]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(W, W + K):
            token(i)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / K
        after = [moe.pager_tables(cfg, N, st) for st in states]
        d = {c: sum(a[c] - b[c] for a, b in zip(after, before)) for c in moe.PAGER_COUNTERS}
        rec = {"slots_per_block": N, "arena_GiB": round(L * N * expert_bytes / 2 ** 30, 3),
               "tokens_per_s": round(1e3 / ms, 2), "ms_per_token": round(ms, 4),
               "hot_rate": round(d["hits"] / max(1, d["lookups"]), 4),
               "MiB_per_token_from_host": round(d["bytes_copied"] / K / 2 ** 20, 2),
               "host_GB_per_s": round(d["bytes_copied"] / K / (ms * 1e-3) / 1e9, 2)}
        log(json.dumps(rec))
        sweep.append(rec)
        del arenas, states, ws
        torch.cuda.empty_cache()
    mid = next(r for r in sweep if r["slots_per_block"] == 32)
    link = max(r["host_GB_per_s"] for r in sweep)
    res = {
        "metric": METRIC, "value": mid["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": mid["ms_per_token"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "paged", "blocks": L, "T": 1, "H": shape.H, "I": shape.I,
                   "E": shape.E, "G": shape.G, "Gk": shape.Gk, "k": shape.k,
                   "router_bias_std": shape.bias_std, "slots_per_block": 32,
                   "store": "pinned host memory, one copy of the block's experts per block"},
        "arena_sweep": sweep,
        "roofline": {"bound": "host_link", "achieved": link, "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(link / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                     "kernel": "expert copies host -> HBM (k_pager_copy), best arena size",
                     "per_launch": f"misses x {expert_bytes} B per expert"},
    }
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
    if args.library_gemm:
        library_gemm()
        return
    if args.peaks:
        peaks()
        return
    if args.workload == "decode_stack":
        run_stack(args)
        return
    if args.workload == "paged":
        run_paged(args)
        return
    import torch
    import mixture_experts_layer_route_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    res, shape, cpu = measure(args.workload, args.sets or DEFAULT_SETS[args.workload], args.steps,
                              args.warmup, args.event_every)
    if args.workload == "decode" and not args.no_prefill_leg:
        # the metric's second half: the 8192-token prefill layer, timed the same way
        leg, _, _ = measure("prefill", DEFAULT_SETS["prefill"], min(args.steps, 50),
                            min(args.warmup, 10), args.event_every)
        res["prefill_leg"] = {k: leg[k] for k in (
            "value", "unit", "ms_per_step", "steps", "warmup", "config", "kernel_us",
            "ms_per_step_without_kernel_events", "step_us_p10_p50_p90", "settle", "parity_rel_l2",
            "roofline", "step_roofline")}
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(shape, cpu, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
