"""Documented contracts of the C ABI on the GPU.

* Concurrent calls on different streams with distinct workspaces give the same bits as
  the same calls run alone (the library keeps no device state; TensorFold #1247, list
  "What #874's CUDA path now covers", holds its own path to concurrent == solo).
* moe_combine called directly with shared experts and bf16 output: the fixed-order fp32
  sum of reading R7, rounded once to bf16.
* Chunked == whole (the same list's equivalence tests): each token's output depends only
  on that token, so a batch run in two pieces gives the same bits as the whole batch, as
  long as both pieces take the same kernels (matrix-core experts, the same router-logit
  tiles).
* The largest expert count the ABI accepts, E + S = 1024: the permutation (whose total
  row count then lies past the last thread of the scan blocks) and whole layers on
  every path (decode kernels, small-batch route+permute, skinny and matrix-core
  expert kernels)."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from tests.helpers import config_for, to_device
from tests.test_gpu_parity import _forward_check

pytestmark = pytest.mark.gpu

S_ = synth.LayerShape


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


def test_concurrent_streams_equal_solo(moe):
    print("case: concurrent == solo", flush=True)
    jobs = []
    for name, T in (("decode", None), ("prefill", 700), ("fp8", 300), ("inkling", 40)):
        base = synth.WORKLOADS[name]
        shape = base if T is None else base.with_tokens(T)
        cpu = synth.make_layer(shape)
        dev = to_device(cpu)
        cfg = config_for(shape)
        jobs.append((shape, dev, cfg, moe.weights_struct(dev)))
    # solo: one call at a time on the default stream
    solo = []
    for shape, dev, cfg, wst in jobs:
        ws = moe.alloc_workspace(cfg)
        solo.append(moe.forward(cfg, dev["x"], None, ws, wst=wst).clone())
        torch.cuda.synchronize()
    # concurrent: each job on its own stream and workspace, several rounds with no sync
    streams = [torch.cuda.Stream() for _ in jobs]
    wss = [moe.alloc_workspace(cfg) for _, _, cfg, _ in jobs]
    outs = [[torch.empty_like(s) for _ in range(6)] for s in solo]
    torch.cuda.synchronize()
    for rnd in range(6):
        for j, (shape, dev, cfg, wst) in enumerate(jobs):
            with torch.cuda.stream(streams[j]):
                moe.forward(cfg, dev["x"], None, wss[j], y=outs[j][rnd], wst=wst)
    torch.cuda.synchronize()
    for j, (shape, _, _, _) in enumerate(jobs):
        for rnd in range(6):
            assert torch.equal(outs[j][rnd], solo[j]), (shape.name, rnd)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_combine_direct_shared_experts(moe, out):
    print("case: combine direct S=2", out, flush=True)
    T, H, E, k, S = 150, 512, 32, 6, 2
    rng = np.random.default_rng(81)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    w = w.astype(np.float32)
    R = T * (k + S)
    y_perm = rng.standard_normal((R, H)).astype(np.float32)
    cfg = moe.make_config(T, H, 128, E, 1, 1, k, S, out, out)
    ws = moe.alloc_workspace(cfg)
    off, rt, inv = moe.permute(cfg, torch.from_numpy(ids).cuda(), ws)
    y = moe.combine(cfg, torch.from_numpy(y_perm).cuda(), off, inv, torch.from_numpy(w).cuda(),
                    torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    o_off, _, o_inv = mo.permute(ids, E, S)
    assert np.array_equal(off.cpu().numpy(), o_off) and np.array_equal(inv.cpu().numpy(), o_inv)
    ref = mo.combine(y_perm, o_off, o_inv, w, S)
    got = y.float().cpu().numpy().astype(np.float64)
    # fp32 sum of k + S terms in a fixed order: error below (k+S) * 2^-24 * sum |terms|
    mag = np.zeros_like(ref)
    for j in range(k):
        mag += np.abs(w[:, j:j + 1].astype(np.float64) * y_perm[o_inv[:, j]])
    for s in range(S):
        mag += np.abs(y_perm[o_off[E + s]:o_off[E + s] + T])
    bound = (k + S) * 2.0 ** -24 * mag
    if out == "bf16":
        a = np.abs(ref)
        half_step = 0.5 * 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
        bound = bound * (1 + 2.0 ** -8) + np.where(a > 0, half_step, 0) * (1 + 2.0 ** -7)
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("T,E,k,S", [(300, 1024, 8, 0), (2000, 1024, 4, 0), (3000, 1022, 8, 2),
                                     (40, 1023, 6, 1)])
def test_permute_1024_experts(moe, T, E, k, S):
    print("case: permute E+S=1024", T, E, k, S, flush=True)
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    for t in range(0, T, 3):                   # the last routed expert gets rows
        if E - 1 not in ids[t]:
            ids[t, 0] = E - 1
    cfg = moe.make_config(T, 256, 128, E, 1, 1, k, S, "bf16", "bf16")
    ws = moe.alloc_workspace(cfg)
    off, rt, inv = moe.permute(cfg, torch.from_numpy(ids).cuda(), ws)
    torch.cuda.synchronize()
    o_off, o_rt, o_inv = mo.permute(ids, E, S)
    assert int(o_off[-1]) == T * (k + S)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(rt.cpu().numpy(), o_rt)
    assert np.array_equal(inv.cpu().numpy(), o_inv)


CASES_1024 = [
    # name, T, H, I, E, G, Gk, k, S, act, wt, x_dist, bias_std, seed
    ("e1024_dec", 4, 256, 128, 1024, 1, 1, 8, 0, "bf16", "bf16", "normal", 0.0, 91),
    ("e1022s2_dec", 3, 256, 128, 1022, 2, 1, 6, 2, "bf16", "bf16", "normal", 0.0, 92),
    ("e1024_small", 40, 256, 128, 1024, 1, 1, 6, 0, "bf16", "bf16", "normal", 0.0, 93),
    ("e1022s2_small", 40, 256, 128, 1022, 2, 1, 6, 2, "bf16", "bf16", "normal", 0.0, 94),
    ("e1022s2_skinny", 600, 256, 128, 1022, 2, 2, 8, 2, "bf16", "bf16", "normal", 0.5, 95),
    ("e1024_mfma", 1200, 256, 128, 1024, 8, 4, 8, 0, "bf16", "bf16", "normal", 0.5, 96),
    ("e1022s2_fp8", 600, 256, 128, 1022, 2, 2, 8, 2, "bf16", "e4m3", "normal", 0.5, 97),
]


@pytest.mark.parametrize("case", CASES_1024, ids=[c[0] for c in CASES_1024])
def test_forward_1024_experts(moe, case):
    print("case: forward E+S=1024", case, flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


# splits whose pieces stay on the whole batch's kernels: matrix-core experts (more than 8
# rows per expert on average) and the 32 x 32 router-logit tiles
@pytest.mark.parametrize("name,T,split", [("prefill", 3000, 1500), ("prefill", 3000, 1100),
                                          ("fp8", 2048, 1024), ("inkling", 1200, 600),
                                          ("prefill_nvfp4", 3000, 1300),
                                          ("prefill_mxfp4", 3000, 1700)])
def test_chunked_equals_whole(moe, name, T, split):
    print("case: chunked == whole", name, T, split, flush=True)
    shape = synth.WORKLOADS[name].with_tokens(T)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    cfg = config_for(shape)
    whole = moe.forward(cfg, dev["x"], dev, moe.alloc_workspace(cfg))
    parts = []
    for a, b in ((0, split), (split, T)):
        pc = config_for(shape.with_tokens(b - a))
        parts.append(moe.forward(pc, dev["x"][a:b].contiguous(), dev, moe.alloc_workspace(pc)))
    torch.cuda.synchronize()
    got = torch.cat(parts)
    diff = int((got.view(torch.int16) != whole.view(torch.int16)).sum())
    print(f"{name} T={T} split {split}: {diff} elements differ")
    assert diff == 0
