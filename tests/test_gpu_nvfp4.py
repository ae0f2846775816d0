"""GPU parity of the layer with NVFP4 experts (4-bit E2M1 codes, an e4m3 scale per
16 inputs, an fp32 scale per expert matrix) against the float64 oracle on the same
stored codes, on the decode workload, its token-count edges, shared experts, the
Inkling-shaped router, hidden/intermediate sizes that leave lanes of the 16-lane
rows idle, and a skewed router; then batches beyond the decode kernels (the
expert-major kernels, on both permutation paths) and the expert-FFN entry point.  Same bar as the other layers: exact ids where the
logit margin is clear, rel L2 of y within the bf16 bound."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from tests.helpers import config_for, np_exact, oracle_experts, to_device
from tests.test_gpu_parity import _forward_check, full_size_check

pytestmark = pytest.mark.gpu

S_ = synth.LayerShape


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


_CACHE = {}


def _decode_layer(T=None, seed=None):
    base = synth.WORKLOADS["decode_nvfp4"]
    shape = base if T is None else base.with_tokens(T, seed)
    if shape not in _CACHE:
        cpu = synth.make_layer(shape)
        _CACHE.clear()
        _CACHE[shape] = (cpu, to_device(cpu))
    return (shape,) + _CACHE[shape]


@pytest.mark.parametrize("T,seed", [(None, None), (1, 41), (16, 42), (9, 43)])
def test_forward_nvfp4_decode(moe, T, seed):
    print("case: nvfp4 decode", T, seed, flush=True)
    shape, cpu, dev = _decode_layer(T, seed)
    _forward_check(moe, shape, cpu, dev)


CASES = [
    # name, T, H, I, E, G, Gk, k, S, act, wt, x_dist, bias_std, seed
    ("nv_ling_sh", 5, 1536, 512, 128, 8, 4, 8, 2, "bf16", "nvfp4", "rms", 0.0, 51),
    ("nv_inkling", 8, 1024, 256, 256, 1, 1, 6, 2, "bf16", "nvfp4", "normal", 0.0, 52),
    ("nv_ragged", 3, 640, 384, 64, 4, 2, 4, 0, "bf16", "nvfp4", "rms", 0.3, 53),   # idle lanes
    ("nv_i1024", 6, 512, 1024, 32, 1, 1, 4, 1, "bf16", "nvfp4", "normal", 0.0, 54),
    ("nv_g64", 3, 512, 256, 256, 64, 8, 16, 0, "bf16", "nvfp4", "rms", 0.0, 55),
    ("nv_h2048", 12, 2048, 256, 16, 4, 2, 4, 0, "bf16", "nvfp4", "rms", 0.0, 56),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_nvfp4_edge(moe, case):
    print("case: nvfp4 edge", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_forward_nvfp4_skewed_router(moe):
    """Every token prefers the same eight experts (all in group 0)."""
    print("case: nvfp4 skew", flush=True)
    shape = S_("nv_skew", 16, 768, 256, 128, 8, 4, 8, 0, "bf16", "nvfp4", "rms", 0.01, 57)
    cpu = synth.make_layer(shape)
    b = torch.zeros(shape.E, dtype=torch.float32)
    b[:8] = 8.0 + torch.arange(8, dtype=torch.float32) * 0.5
    cpu["router_bias"] = b
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_nvfp4_deterministic_and_graph(moe):
    """Two eager calls agree bit for bit (workspace refilled in between), and a captured
    HIP graph replays to the same bits, also after new activations are copied in."""
    print("case: nvfp4 determinism + graph", flush=True)
    shape, cpu, dev = _decode_layer()
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    wst = moe.weights_struct(dev)
    x = dev["x"].clone()
    y1 = moe.forward(cfg, x, dev, ws, wst=wst).clone()
    ws.fill_(0x5A)
    y2 = moe.forward(cfg, x, dev, ws, wst=wst)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)

    y = torch.empty_like(y1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(cfg, x, dev, ws, y=y, wst=wst)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(cfg, x, dev, ws, y=y, wst=wst)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y1), rep
        moe.forward(cfg, x, dev, ws, wst=wst)
    x2 = torch.roll(dev["x"], shifts=1, dims=0).contiguous()
    ref2 = moe.forward(cfg, x2, dev, ws, wst=wst).clone()
    x.copy_(x2)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, ref2)
    assert not torch.equal(ref2, y1)


@pytest.mark.parametrize("T", [17, 40, 64, 300, 1200])
def test_forward_nvfp4_batch(moe, T):
    """Beyond 16 tokens: selection + permutation (one block up to 64 tokens, the scan
    beyond), the expert-major 4-bit kernels and the combine."""
    print("case: nvfp4 batch", T, flush=True)
    shape, cpu, dev = _decode_layer(T, 600 + T)
    _forward_check(moe, shape, cpu, dev)


# up to T*k <= 8E rows (and for shapes the matrix-core tiles do not divide) the
# expert-major VALU kernels run; beyond, the matrix-core kernels (fp4 -> bf16 in LDS)
BATCH_CASES = [
    ("nvb_ling_sh", 100, 1536, 512, 128, 8, 4, 8, 2, "bf16", "nvfp4", "rms", 0.0, 71),
    ("nvb_ling_sh_mfma", 400, 1536, 512, 128, 8, 4, 8, 2, "bf16", "nvfp4", "rms", 0.2, 76),
    ("nvb_inkling_mfma", 300, 1024, 256, 256, 1, 1, 6, 2, "bf16", "nvfp4", "normal", 0.0, 77),
    ("nvb_ragged", 200, 640, 384, 64, 4, 2, 4, 0, "bf16", "nvfp4", "rms", 0.3, 72),
    ("nvb_i1024", 150, 512, 1024, 32, 1, 1, 4, 1, "bf16", "nvfp4", "normal", 0.0, 73),
    ("nvb_h2048_t16", 16, 2048, 256, 16, 4, 2, 4, 0, "bf16", "nvfp4", "rms", 0.0, 74),
]


@pytest.mark.parametrize("case", BATCH_CASES, ids=[c[0] for c in BATCH_CASES])
def test_forward_nvfp4_batch_edge(moe, case):
    print("case: nvfp4 batch edge", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


@pytest.mark.parametrize("T", [40, 130])
def test_expert_ffn_nvfp4(moe, T):
    """moe_expert_ffn on the oracle's own permutation: unweighted fp32 rows (T = 40 on
    the VALU kernels, T = 130 on the matrix-core ones, whose h is bf16 as in the bf16
    path)."""
    print("case: nvfp4 expert_ffn", T, flush=True)
    shape = S_("nvb_ffn", T, 1536, 512, 128, 8, 4, 8, 1, "bf16", "nvfp4", "rms", 0.0, 75)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    ex = oracle_experts(cpu)
    x64 = np_exact(cpu["x"])
    ids, _, _ = mo.route(x64, np_exact(cpu["w_router"]), None, shape.G, shape.Gk, shape.k)
    off, rt, _ = mo.permute(ids, shape.E, shape.S)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    yp = moe.expert_ffn(cfg, dev["x"], torch.from_numpy(off.astype(np.int32)).cuda(),
                        torch.from_numpy(rt.astype(np.int32)).cuda(), dev, ws)
    torch.cuda.synchronize()
    ref = mo.expert_ffn(x64, off, rt, ex)
    err = mo.rel_l2(yp.cpu().numpy(), ref)
    print(f"nvfp4 expert_ffn T={T} rel_l2 {err:.3e}")
    assert err <= (1e-4 if T <= 128 else 5e-3)   # fp32 h (VALU) or bf16 h (matrix cores)


def test_forward_nvfp4_full_size(moe):
    """The 8192-token prefill layer with NVFP4 experts in the benchmark's launch
    configuration: every token against the expert-major oracle, and a sample through the
    token-major formulation."""
    print("case: nvfp4 full prefill", flush=True)
    shape = synth.WORKLOADS["prefill_nvfp4"]
    cpu = synth.make_layer(shape)
    full_size_check(moe, shape, cpu, to_device(cpu))
