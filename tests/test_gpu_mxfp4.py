"""GPU parity of the layer with MXFP4 experts (E2M1 codes with an E8M0 scale per 32
inputs; activations quantised per 32 to MXFP8 by the layer) against the float64 oracle
on the same stored codes (readings R19, R20): up to 16 tokens on the decode kernels
(E2M1 x E4M3 products on the vector units), larger batches on the block-scaled matrix
cores.

Same bar as the block-FP8 layer (the activations are quantised to E4M3 likewise):
exact ids where the logit margin is clear, rel L2 of y within 2e-2; every token of the
8192-token prefill layer; the activation codes and scales of x bit for bit; the
expert-FFN entry point on its own; determinism."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from tests.helpers import config_for, np_exact, oracle_experts, to_device, TOL
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


def _layer(name, T=None, seed=None):
    base = synth.WORKLOADS[name]
    shape = base if T is None else base.with_tokens(T, seed)
    if shape not in _CACHE:
        cpu = synth.make_layer(shape)
        _CACHE.clear()
        _CACHE[shape] = (cpu, to_device(cpu))
    return (shape,) + _CACHE[shape]


@pytest.mark.parametrize("name,T", [("decode_mxfp4", None), ("decode_mxfp4", 1),
                                    ("decode_mxfp4", 16), ("decode_mxfp4", 40),
                                    ("prefill_mxfp4", 300), ("prefill_mxfp4", 1500)])
def test_forward_mxfp4(moe, name, T):
    print("case: mxfp4 forward", name, T, flush=True)
    shape, cpu, dev = _layer(name, T)
    _forward_check(moe, shape, cpu, dev)


DECODE_CASES = [
    # name, T, H, I, E, G, Gk, k, S, act, wt, x_dist, bias_std, seed
    ("mxd_ling_sh", 5, 1536, 512, 128, 8, 4, 8, 2, "bf16", "mxfp4", "rms", 0.0, 91),
    ("mxd_inkling", 8, 1024, 256, 256, 1, 1, 6, 2, "bf16", "mxfp4", "normal", 0.0, 92),
    ("mxd_ragged", 3, 768, 384, 64, 4, 2, 4, 0, "bf16", "mxfp4", "rms", 0.3, 93),    # idle lanes
    ("mxd_i1024", 6, 512, 1024, 32, 1, 1, 4, 1, "bf16", "mxfp4", "normal", 0.0, 94),  # wave selection
    ("mxd_g64", 3, 512, 256, 256, 64, 8, 16, 0, "bf16", "mxfp4", "rms", 0.0, 95),
    ("mxd_h2048", 12, 2048, 256, 16, 4, 2, 4, 0, "bf16", "mxfp4", "rms", 0.0, 96),
    ("mxd_t16", 16, 1536, 512, 128, 8, 4, 8, 0, "bf16", "mxfp4", "rms", 0.5, 97),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_forward_mxfp4_decode_shapes(moe, case):
    """The decode kernels (in-block routing, x quantised in LDS, h quantised per 32 in
    the down kernel's lanes) over the shapes their item layouts branch on."""
    print("case: mxfp4 decode shape", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_forward_mxfp4_decode_skewed_router(moe):
    """Every token prefers the same eight experts (all in group 0)."""
    print("case: mxfp4 decode skew", flush=True)
    shape = S_("mxd_skew", 16, 768, 256, 128, 8, 4, 8, 0, "bf16", "mxfp4", "rms", 0.01, 98)
    cpu = synth.make_layer(shape)
    b = torch.zeros(shape.E, dtype=torch.float32)
    b[:8] = 8.0 + torch.arange(8, dtype=torch.float32) * 0.5
    cpu["router_bias"] = b
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_mxfp4_decode_deterministic_and_graph(moe):
    """Two eager decode calls agree bit for bit (workspace refilled in between), and a
    captured HIP graph replays to the same bits, also after new activations are copied in."""
    print("case: mxfp4 decode determinism + graph", flush=True)
    shape, cpu, dev = _layer("decode_mxfp4")
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


CASES = [
    # Inkling-shaped: 256 experts ungrouped, top-6, 2 shared experts, hidden 2048
    ("mx_inkling", 100, 2048, 512, 256, 1, 1, 6, 2, "bf16", "mxfp4", "normal", 0.0, 81),
    ("mx_i1024", 70, 512, 1024, 64, 4, 2, 8, 0, "bf16", "mxfp4", "rms", 0.3, 82),      # I = 1024
    ("mx_h256", 130, 256, 128, 32, 4, 2, 4, 1, "bf16", "mxfp4", "normal", 0.0, 83),    # smallest sizes
    ("mx_k2048", 50, 2048, 2048, 16, 2, 1, 2, 0, "bf16", "mxfp4", "rms", 0.0, 84),      # K = 2048 both GEMMs
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_mxfp4_shapes(moe, case):
    print("case: mxfp4 shape", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_forward_mxfp4_full_size(moe):
    print("case: mxfp4 full prefill", flush=True)
    shape, cpu, dev = _layer("prefill_mxfp4")
    full_size_check(moe, shape, cpu, dev)


@pytest.mark.parametrize("T", [4, 2000])
def test_mxfp8_activation_codes_bit_exact(moe, T):
    """x's MXFP8 codes and E8M0 scales, read back from the workspace after moe_forward,
    equal the oracle's quantiser (reading R20) byte for byte: at 4 tokens from the decode
    kernel's in-LDS quantiser, at 2000 from the matrix-core path's quantiser kernel."""
    print("case: mxfp4 act codes", T, flush=True)
    shape, cpu, dev = _layer("decode_mxfp4", T, 85 if T != 4 else None)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    moe.forward(cfg, dev["x"], dev, ws)
    torch.cuda.synchronize()
    oc, nc = moe.workspace_slot(cfg, moe.WS_ACT_CODES)
    os_, ns = moe.workspace_slot(cfg, moe.WS_ACT_SCALES)
    assert ns == shape.T * shape.H // 32
    codes = ws[oc:oc + nc].cpu().numpy().reshape(shape.T, shape.H)
    scales = ws[os_:os_ + ns].cpu().numpy().reshape(shape.T, shape.H // 32)
    ref_codes, ref_scales = mo.quantize_mxfp8_codes(np_exact(cpu["x"]))
    assert np.array_equal(scales, ref_scales)
    bad = np.count_nonzero(codes != ref_codes)
    assert bad == 0, f"{bad} of {codes.size} codes differ"


@pytest.mark.parametrize("T", [4, 300])
def test_expert_ffn_mxfp4(moe, T):
    """Unweighted expert outputs (fp32) on the oracle's own permutation."""
    print("case: mxfp4 expert_ffn", T, flush=True)
    shape, cpu, dev = _layer("decode_mxfp4", T, 86 if T != 4 else None)
    ex = oracle_experts(cpu)
    x64 = np_exact(cpu["x"])
    ids, _, _ = mo.route(x64, np_exact(cpu["w_router"]), None, shape.G, shape.Gk, shape.k)
    off, rt, _ = mo.permute(ids, shape.E, shape.S)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    yp = moe.expert_ffn(cfg, dev["x"], torch.from_numpy(off.astype(np.int32)).cuda(),
                        torch.from_numpy(rt.astype(np.int32)).cuda(), dev, ws)
    torch.cuda.synchronize()
    err = mo.rel_l2(yp.cpu().numpy(), mo.expert_ffn(x64, off, rt, ex))
    print(f"mxfp4 expert_ffn T={T} rel_l2 {err:.3e}")
    assert err <= TOL["mxfp4"]


def test_forward_mxfp4_deterministic(moe):
    print("case: mxfp4 determinism", flush=True)
    shape, cpu, dev = _layer("prefill_mxfp4", 600)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    y1 = moe.forward(cfg, dev["x"], dev, ws).clone()
    ws.fill_(0x5A)
    y2 = moe.forward(cfg, dev["x"], dev, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
