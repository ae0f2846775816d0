"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Routing: expert ids bit-exact wherever the float64 top-k margin exceeds 1e-4
logits (near-tie tokens are counted and only checked for validity), weights
within 2e-6.  Permutation: bit-exact.  Layer outputs: relative L2 within 5e-3
(bf16, fp32) or 2e-2 (block FP8); fp32 layers also within 1e-5.  Near-tie
tokens are compared against the oracle forced onto the GPU's routing.
"""
import functools

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
import synth
from tests.helpers import (TOKEN_FACTOR, TOL, TOL_F32_INTERNAL, check_routing, config_for,
                           np_exact, oracle_experts, to_device)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _shape(name, T=None, seed=None):
    s = W[name]
    return s if T is None else s.with_tokens(T, seed)


@functools.lru_cache(maxsize=4)
def _layer(name, T=None, seed=None):
    shape = _shape(name, T, seed)
    cpu = synth.make_layer(shape)
    return shape, cpu, to_device(cpu)


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


def _print_case(*a):
    print("case:", *a, flush=True)


# ----------------------------------------------------------------------------- routing
@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", 300),
                                    ("fp8", 130), ("inkling", 257), ("decode", 1), ("tiny", 300),
                                    ("prefill", 8192)])
def test_route(moe, name, T):
    _print_case("route", name, T)
    shape, cpu, dev = _layer(name, T)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    logits = torch.empty((shape.T, shape.E), dtype=torch.float32, device="cuda")
    ids, w = moe.route(cfg, dev["x"], dev["w_router"], dev["router_bias"], ws, logits)
    torch.cuda.synchronize()
    l64 = mo.router_logits(np_exact(cpu["x"]), np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]))
    np.testing.assert_allclose(logits.cpu().numpy(), l64, rtol=0, atol=2e-5)
    near, _ = check_routing(ids.cpu().numpy(), w.cpu().numpy(), l64, shape)
    print(f"near-ties {int(near.sum())}/{shape.T}")


# Router-logit tile choices: the 32 x 32 tiles (H/128 = 8, 12 or 16 MFMA steps per wave;
# E a multiple of 32 but not of 64; ragged token tiles) and the 64 x 64 tiles once their
# grid reaches one workgroup per CU.  Logits against float64, then the routing rule.
@pytest.mark.parametrize("case", [
    ("lt_h1024_e32", 40, 1024, 32, 4, 2, 4),
    ("lt_h1536_e96", 300, 1536, 96, 6, 3, 8),
    ("lt_h2048_e64", 17, 2048, 64, 1, 1, 6),
    ("lt_h1536_t4095", 4095, 1536, 128, 8, 4, 8),
    ("lt_h1536_e256_t4096", 4096, 1536, 256, 1, 1, 6),
], ids=lambda c: c[0])
def test_route_logit_tiles(moe, case):
    name, T, H, E, G, Gk, k = case
    _print_case("route tiles", name)
    shape = synth.LayerShape(name, T=T, H=H, I=128, E=E, G=G, Gk=Gk, k=k, S=0, act="bf16",
                             wt="bf16", x_dist="rms", bias_std=0.3, seed=31)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids, w = moe.route(cfg, dev["x"], dev["w_router"], dev["router_bias"], ws, logits)
    torch.cuda.synchronize()
    l64 = mo.router_logits(np_exact(cpu["x"]), np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]))
    np.testing.assert_allclose(logits.cpu().numpy(), l64, rtol=0, atol=2e-5)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), l64, shape)


def test_route_e64_generic_path(moe):
    """E = 64 bf16 experts in 4 groups (vector-FMA logits + thread-per-token selection)."""
    _print_case("route e64")
    shape = synth.LayerShape("e64", T=200, H=512, I=128, E=64, G=4, Gk=2, k=6, S=0, act="bf16",
                             wt="bf16", x_dist="normal", bias_std=0.3, seed=12)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    ids, w = moe.route(cfg, dev["x"], dev["w_router"], dev["router_bias"], ws)
    torch.cuda.synchronize()
    l64 = mo.router_logits(np_exact(cpu["x"]), np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]))
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), l64, shape)
    _forward_check(moe, shape, cpu, dev)


def test_route_forced_ties(moe):
    """Duplicated router rows give bit-identical fp32 logits: the lower index must win."""
    _print_case("route ties")
    shape = synth.LayerShape("ties", T=64, H=256, I=128, E=16, G=4, Gk=2, k=4, S=0, act="f32",
                             wt="f32", x_dist="normal", bias_std=0.0, seed=11)
    cpu = synth.make_layer(shape)
    wr = cpu["w_router"].clone()
    wr[5] = wr[3]       # same group (1): expert 3 beats 5
    wr[9] = wr[1]       # group 2 vs group 0: equal group maxima when they lead
    wr[14] = wr[2]
    cpu["w_router"] = wr
    dev = to_device(cpu)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    logits = torch.empty((shape.T, shape.E), dtype=torch.float32, device="cuda")
    ids, w = moe.route(cfg, dev["x"], dev["w_router"], None, ws, logits)
    torch.cuda.synchronize()
    lg = logits.cpu().numpy().astype(np.float64)
    assert np.all(lg[:, 3] == lg[:, 5]) and np.all(lg[:, 1] == lg[:, 9])
    # the oracle run on the GPU's own fp32 logits must pick exactly the same ids
    o_ids, _ = mo.select_experts(mo.gate_scores(lg), shape.G, shape.Gk, shape.k)
    assert np.array_equal(ids.cpu().numpy(), o_ids)


# ----------------------------------------------------------------------------- permutation
# the last five reach the scan's register paths with 5, 16, 17 and 24 histogram blocks per
# thread, and its LDS-staged path (E = 1000: one thread per expert, 40 blocks each)
@pytest.mark.parametrize("T,E,k,S", [(1, 16, 4, 0), (4, 128, 8, 0), (257, 128, 8, 0),
                                     (1000, 128, 8, 0), (333, 256, 6, 2), (64, 16, 4, 1),
                                     (20000, 16, 4, 0), (8192, 128, 8, 0), (4100, 256, 6, 2),
                                     (3000, 512, 8, 0), (2500, 1000, 8, 0)])
def test_permute_bit_exact(moe, T, E, k, S):
    _print_case("permute", T, E, k, S)
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if T > 8:
        ids[: T // 3] = np.sort(ids[: T // 3], axis=1)   # hot experts: many rows, multi-block
        ids[: T // 3, 0] = 0
    cfg = moe.make_config(T, 256, 128, E, 1, 1, k, S, "bf16", "bf16")
    ws = moe.alloc_workspace(cfg)
    off, rt, inv = moe.permute(cfg, torch.from_numpy(ids).cuda(), ws)
    torch.cuda.synchronize()
    o_off, o_rt, o_inv = mo.permute(ids, E, S)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(rt.cpu().numpy(), o_rt)
    assert np.array_equal(inv.cpu().numpy(), o_inv)


# ----------------------------------------------------------------------------- experts
@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", 300),
                                    ("fp8", 130), ("inkling", 100), ("inkling", 420)])
def test_expert_ffn(moe, name, T):
    """Unweighted expert outputs on the oracle's own permutation."""
    _print_case("expert_ffn", name, T)
    shape, cpu, dev = _layer(name, T)
    ex = oracle_experts(cpu)
    x64 = np_exact(cpu["x"])
    ids, _, _ = mo.route(x64, np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]), shape.G, shape.Gk,
                         shape.k)
    off, rt, _ = mo.permute(ids, shape.E, shape.S)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    yp = moe.expert_ffn(cfg, dev["x"], torch.from_numpy(off.astype(np.int32)).cuda(),
                        torch.from_numpy(rt.astype(np.int32)).cuda(), dev, ws)
    torch.cuda.synchronize()
    ref = mo.expert_ffn(x64, off, rt, ex)
    err = mo.rel_l2(yp.cpu().numpy(), ref)
    print(f"rel_l2 {err:.3e}")
    assert err <= TOL[shape.wt]
    if shape.wt == "f32":
        assert err <= TOL_F32_INTERNAL


def test_combine_identity_round_trip(moe):
    """Permute then combine with identity experts returns x (weights sum to 1)."""
    _print_case("combine identity")
    shape, cpu, dev = _layer("tiny")
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    ids, w = moe.route(cfg, dev["x"], dev["w_router"], None, ws)
    off, rt, inv = moe.permute(cfg, ids, ws)
    y_perm = dev["x"][rt.long()].contiguous()
    y = moe.combine(cfg, y_perm, off, inv, w, torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_allclose(y.cpu().numpy(), cpu["x"].numpy(), rtol=0, atol=2e-6)


# ----------------------------------------------------------------------------- whole layer
def _forward_check(moe, shape, cpu, dev, sample=None):
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    y = moe.forward(cfg, dev["x"], dev, ws, ids=ids, wts=wts)
    torch.cuda.synchronize()
    x64 = np_exact(cpu["x"])
    l64 = mo.router_logits(x64, np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]))
    g_ids = ids.cpu().numpy()
    near, o_ids = check_routing(g_ids, wts.cpu().numpy(), l64, shape)
    rows = np.arange(shape.T) if sample is None else sample
    # oracle on the sampled tokens, forced onto the GPU's routing for near-tie tokens
    use_ids = np.where(near[:, None], g_ids, o_ids)[rows]
    w64 = mo.renormalise(mo.gate_scores(l64[rows]), use_ids)
    ex = oracle_experts(cpu)
    if sample is None:
        off, rt, inv = mo.permute(use_ids, shape.E, shape.S)
        ref = mo.combine(mo.expert_ffn(x64, off, rt, ex), off, inv, w64, shape.S)
    else:
        ref = mo.forward_tokenmajor(x64[rows], ex, use_ids, w64)
    got = y.float().cpu().numpy()[rows]
    err = mo.rel_l2(got, ref)
    worst = float(mo.row_rel_l2(got, ref).max())
    print(f"{shape.name} T={shape.T} rel_l2 {err:.3e} worst token {worst:.3e} "
          f"near-ties {int(near.sum())}")
    assert err <= TOL[shape.wt]
    assert worst <= TOKEN_FACTOR * TOL[shape.wt], "one token's output is far off"
    if shape.wt == "f32":
        assert err <= TOL_F32_INTERNAL
    return y, g_ids, near


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("decode", 1),
                                    ("decode", 16), ("decode", 40), ("prefill", 300),
                                    ("prefill", 1500), ("fp8", 130), ("fp8", 16),
                                    ("inkling", 100), ("inkling", 420), ("tiny", 300),
                                    ("tiny", 65), ("inkling", 8), ("decode", 7)])
def test_forward(moe, name, T):
    _print_case("forward", name, T)
    shape, cpu, dev = _layer(name, T)
    _forward_check(moe, shape, cpu, dev)


def full_size_check(moe, shape, cpu, dev):
    """A full-size workload in the benchmark's launch configuration: every token against
    the expert-major oracle (on the GPU's routing for near-tie tokens), then a sample of
    tokens through the token-major formulation, an independent second path."""
    y, g_ids, near = _forward_check(moe, shape, cpu, dev)
    rng = np.random.default_rng(99)
    sample = np.unique(np.concatenate([[0, shape.T - 1], rng.choice(shape.T, 30, replace=False)]))
    x64 = np_exact(cpu["x"])
    l64 = mo.router_logits(x64, np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]))
    w64 = mo.renormalise(mo.gate_scores(l64[sample]), g_ids[sample])
    ref = mo.forward_tokenmajor(x64[sample], oracle_experts(cpu), g_ids[sample], w64)
    err = mo.rel_l2(y.float().cpu().numpy()[sample], ref)
    print(f"token-major sample of {len(sample)}: rel_l2 {err:.3e}")
    assert err <= TOL[shape.wt]


@pytest.mark.parametrize("name", ["prefill", "fp8", "inkling"])
def test_forward_full_size(moe, name):
    _print_case("forward full", name)
    shape, cpu, dev = _layer(name)
    full_size_check(moe, shape, cpu, dev)


@pytest.mark.parametrize("T", [2048, 130])
def test_fp8_activation_codes_bit_exact(moe, T):
    """The block-FP8 layer's e4m3 codes and fp32 scales of x, read back from the
    workspace after moe_forward, equal the oracle's quantiser (reading R9) byte for byte."""
    _print_case("fp8 codes", T)
    shape, cpu, dev = _layer("fp8", None if T == 2048 else T)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    moe.forward(cfg, dev["x"], dev, ws)
    torch.cuda.synchronize()
    oc, nc = moe.workspace_slot(cfg, moe.WS_ACT_CODES)
    os_, ns = moe.workspace_slot(cfg, moe.WS_ACT_SCALES)
    codes = ws[oc:oc + nc].cpu().numpy().reshape(shape.T, shape.H)
    scales = ws[os_:os_ + ns].cpu().view(torch.float32).numpy().reshape(shape.T, shape.H // 128)
    ref_codes, ref_scales = mo.quantize_act_codes(np_exact(cpu["x"]))
    assert np.array_equal(scales.view(np.uint32), ref_scales.view(np.uint32))
    bad = np.count_nonzero(codes != ref_codes)
    assert bad == 0, f"{bad} of {codes.size} codes differ"


@pytest.mark.parametrize("name,T", [("decode", None), ("prefill", 600), ("fp8", 200)])
def test_forward_deterministic(moe, name, T):
    _print_case("determinism", name, T)
    shape, cpu, dev = _layer(name, T)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    y1 = moe.forward(cfg, dev["x"], dev, ws).clone()
    ws.fill_(0x5A)
    y2 = moe.forward(cfg, dev["x"], dev, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
