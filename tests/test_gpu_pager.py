"""Expert paging on the GPU (moe_forward_paged): routed experts in pinned host memory,
an HBM arena of N slots, residency decided on the device.

Each case runs a sequence of calls on fresh tokens (a skewed router, so some experts
recur and others are evicted) and checks after every call:
  * the device's residency tables and counters equal the slot-arena model of
    oracle/pager.py (reading R18) stepped with the GPU's own routing, bit for bit;
  * y equals, bit for bit, moe_route + moe_permute + moe_expert_ffn + moe_combine on
    the same layer held entirely in HBM (the arena changes where weights are read
    from, never what is computed);
  * y is within the layer's bar of the float64 oracle on the GPU's routing."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from oracle.pager import SlotArena
from tests.helpers import TOL, config_for, np_exact, oracle_experts, to_device

pytestmark = pytest.mark.gpu

S_ = synth.LayerShape

CASES = [
    # (shape, slots, calls)
    (S_("pg_decode", 4, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 1.0, 51), 40, 12),
    (S_("pg_one", 1, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 1.0, 52), 8, 12),
    (S_("pg_shared", 3, 1024, 256, 64, 1, 1, 6, 2, "bf16", "bf16", "normal", 1.0, 53), 24, 10),
    (S_("pg_f32", 2, 256, 128, 16, 4, 2, 4, 0, "f32", "f32", "normal", 0.5, 54), 8, 10),
    (S_("pg_batch", 40, 512, 256, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 1.0, 55), 128, 4),
]


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


def _tokens(shape, rng):
    z = rng.standard_normal((shape.T, shape.H), dtype=np.float32)
    if shape.x_dist == "rms":
        z64 = z.astype(np.float64)
        z = (z64 / np.sqrt(np.mean(z64 * z64, axis=1, keepdims=True))).astype(np.float32)
    t = torch.from_numpy(z)
    return t if shape.act == "f32" else t.to(torch.bfloat16)


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_paged_layer_sequence(moe, case):
    shape, N, calls = case
    print("case: paged", shape.name, "slots", N, flush=True)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    cfg = config_for(shape)
    store = {k: cpu[k].contiguous().pin_memory() for k in ("w_gate", "w_up", "w_down")}
    host = moe.weights_struct_host(store)
    dt = cpu["w_gate"].dtype
    arena = {"w_gate": torch.zeros((N, shape.I, shape.H), dtype=dt, device="cuda"),
             "w_up": torch.zeros((N, shape.I, shape.H), dtype=dt, device="cuda"),
             "w_down": torch.zeros((N, shape.H, shape.I), dtype=dt, device="cuda")}
    resident = dict(dev)
    resident.update(arena)
    res_w = moe.weights_struct(resident)
    state = moe.alloc_pager_state(cfg, N)
    ws = moe.paged_workspace(cfg, N)
    ws_ref = moe.alloc_workspace(cfg)
    model = SlotArena(shape.E, N)
    rng = np.random.default_rng(shape.seed + 1000)
    ex = oracle_experts(cpu)
    for call in range(calls):
        x = _tokens(shape, rng).cuda()
        ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
        y = moe.forward_paged(cfg, x, host, res_w, N, state, ws, ids=ids, wts=wts)
        # the same layer resident in HBM through the component calls
        r_ids, r_w = moe.route(cfg, x, dev["w_router"], dev["router_bias"], ws_ref)
        off, rt, inv = moe.permute(cfg, r_ids, ws_ref)
        yp = moe.expert_ffn(cfg, x, off, rt, dev, ws_ref)
        y_ref = moe.combine(cfg, yp, off, inv, r_w, x.dtype)
        torch.cuda.synchronize()
        g_ids = ids.cpu().numpy()
        assert np.array_equal(g_ids, r_ids.cpu().numpy()) and torch.equal(wts, r_w)
        assert torch.equal(y, y_ref), f"call {call}: paged output differs from the resident path"
        model.step(g_ids)
        tab = moe.pager_tables(cfg, N, state)
        assert np.array_equal(tab["key_slot"], model.key_slot), call
        assert np.array_equal(tab["slot_key"], model.slot_key), call
        assert np.array_equal(tab["stamp"], model.stamp), call
        assert (tab["calls"], tab["refs"], tab["lookups"], tab["hits"], tab["misses"]) == \
            (model.calls, model.refs, model.lookups, model.hits, model.misses), call
        assert tab["bytes_copied"] == model.misses * 3 * shape.I * shape.H * dt.itemsize
        # the arena holds the resident experts' weights
        for s in np.nonzero(model.slot_key >= 0)[0][:4]:
            e = int(model.slot_key[s])
            assert torch.equal(arena["w_down"][s].cpu(), cpu["w_down"][e])
        if call in (0, calls - 1):
            x64 = np_exact(x.cpu())
            ref = mo.forward(x64, np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]), ex,
                             shape.G, shape.Gk, shape.k, ids=g_ids)["y"]
            err = mo.rel_l2(y.float().cpu().numpy(), ref)
            assert err <= TOL[shape.wt], err
    print(f"hot rate {model.hot_rate():.3f} over {model.lookups} lookups, {model.misses} copies")
    assert model.hits > 0 and model.misses > 0 or N == shape.E


def test_paged_rejects_an_arena_too_small_for_one_call(moe):
    print("case: paged validation", flush=True)
    shape = synth.WORKLOADS["decode"]
    cfg = config_for(shape)
    with pytest.raises(moe.MoeError) as e:
        moe.paged_workspace(cfg, 31)                  # one call can need 32 experts
    assert e.value.status == -2
    with pytest.raises(moe.MoeError) as e:
        moe.paged_workspace(cfg, 129)                 # more slots than experts
    assert e.value.status == -2
