"""moe_forward_noalloc (the library's fixed per-GPU scratch, no workspace argument, no
allocation in the call) against moe_forward with a caller-owned workspace: outputs,
expert ids and weights equal bit for bit, on two calls in a row whose second input is
smaller (it runs on whatever the first left in the shared scratch), for every expert
type and routing path the scratch is large enough for; a config beyond the scratch
is refused before any work."""
import pytest
import torch

import synth
from tests.helpers import config_for, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


SEQUENCES = [
    [("decode", 16), ("decode", 4)],                 # decode kernels
    [("decode", 200), ("decode", 40)],               # batch routing, skinny experts
    [("prefill", 256), ("prefill", 100)],            # matrix-core experts (with the router bias)
    [("inkling", 150), ("inkling", 7)],              # shared experts, ungrouped routing
    [("fp8", 130), ("fp8", 16)],                     # block-FP8 experts
    [("tiny", 300), ("tiny", 16)],                   # fp32 layer
    [("decode_nvfp4", 9), ("decode_nvfp4", 4)],      # NVFP4 decode kernels
    [("decode_mxfp4", 12), ("decode_mxfp4", 3)],     # MXFP4 decode kernels
    [("prefill_mxfp4", 300), ("prefill_mxfp4", 40)], # block-scaled matrix-core experts
]


def _one(moe, name, T):
    shape = synth.WORKLOADS[name].with_tokens(T)
    cpu = synth.make_layer(shape)
    dev = to_device(cpu)
    cfg = config_for(shape)
    assert moe.workspace_size(cfg) <= moe.NOALLOC_SCRATCH_BYTES
    wst = moe.weights_struct(dev)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    y = moe.forward(cfg, dev["x"], None, ws, ids=ids, wts=wts, wst=wst)
    ids2 = torch.full_like(ids, -1)
    wts2 = torch.full_like(wts, -1.0)
    y2 = moe.forward_noalloc(cfg, dev["x"], None, ids=ids2, wts=wts2, wst=wst)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), (name, T)
    assert torch.equal(ids2, ids) and torch.equal(wts2, wts), (name, T)


@pytest.mark.parametrize("seq", SEQUENCES, ids=[f"{s[0][0]}-{s[0][1]}-{s[1][1]}" for s in SEQUENCES])
def test_noalloc_equals_forward_two_calls(moe, seq):
    for name, T in seq:
        print("case: noalloc", name, T, flush=True)
        _one(moe, name, T)


def test_noalloc_refuses_configs_beyond_its_scratch(moe):
    print("case: noalloc too large", flush=True)
    shape = synth.WORKLOADS["prefill"]
    cfg = config_for(shape)
    assert moe.workspace_size(cfg) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((shape.T, shape.H), dtype=torch.bfloat16, device="cuda")
    fake = {k: x for k in ("w_router", "w_gate", "w_up", "w_down")}
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(cfg, x, fake)
    assert e.value.status == -5
