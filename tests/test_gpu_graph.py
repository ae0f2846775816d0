"""moe_forward captured in a HIP graph (the library enqueues kernels only: no host
sync, no allocation, no memset), replayed several times with eager work and
synchronisations in between.  Every replay must equal the eager call bit for bit
(the kernels are deterministic), also after new inputs are copied into the
captured buffers."""
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


@pytest.mark.parametrize("name,T", [("decode", None), ("tiny", None), ("prefill", 700),
                                    ("fp8", 260), ("inkling", 300)])
def test_graph_replay(moe, name, T):
    print("case: graph", name, T, flush=True)
    base = synth.WORKLOADS[name]
    shape = base if T is None else base.with_tokens(T, 77)
    dev = to_device(synth.make_layer(shape))
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    wst = moe.weights_struct(dev)
    x = dev["x"].clone()
    y = torch.empty((shape.T, shape.H), dtype=x.dtype, device="cuda")
    ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")

    def eager(xin):
        ye = torch.empty_like(y)
        moe.forward(cfg, xin, dev, ws, y=ye, wst=wst)
        torch.cuda.synchronize()
        return ye

    ref1 = eager(x)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.forward(cfg, x, dev, ws, y=y, ids=ids, wts=wts, wst=wst)   # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        moe.forward(cfg, x, dev, ws, y=y, ids=ids, wts=wts, wst=wst)
    torch.cuda.synchronize()

    for rep in range(3):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref1), f"replay {rep} differs from the eager call"
        _ = eager(x)                      # eager work on the same workspace between replays

    # new activations in the captured input buffer
    x2 = torch.roll(dev["x"], shifts=1, dims=0).contiguous()   # other tokens in each row
    ref2 = eager(x2)
    x.copy_(x2)
    torch.cuda.synchronize()
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref2), f"replay {rep} on new inputs differs from the eager call"
