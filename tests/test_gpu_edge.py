"""GPU parity on shapes at the edges of what the kernels cover: many small groups,
the largest and smallest k, expert counts that are not powers of two, shared
experts on the Ling shape, a router so skewed that one expert receives every
token and most receive none, and hidden sizes that the pipelined expert kernels do
not cover (so the register-staged ones run).  Same bar as the main parity tests."""
import pytest
import torch

import synth
from tests.helpers import to_device
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


CASES = [
    # name, T, H, I, E, G, Gk, k, S, act, wt, x_dist, bias_std, seed
    ("g64", 3, 512, 256, 256, 64, 8, 16, 0, "bf16", "bf16", "rms", 0.0, 21),     # decode kernels
    ("g64b", 200, 512, 256, 256, 64, 8, 16, 0, "bf16", "bf16", "rms", 0.2, 22),  # batch path
    ("k1", 40, 256, 128, 32, 2, 1, 1, 0, "bf16", "bf16", "normal", 0.0, 23),
    ("e96", 5, 384, 256, 96, 6, 3, 6, 0, "bf16", "bf16", "rms", 0.0, 24),        # E/G = 16, E not 2^n
    ("e96b", 300, 384, 256, 96, 6, 3, 6, 0, "bf16", "bf16", "rms", 0.0, 25),
    ("ling_sh", 5, 1536, 512, 128, 8, 4, 8, 2, "bf16", "bf16", "rms", 0.0, 26),  # shared experts
    ("ling_shb", 260, 1536, 512, 128, 8, 4, 8, 2, "bf16", "bf16", "rms", 0.0, 27),
    ("h640", 300, 640, 384, 64, 4, 2, 4, 0, "bf16", "bf16", "rms", 0.0, 28),     # register-staged bf16
    ("h640f8", 300, 640, 384, 64, 4, 2, 4, 0, "bf16", "e4m3", "rms", 0.0, 29),   # register-staged fp8
    ("f32b", 90, 256, 128, 16, 4, 2, 4, 1, "f32", "f32", "normal", 0.0, 30),     # fp32 + shared
    # decode routing tables built by one wave: 64 slots (its slot-mask limit) with
    # shared experts, and just past its 256-expert limit (the block-wide path)
    ("w64slots", 4, 512, 256, 128, 8, 4, 16, 2, "bf16", "bf16", "rms", 0.0, 32),
    ("w258", 4, 512, 256, 256, 8, 4, 8, 2, "bf16", "bf16", "rms", 0.0, 33),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_edge(moe, case):
    print("case: edge", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))


def test_forward_skewed_router(moe):
    """Biases of +8 .. +11.5 on experts 0..7 (all in group 0) send (nearly) every token
    to those eight: each of them holds about T rows (many M tiles), most of the other
    120 experts hold none."""
    print("case: edge skew", flush=True)
    shape = S_("skew", 1000, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 0.01, 31)
    cpu = synth.make_layer(shape)
    b = torch.zeros(shape.E, dtype=torch.float32)
    b[:8] = 8.0 + torch.arange(8, dtype=torch.float32) * 0.5    # distinct: no cross-expert ties
    cpu["router_bias"] = b
    _forward_check(moe, shape, cpu, to_device(cpu))
