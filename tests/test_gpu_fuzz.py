"""Seeded randomized shapes through the whole layer and the decoder step: 24 valid
configurations drawn once from a fixed seed across every expert type (fp32, bf16, block
FP8, NVFP4), grouped and ungrouped routers, shared experts and token counts from 1 to
300, plus 16 few-token draws and 12 MXFP4 draws, each checked against the oracle at the
layer's bar.  The draw only picks sizes
within the documented limits; nothing here is meant to fail."""
import numpy as np
import pytest
import torch

import synth
from tests.helpers import to_device
from tests.test_gpu_parity import _forward_check

pytestmark = pytest.mark.gpu


def _draw_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    wts = ["f32", "bf16", "e4m3", "nvfp4"]
    for i in range(n):
        wt = wts[i % 4]
        act = "f32" if wt == "f32" else "bf16"
        hm = {"f32": 8, "bf16": 8, "e4m3": 128, "nvfp4": 32}[wt]
        H = int(rng.choice([hm * m for m in range(1, 1 + 1024 // hm)]))
        I = int(rng.choice([hm * m for m in range(1, 1 + 512 // hm)]))
        G = int(rng.choice([1, 2, 4, 8]))
        n_per = int(rng.choice([2, 4, 8, 16]))
        E = G * n_per
        Gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, Gk * n_per) + 1))
        S = int(rng.choice([0, 0, 1, 2]))
        T = int(rng.choice([1, 3, 7, 16, 40, 130, 300]))
        cases.append((f"fz{i}_{wt}", T, H, I, E, G, Gk, k, S, act, wt,
                      "rms" if i % 2 else "normal", float(rng.choice([0.0, 0.3])), 3000 + i))
    return cases


def _draw_decode_cases(n=16, seed=2025):
    """Few-token draws on expert counts the sixteen-lane selection covers (E = 16 V),
    where up to four tokens build their row tables in one wave: 1-5 tokens, grouped or
    not, shared experts, every expert type."""
    rng = np.random.default_rng(seed)
    cases = []
    wts = ["f32", "bf16", "e4m3", "nvfp4"]
    for i in range(n):
        wt = wts[i % 4]
        act = "f32" if wt == "f32" else "bf16"
        hm = {"f32": 8, "bf16": 8, "e4m3": 128, "nvfp4": 32}[wt]
        H = int(rng.choice([hm * m for m in range(1, 1 + 1536 // hm)]))
        I = int(rng.choice([hm * m for m in range(1, 1 + 512 // hm)]))
        E = int(rng.choice([16, 64, 128, 256]))
        G = int(rng.choice([g for g in (1, 2, 4, 8) if E // g >= 2]))
        n_per = E // G
        Gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, Gk * n_per) + 1))
        S = int(rng.choice([0, 1, 2]))
        T = int(rng.choice([1, 2, 3, 4, 5]))
        cases.append((f"fzd{i}_{wt}", T, H, I, E, G, Gk, k, S, act, wt,
                      "rms" if i % 2 else "normal", float(rng.choice([0.0, 0.3])), 4000 + i))
    return cases


def _draw_mx_cases(n=12, seed=2026):
    """MXFP4 experts (H a multiple of 256, I of 128): token counts on both sides of the
    16-token switch between the decode kernels and the block-scaled matrix-core path."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        H = int(rng.choice([256 * m for m in range(1, 9)]))
        I = int(rng.choice([128 * m for m in range(1, 9)]))
        E = int(rng.choice([16, 32, 64, 128, 256]))
        G = int(rng.choice([g for g in (1, 2, 4, 8) if E // g >= 2]))
        n_per = E // G
        Gk = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(16, Gk * n_per) + 1))
        S = int(rng.choice([0, 0, 1, 2]))
        T = int(rng.choice([1, 3, 5, 16, 17, 40, 130, 300]))
        cases.append((f"fzm{i}_mxfp4", T, H, I, E, G, Gk, k, S, "bf16", "mxfp4",
                      "rms" if i % 2 else "normal", float(rng.choice([0.0, 0.3])), 5000 + i))
    return cases


CASES = _draw_cases() + _draw_decode_cases() + _draw_mx_cases()


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fuzz_forward(moe, case):
    print("case: fuzz", case, flush=True)
    shape = synth.LayerShape(*case)
    cpu = synth.make_layer(shape)
    _forward_check(moe, shape, cpu, to_device(cpu))
