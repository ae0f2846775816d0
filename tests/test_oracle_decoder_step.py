"""Pins of the oracle's decoder-step pieces (reading R16): bf16 rounding, RMSNorm and the
residual MoE block, against torch's own casts and rms_norm, closed forms, and special
cases that fix which tensor feeds which step."""
import numpy as np
import torch

from oracle import moe_oracle as mo


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(50000), rng.standard_normal(5000) * 1e-3,
                        rng.standard_normal(5000) * 1e3]).astype(np.float32)
    # exact midpoints between neighbouring bf16 values: low 16 bits = 0x8000
    mid = (rng.integers(0x3000, 0x4F00, 4000).astype(np.uint32) << 16) | 0x8000
    v = np.concatenate([v, mid.view(np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(mo.round_bf16(v.astype(np.float64)), want)


def test_round_bf16_rounds_once():
    """1 + 2^-8 is a bf16 tie; 2^-30 above it must round up.  Going through fp32 first
    would land exactly on the tie and round down to even (1.0)."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert np.float32(v) == np.float32(1.0 + 2.0 ** -8)
    assert mo.round_bf16(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert mo.round_bf16(np.array([-v]))[0] == -(1.0 + 2.0 ** -7)
    assert mo.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0            # tie -> even


def test_rms_norm_against_torch_and_closed_form():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96)) * rng.uniform(0.01, 10, (7, 1))
    g = rng.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g),
                                        eps=1e-6).numpy()
    np.testing.assert_allclose(mo.rms_norm(x, g, 1e-6), want, rtol=1e-13, atol=0)
    c = 0.37
    row = np.full((1, 50), c)
    np.testing.assert_allclose(mo.rms_norm(row, g[:50], 1e-6)[0], c / np.sqrt(c * c + 1e-6) * g[:50],
                               rtol=1e-14)


def _small_layer(rng, E=8, H=32, I=16, zero_down=False):
    wg = rng.standard_normal((E, I, H)) * 0.1
    wu = rng.standard_normal((E, I, H)) * 0.1
    wd = np.zeros((E, H, I)) if zero_down else rng.standard_normal((E, H, I)) * 0.1
    return mo.Experts(wg, wu, wd), rng.standard_normal((E, H)) * 0.3


def test_residual_block_adds_the_unnormalised_input():
    """With every down projection zero the block is the identity on x (a bf16 x comes
    back bit for bit), so the residual is x itself, not the normalised rows."""
    rng = np.random.default_rng(3)
    ex, wr = _small_layer(rng, zero_down=True)
    x = mo.round_bf16(rng.standard_normal((5, 32)) * 3.0)
    g = rng.standard_normal(32)
    out = mo.residual_layer(x, g, wr, None, ex, 2, 1, 2)
    np.testing.assert_array_equal(out["x_out"], x)
    assert not np.allclose(out["x_norm"], x)


def test_residual_block_routes_and_runs_on_the_normalised_rows():
    rng = np.random.default_rng(4)
    ex, wr = _small_layer(rng)
    x = mo.round_bf16(rng.standard_normal((6, 32)) * 5.0)
    g = rng.uniform(0.5, 1.5, 32)
    out = mo.residual_layer(x, g, wr, None, ex, 2, 1, 2)
    xn = mo.round_bf16(mo.rms_norm(x, g))
    np.testing.assert_array_equal(out["x_norm"], xn)
    np.testing.assert_allclose(out["logits"], xn @ wr.T, rtol=1e-13)
    # the experts see x_n too: scaling x leaves x_n (hence y) nearly unchanged
    out2 = mo.residual_layer(x * 4.0, g, wr, None, ex, 2, 1, 2)
    np.testing.assert_allclose(out2["y"], out["y"], rtol=0, atol=2e-2 * np.abs(out["y"]).max())
    np.testing.assert_allclose(out["x_out"], mo.round_bf16(x + out["y"]), rtol=0, atol=0)
