"""Pins of the oracle's MX formats (readings R19, R20): E8M0 scales against torch's
float8_e8m0fnu, an MXFP4 row dequantised by hand (tests/golden/mxfp4_worked.txt), the
MXFP8 activation quantiser against hand-worked blocks (including the clipping the OCP
conversion allows) and against torch's e4m3 cast with the shared exponent computed by
log2, its error bound, the generator's codes being nearest under the oracle's decode,
and a layer whose quantisation steps are exact reducing to the dense expert."""
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as mo
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_worked.txt")


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = mo.e8m0_values()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_mxfp4_worked_row():
    vals = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        key, *rest = line.split()
        vals[key] = rest
    packed = np.array([int(b, 16) for b in vals["packed"]], dtype=np.uint8)[None]
    scales = np.array([int(v) for v in vals["scales"]], dtype=np.uint8)[None]
    w = mo.dequant_mxfp4(packed, scales)[0]
    assert w.shape == (64,)
    exp0 = np.array([float(v) for v in vals["values0"]])
    exp1 = np.array([float(v) for v in vals["values1"]])
    assert np.array_equal(w[:16], exp0) and np.array_equal(np.signbit(w[:16]), np.signbit(exp0))
    assert np.array_equal(w[32:48], exp1) and np.array_equal(np.signbit(w[32:48]), np.signbit(exp1))
    assert np.all(w[16:32] == 0.0625)                  # bytes 0x11: codes 1, 1 -> 0.5 / 8


def test_mxfp8_hand_blocks():
    v = np.zeros((1, 128), np.float32)
    v[0, 0] = 3.0           # amax 3: floor(log2 3) = 1, X = -7, 3 * 128 = 384 = 1.5 * 2^8
    v[0, 1] = -0.5          # -64 = -1.0 * 2^6: sign, exponent field 6 + 7 = 13, mantissa 0
    v[0, 32] = 3.75         # amax 3.75: X = -7, 480 clips to 448
    v[0, 33] = 3.5          # 448 exactly
    v[0, 34] = 1e-3         # 0.128 = 1.024 * 2^-3: rounds to 1.0 * 2^-3
    v[0, 96:128] = 2.0 ** -10   # amax 2^-10: X = -18, every element 256 = 1.0 * 2^8
    codes, sc = mo.quantize_mxfp8_codes(v)
    assert sc.tolist() == [[120, 120, 0, 109]]          # block 2 is all zero: code 0 (X = -127)
    assert codes[0, 0] == 0x7C and codes[0, 1] == 0xE8
    assert codes[0, 32] == 0x7E and codes[0, 33] == 0x7E
    assert codes[0, 34] == 0x20                          # exponent field -3 + 7 = 4
    assert np.all(codes[0, 64:96] == 0) and np.all(codes[0, 96:128] == 0x78)
    deq = mo.quantize_mxfp8(v)
    assert deq[0, 0] == 3.0 and deq[0, 32] == 3.5 and deq[0, 96] == 2.0 ** -10


def test_mxfp8_codes_match_log2_and_torch():
    rng = np.random.default_rng(51)
    v = (rng.standard_normal((64, 256)) * rng.choice([1e-3, 1.0, 40.0], size=(64, 1))).astype(np.float32)
    v[3, :32] = 0.0
    codes, sc = mo.quantize_mxfp8_codes(v)
    blocks = v.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(blocks).max(axis=2)
    X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127).astype(np.int64)
    assert np.array_equal(sc.astype(np.int64), X + 127)
    q = np.clip(blocks / np.ldexp(1.0, X)[:, :, None], -448, 448).astype(np.float32)
    ref = torch.from_numpy(q.reshape(64, 256)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # error bound: half an e4m3 step of the element, at most 2^-4 relative for normals
    deq = mo.quantize_mxfp8(v)
    scale = np.repeat(np.ldexp(1.0, X), 32, axis=1)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 1e-9)
    clipped = np.abs(v) > 448 * scale
    assert np.all((np.abs(deq - v) <= bound) | clipped)


def test_generator_codes_are_nearest():
    w = np.random.default_rng(52).standard_normal((2, 8, 64)).astype(np.float32) * 0.02
    packed, sc = synth._encode_mxfp4(w)
    deq = np.stack([mo.dequant_mxfp4(packed[i].numpy(), sc[i].numpy()) for i in range(2)])
    step = np.repeat(mo.e8m0_values()[sc.numpy()], 32, axis=-1)
    mags = mo.e2m1_values()[:8]
    # every weight decodes to the E2M1 value nearest to w / scale (within saturation at 6)
    q = np.clip(np.abs(w) / step, 0, 6)
    nearest = mags[np.abs(q[..., None] - mags).argmin(axis=-1)]
    assert np.all(np.abs(np.abs(deq) / step - q) <= np.abs(nearest - q) + 1e-12)
    assert np.array_equal(np.signbit(deq) & (deq != 0), np.signbit(w) & (deq != 0))


def test_mx_layer_with_exact_values_equals_dense_expert():
    """Unit scales (code 127) and activations already on the MXFP8 grid with a 448-sized
    element per block: the quantisation of x changes nothing, so the MX expert equals the
    dense expert on the decoded weights with only h quantised."""
    rng = np.random.default_rng(53)
    H, I, T = 64, 64, 3
    codes = lambda r, c: rng.integers(0, 256, size=(r, c // 2), dtype=np.uint8)
    cg, cu, cd = codes(I, H), codes(I, H), codes(H, I)
    ones = lambda r, c: np.full((r, c // 32), 127, np.uint8)
    ex = mo.Experts(cg[None], cu[None], cd[None], mx=(ones(I, H)[None], ones(I, H)[None],
                                                      ones(H, I)[None]))
    assert ex.quant == "mx"
    Wg, Wu, Wd = ex.expert(0)
    vals = mo.e4m3_values()
    x = rng.choice(vals[np.isfinite(vals) & (np.abs(vals) <= 2)], size=(T, H)) * 2.0 ** -8
    x[:, 0] = x[:, 32] = 448 * 2.0 ** -8                       # amax 1.75: X = -8
    assert np.array_equal(mo.quantize_mxfp8(x), x)
    y = mo.expert_ffn(x, np.array([0, T]), np.arange(T), ex)
    g, u = x @ Wg.T, x @ Wu.T
    h = g * mo.sigmoid(g) * u
    assert mo.rel_l2(y, mo.quantize_mxfp8(h) @ Wd.T) < 1e-14


def test_mx_token_major_equals_expert_major():
    shape = synth.LayerShape("mx_small", T=6, H=128, I=64, E=8, G=2, Gk=1, k=2, S=1,
                             act="bf16", wt="mxfp4", x_dist="rms", bias_std=0.0, seed=54)
    cpu = synth.make_layer(shape)
    from tests.helpers import np_exact, oracle_experts
    ex = oracle_experts(cpu)
    assert ex.mx and ex.quant == "mx"
    out = mo.forward(np_exact(cpu["x"]), np_exact(cpu["w_router"]), None, ex, shape.G, shape.Gk,
                     shape.k)
    tm = mo.forward_tokenmajor(np_exact(cpu["x"]), ex, out["ids"], out["w"])
    assert mo.rel_l2(out["y"], tm) < 1e-12
