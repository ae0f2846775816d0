"""Pins of the oracle's permutation, SwiGLU experts, combine and FP8 codec."""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as mo
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, *vals = line.split()
                out[key] = vals
    return out


def _ints(vals):
    return [int(v) for v in vals]


# ----------------------------------------------------------------- permutation
def test_permute_worked_example():
    g = _golden("permute_worked.txt")
    T, k, E, S = (int(g[n][0]) for n in ("T", "k", "E", "S"))
    ids = np.array(_ints(g["ids"])).reshape(T, k)
    off, rt, inv = mo.permute(ids, E, S)
    assert off.tolist() == _ints(g["offsets"])
    assert rt.tolist() == _ints(g["row_token"])
    assert inv.ravel().tolist() == _ints(g["inv"])


@pytest.mark.parametrize("T,k,E,S", [(1, 1, 1, 0), (37, 4, 16, 0), (64, 8, 128, 0), (50, 6, 256, 2)])
def test_permute_against_tuple_sort(T, k, E, S):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    off, rt, inv = mo.permute(ids, E, S)
    # independent construction: sort (expert, token, slot) tuples with Python's sort
    slots = sorted((int(ids[t, j]), t, j) for t in range(T) for j in range(k))
    assert rt[:T * k].tolist() == [t for _, t, _ in slots]
    for r, (_, t, j) in enumerate(slots):
        assert inv[t, j] == r
    counts = [0] * (E + S)
    for e, _, _ in slots:
        counts[e] += 1
    for s in range(S):
        counts[E + s] = T
    running = [0]
    for c in counts:
        running.append(running[-1] + c)
    assert off.tolist() == running
    assert sorted(inv.ravel().tolist()) == list(range(T * k))   # bijection onto routed rows
    for s in range(S):
        assert rt[off[E + s]:off[E + s + 1]].tolist() == list(range(T))


# ----------------------------------------------------------------- experts
def test_swiglu_worked_example():
    g = _golden("swiglu_worked.txt")
    x = np.array([[float(v) for v in g["x"]]])
    Wg = np.array([[float(v) for v in g["w_gate"]]])
    Wu = np.array([[float(v) for v in g["w_up"]]])
    Wd = np.array([[float(v)] for v in g["w_down"]])
    h = 2.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(mo.swiglu_expert(x, Wg, Wu, Wd), [[h, -2 * h]], rtol=1e-15)


def test_dense_layer_equals_torch_swiglu():
    """E=1, k=1, G=1 reduces the layer to one dense SwiGLU MLP (torch float64 library ops)."""
    rng = np.random.default_rng(21)
    T, H, I = 9, 64, 48
    x = rng.standard_normal((T, H))
    wg, wu, wd = (rng.standard_normal(s) * 0.1 for s in ((1, I, H), (1, I, H), (1, H, I)))
    out = mo.forward(x, rng.standard_normal((1, H)), None, mo.Experts(wg, wu, wd), 1, 1, 1)
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.silu(xt @ torch.from_numpy(wg[0]).T) * (xt @ torch.from_numpy(wu[0]).T)
    ref = ref @ torch.from_numpy(wd[0]).T
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-15)
    assert np.all(out["w"] == 1.0)


def test_sigmoid_matches_scipy():
    z = np.linspace(-700, 700, 20001)
    np.testing.assert_allclose(mo.sigmoid(z), scipy.special.expit(z), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("zero", ["gate", "up"])
def test_zero_gate_or_up_gives_zero(zero):
    rng = np.random.default_rng(22)
    x = rng.standard_normal((6, 32))
    wg, wu, wd = rng.standard_normal((16, 32)), rng.standard_normal((16, 32)), rng.standard_normal((32, 16))
    if zero == "gate":
        wg[:] = 0
    else:
        wu[:] = 0
    assert np.all(mo.swiglu_expert(x, wg, wu, wd) == 0.0)


def _small_layer(shape):
    lay = synth.make_layer(shape)
    f = lambda t: None if t is None else (t.numpy() if t.dtype == torch.uint8 else t.float().numpy())
    ex = mo.Experts(*(f(lay[n]) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                          "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up",
                                          "sh_s_down")))
    return lay, ex, f


@pytest.mark.parametrize("name,T", [("tiny", 16), ("inkling_small", 5), ("fp8_small", 4)])
def test_token_major_equals_expert_major(name, T):
    if name == "tiny":
        shape = synth.WORKLOADS["tiny"]
    elif name == "inkling_small":
        shape = synth.LayerShape("ink_s", T=T, H=128, I=64, E=32, G=1, Gk=1, k=6, S=2, act="bf16",
                                 wt="bf16", x_dist="normal", bias_std=0.0, seed=5)
    else:
        shape = synth.LayerShape("fp8_s", T=T, H=256, I=128, E=8, G=2, Gk=1, k=2, S=1, act="bf16",
                                 wt="e4m3", x_dist="rms", bias_std=0.0, seed=6)
    lay, ex, f = _small_layer(shape)
    out = mo.forward(f(lay["x"]), f(lay["w_router"]), f(lay["router_bias"]), ex, shape.G, shape.Gk, shape.k)
    y2 = mo.forward_tokenmajor(f(lay["x"]), ex, out["ids"], out["w"])
    assert mo.rel_l2(out["y"], y2) < 1e-12


def test_identity_experts_round_trip():
    """Permute, apply f(x) = x, combine with the routing weights: returns x since sum w = 1."""
    rng = np.random.default_rng(23)
    T, H, E, G, Gk, k = 40, 24, 16, 4, 2, 4
    x = rng.standard_normal((T, H))
    ids, w, _ = mo.route(x, rng.standard_normal((E, H)), None, G, Gk, k)
    off, rt, inv = mo.permute(ids, E)
    y = mo.combine(x[rt], off, inv, w)
    np.testing.assert_allclose(y, x, rtol=1e-13, atol=1e-14)


def test_one_hot_weights_select_one_row():
    rng = np.random.default_rng(24)
    T, k, E, H = 10, 3, 8, 5
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    off, rt, inv = mo.permute(ids, E)
    y_perm = rng.standard_normal((T * k, H))
    w = np.zeros((T, k))
    w[:, 1] = 1.0
    y = mo.combine(y_perm, off, inv, w)
    assert np.array_equal(y, y_perm[inv[:, 1]])


# ----------------------------------------------------------------- FP8 codec
def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = mo.e4m3_decode(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_rne_at_midpoints_and_values():
    vals = mo.e4m3_values()
    pos = np.sort(vals[:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2          # exact in float32 for e4m3 spacing
    probes = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    probes = np.concatenate([probes, -probes]).astype(np.float32)
    ours = mo.e4m3_encode(probes)
    ref = torch.from_numpy(probes).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    rng = np.random.default_rng(25)
    r = (rng.standard_normal(100000) * rng.choice([1e-3, 1, 50], 100000)).astype(np.float32)
    r = np.clip(r, -448, 448)
    assert np.array_equal(mo.e4m3_encode(r), torch.from_numpy(r).to(torch.float8_e4m3fn)
                          .view(torch.uint8).numpy())


def test_e4m3_encode_saturates():
    assert mo.e4m3_encode(np.array([449.0, 464.0, 1e6, -1e6], np.float32)).tolist() == \
        [0x7E, 0x7E, 0x7E, 0xFE]


def test_quantize_act_identity_zero_and_error_bound():
    rng = np.random.default_rng(26)
    vals = mo.e4m3_values()
    fin = vals[np.isfinite(vals)]
    # blocks of exactly representable values whose |max| is 448: scale 1, exact
    v = rng.choice(fin, size=(3, 256))
    v[:, 0] = 448.0
    v[:, 128] = -448.0
    assert np.array_equal(mo.quantize_act(v), v)
    assert np.array_equal(mo.quantize_act(np.zeros((2, 128))), np.zeros((2, 128)))
    # round-to-nearest: error at most half a step, relative step 2^-3 for normals
    x = rng.standard_normal((64, 512)).astype(np.float32)
    q = mo.quantize_act(x)
    amax = np.abs(x.reshape(64, 4, 128)).max(axis=2, keepdims=True)
    scale = np.repeat((amax / 448.0), 128, axis=2).reshape(64, 512)
    err = np.abs(q - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.array_equal(mo.quantize_act(q), q) or mo.rel_l2(mo.quantize_act(q), q) < 1e-6


def test_dequant_blocks_scale_identity():
    codes = np.full((256, 128), 0x38, dtype=np.uint8)          # 0x38 = 1.0
    scales = np.array([[0.25], [3.0]], dtype=np.float32)
    w = mo.dequant_blocks(codes, scales)
    assert np.all(w[:128] == 0.25) and np.all(w[128:] == 3.0)


def test_fp8_layer_with_exact_values_equals_dense_with_h_quantised():
    """Integer-valued codes with unit scales: the fp8 expert equals the dense expert on the same
    values when x is already representable (the only remaining step is h's quantisation)."""
    rng = np.random.default_rng(27)
    vals = mo.e4m3_values()
    small = vals[(np.abs(vals) <= 2) & np.isfinite(vals)]
    H, I, T = 256, 128, 3
    cg, cu, cd = (rng.choice(np.arange(256)[np.isin(vals, small)], size=s).astype(np.uint8)
                  for s in ((I, H), (I, H), (H, I)))
    ones = lambda r, c: np.ones((r // 128, c // 128), np.float32)
    Wg, Wu, Wd = mo.e4m3_decode(cg), mo.e4m3_decode(cu), mo.e4m3_decode(cd)
    x = rng.choice(vals[np.isfinite(vals)], size=(T, H))
    x[:, 0], x[:, 128] = 448.0, 448.0
    ex = mo.Experts(cg[None], cu[None], cd[None], ones(I, H)[None], ones(I, H)[None], ones(H, I)[None])
    y8 = mo.expert_ffn(x, np.array([0, T]), np.arange(T), ex)
    g, u = x @ Wg.T, x @ Wu.T
    h = g * scipy.special.expit(g) * u
    assert mo.rel_l2(y8, mo.quantize_act(h) @ Wd.T) < 1e-14


# ----------------------------------------------------------------- parity metrics
def test_rel_l2_hand_values():
    """||a - ref|| / ||ref|| over the whole array, worked by hand: a missing square root,
    a division by ||a||, or a per-row mean would each give a different number."""
    ref = np.array([[3.0, 4.0]])                       # ||ref|| = 5
    a = ref + np.array([[0.6, 0.8]])                   # ||a - ref|| = 1, ||a|| = 6
    assert mo.rel_l2(a, ref) == pytest.approx(0.2, abs=1e-15)      # not 0.04, not 1/6
    ref2 = np.array([[3.0, 4.0], [6.0, 8.0]])          # ||ref2||^2 = 125
    a2 = ref2 + np.array([[0.0, 0.0], [0.0, 5.0]])     # ||a2 - ref2|| = 5
    assert mo.rel_l2(a2, ref2) == pytest.approx(1 / np.sqrt(5), abs=1e-15)   # per-row mean: 0.25
    assert mo.rel_l2(ref2, ref2) == 0.0
    assert mo.rel_l2(-ref2, ref2) == pytest.approx(2.0, abs=1e-15)


def test_row_rel_l2_hand_values():
    ref = np.array([[3.0, 4.0], [6.0, 8.0], [0.0, 2.0]])
    a = ref + np.array([[0.6, 0.8], [0.0, 0.0], [1.0, 0.0]])
    np.testing.assert_allclose(mo.row_rel_l2(a, ref), [0.2, 0.0, 0.5], rtol=0, atol=1e-15)


def test_quantize_act_codes_hand_and_torch():
    """Stored form of reading R9.  A block whose amax is 896 has scale exactly 2, so
    its codes are those of the halved values; other blocks follow fp32 division and
    torch's saturating-free e4m3 cast of the fp32 quotient (a library routine)."""
    vals = mo.e4m3_values()
    fin = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    row = np.zeros((1, 256), np.float32)
    row[0, :128] = 2.0 * np.resize(fin, 128)           # values 2 * e4m3, amax 896
    row[0, 127] = -896.0
    rng = np.random.default_rng(41)
    row[0, 128:] = rng.standard_normal(128).astype(np.float32) * 3
    codes, scales = mo.quantize_act_codes(row)
    assert codes.dtype == np.uint8 and codes.shape == (1, 256) and scales.shape == (1, 2)
    assert scales[0, 0] == np.float32(2.0)
    assert codes[0, 127] == 0xFE                        # -448
    assert np.array_equal(mo.e4m3_decode(codes[0, :127]) * 2.0, row[0, :127].astype(np.float64))
    amax = np.float32(np.abs(row[0, 128:]).max())
    assert scales[0, 1] == amax / np.float32(448.0)    # one IEEE fp32 division
    q32 = (row[0, 128:] / scales[0, 1]).astype(np.float32)
    ref = torch.from_numpy(np.clip(q32, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(codes[0, 128:], ref.numpy())
    # all-zero block: scale 1, codes 0; dequantised form agrees with quantize_act
    z_codes, z_scales = mo.quantize_act_codes(np.zeros((2, 128)))
    assert np.all(z_codes == 0) and np.all(z_scales == 1.0)
    deq = mo.e4m3_decode(codes).reshape(1, 2, 128) * scales[:, :, None].astype(np.float64)
    assert np.array_equal(deq.reshape(1, 256), mo.quantize_act(row))
