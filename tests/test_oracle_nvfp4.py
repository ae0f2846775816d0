"""Pins of the oracle's NVFP4 decoding (reading R15) against things other than itself:
IEEE-754 bit patterns built independently, a row worked by hand, the optimality of the
generator's rounding under the oracle's decode, and the dense path with the same
weights."""
import struct
from pathlib import Path

import numpy as np
import torch

from oracle import moe_oracle as mo
import synth

GOLDEN = Path(__file__).parent / "golden"


def _e2m1_by_bits(code: int) -> float:
    """The E2M1 value of `code` built as a float32 bit pattern: sign to bit 31, the
    exponent rebased from bias 1 to bias 127, the mantissa bit to bit 22."""
    sign, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        bits = (126 << 23) if m else 0          # 0.5 = 2^-1, or zero
    else:
        bits = ((e - 1 + 127) << 23) | (m << 22)
    return struct.unpack("<f", struct.pack("<I", (sign << 31) | bits))[0]


def test_e2m1_table_matches_bit_patterns():
    table = mo.e2m1_values()
    for c in range(16):
        assert table[c] == _e2m1_by_bits(c), c
    assert table.max() == 6.0 and table.min() == -6.0


def _golden():
    f = {}
    for line in (GOLDEN / "nvfp4_worked.txt").read_text().splitlines():
        if line and not line.startswith("#"):
            key, *vals = line.split()
            f[key] = vals
    return f


def test_worked_row():
    f = _golden()
    packed = np.array([int(v, 16) for v in f["packed"]], dtype=np.uint8)[None]
    bs = np.array([int(v, 16) for v in f["block_scales"]], dtype=np.uint8)[None]
    got = mo.dequant_nvfp4(packed, bs, float(f["matrix_scale"][0]))[0]
    want = np.array([float(v) for v in f["expected"]])
    np.testing.assert_array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))   # -0 stays -0


def test_unpack_low_nibble_first():
    assert mo.nvfp4_unpack(np.array([[0x21, 0xF0]], dtype=np.uint8)).tolist() == [[1, 2, 0, 15]]


def test_generator_rounding_is_nearest_under_the_oracle_decode():
    """Every stored code is a nearest E2M1 value of w / (block scale * matrix scale)
    (within the saturating range), so the decode and the encode agree on the format."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((3, 8, 64)) * 0.02).astype(np.float32)
    w[1, 2, :16] = 0.0                                      # an all-zero block
    packed, bs, g = synth._encode_nvfp4(w)
    table = mo.e2m1_values()
    for n in range(3):
        deq = mo.dequant_nvfp4(packed[n].numpy(), bs[n].numpy(), float(g[n]))
        den = np.repeat(mo.e4m3_decode(bs[n].numpy()), 16, axis=1) * float(g[n])
        codes = mo.nvfp4_unpack(packed[n].numpy())
        q = np.where(den > 0, w[n].astype(np.float64) / np.where(den > 0, den, 1), 0.0)
        qs = np.clip(q, -6.0, 6.0)
        best = np.min(np.abs(qs[..., None] - table[None, None, :]), axis=-1)
        assert np.all(np.abs(qs - table[codes]) <= best + 1e-7)
        assert np.all(np.abs(deq - w[n]) <= np.abs(den) * 1.0 + 1e-12)   # within one E2M1 step
    assert np.all(mo.nvfp4_unpack(packed[1].numpy())[2, :16] % 8 == 0)   # zero block -> zero codes


def test_experts_nvfp4_equal_the_dense_path():
    shape = synth.LayerShape("nvt", 6, 64, 32, 4, 2, 1, 2, 1, "bf16", "nvfp4", "rms", 0.0, 9)
    L = synth.make_layer(shape)
    f = lambda t: None if t is None else t.numpy()
    nv = tuple(f(L[k]) for k in ("b_gate", "b_up", "b_down", "g_gate", "g_up", "g_down"))
    sh_nv = tuple(f(L[k]) for k in ("sh_b_gate", "sh_b_up", "sh_b_down", "sh_g_gate", "sh_g_up",
                                    "sh_g_down"))
    ex = mo.Experts(f(L["w_gate"]), f(L["w_up"]), f(L["w_down"]), sh_gate=f(L["sh_gate"]),
                    sh_up=f(L["sh_up"]), sh_down=f(L["sh_down"]), nv=nv, sh_nv=sh_nv)

    def dense(key, bkey, gkey):
        return np.stack([mo.dequant_nvfp4(L[key][e].numpy(), L[bkey][e].numpy(), float(L[gkey][e]))
                         for e in range(len(L[key]))])
    dn = mo.Experts(dense("w_gate", "b_gate", "g_gate"), dense("w_up", "b_up", "g_up"),
                    dense("w_down", "b_down", "g_down"),
                    sh_gate=dense("sh_gate", "sh_b_gate", "sh_g_gate"),
                    sh_up=dense("sh_up", "sh_b_up", "sh_g_up"),
                    sh_down=dense("sh_down", "sh_b_down", "sh_g_down"))
    x = L["x"].float().numpy()
    wr = L["w_router"].float().numpy()
    y1 = mo.forward(x, wr, None, ex, shape.G, shape.Gk, shape.k)
    y2 = mo.forward(x, wr, None, dn, shape.G, shape.Gk, shape.k)
    np.testing.assert_array_equal(y1["y"], y2["y"])
    # the token-major formulation (no permutation) agrees to rounding order
    y3 = mo.forward_tokenmajor(x, dn, y1["ids"], y1["w"])
    np.testing.assert_allclose(y1["y"], y3, rtol=1e-12, atol=1e-14)
    assert not np.allclose(dense("w_gate", "b_gate", "g_gate"), dense("w_up", "b_up", "g_up"))
