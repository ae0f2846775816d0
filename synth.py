"""Seeded synthetic inputs for the fine-grained MoE layer.

This module only draws random numbers and stores them in the element types the
layer reads (fp32, bf16, or e4m3 codes with fp32 block scales).  It holds none
of the layer's arithmetic: no routing, no matmul, no activation function.  Both
the float64 oracle (via the tests) and the GPU path (via the tests, the smoke
check and the benchmark) consume the same tensors from here, so neither side
ever produces the other's inputs.

Shapes and value distributions follow the five workloads of the layer:

  tiny      T=16,   H=256,  I=128, E=16  (4 groups of 4, keep 2), k=4, fp32
  decode    T=4,    H=1536, I=512, E=128 (8 groups of 16, keep 4), k=8, bf16
  prefill   T=8192, same layer as decode, router bias ~N(0, 0.5) (skewed load)
  fp8       T=2048, same layer, experts e4m3 with one fp32 scale per 128x128
  inkling   T=4096, H=2048, I=512, E=256 ungrouped, k=6, 2 shared experts
  decode_nvfp4  the decode layer with NVFP4 experts (4-bit E2M1 codes, an E4M3
            scale per 16 inputs, an fp32 scale per expert matrix)
  prefill_nvfp4 the prefill layer (router bias included) with NVFP4 experts
  decode_mxfp4, prefill_mxfp4  the decode and prefill layers with MXFP4 experts (4-bit
            E2M1 codes, an E8M0 scale per 32 inputs); the layer quantises its
            activations per 32 to MXFP8
  decode_stack  23 decode MoE blocks of a decoder step (x + MoE(RMSNorm(x)) each): the
            decode layer's experts copied per block, a router and a norm weight
            drawn per block (make_router, make_norm_weight)

The Ling-3.0-tiny layer shape (128 routed experts split into 8 groups of 16,
of which 4 groups survive per token; hidden size 1536; SwiGLU experts) comes
from the config paragraph of the TensorFold issue "Ling-3.0-tiny on a Qualcomm
board"; the count of 8 routed experts per token comes from the routing table
("模型與路由") of the HelloSun/ling30tiny model card; the 256-expert, top-6,
two-shared-expert layer comes from the summary of llama.cpp PR "Add TML
Inkling architecture".  The intermediate size 512 and the hidden size
2048 of the Inkling-shaped layer are synthetic choices.

Draw order (numpy PCG64, ``default_rng(seed)``), every tensor drawn in float32:
  x; router weight; router bias (prefill only); then for each expert
  e = 0..E+S-1: gate, up, down (for fp8 each tensor is followed by its
  per-block scale factors u ~ U(0.5, 2); NVFP4 and MXFP4 draw nothing extra).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

F32, BF16, E4M3, NVFP4, MXFP4 = "f32", "bf16", "e4m3", "nvfp4", "mxfp4"


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE layer workload: sizes, element types and input recipe."""
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    I: int                 # expert intermediate size
    E: int                 # routed experts
    G: int                 # expert groups (1 = ungrouped)
    Gk: int                # groups kept per token
    k: int                 # experts per token
    S: int                 # always-on shared experts
    act: str               # element type of x, router weight and y: f32 | bf16
    wt: str                # element type of the experts: f32 | bf16 | e4m3 | nvfp4
    x_dist: str            # "normal" or "rms" (RMS-normalised N(0,1))
    bias_std: float        # std of the per-expert router bias, 0 = no bias
    seed: int
    router_std: float = 0.05
    expert_std: float = 0.02

    def with_tokens(self, T: int, seed: Optional[int] = None) -> "LayerShape":
        return dataclasses.replace(self, T=T, seed=self.seed if seed is None else seed)


WORKLOADS = {
    "tiny": LayerShape("tiny", T=16, H=256, I=128, E=16, G=4, Gk=2, k=4, S=0,
                       act=F32, wt=F32, x_dist="normal", bias_std=0.0, seed=0),
    "decode": LayerShape("decode", T=4, H=1536, I=512, E=128, G=8, Gk=4, k=8, S=0,
                         act=BF16, wt=BF16, x_dist="rms", bias_std=0.0, seed=1),
    "prefill": LayerShape("prefill", T=8192, H=1536, I=512, E=128, G=8, Gk=4, k=8, S=0,
                          act=BF16, wt=BF16, x_dist="rms", bias_std=0.5, seed=2),
    "fp8": LayerShape("fp8", T=2048, H=1536, I=512, E=128, G=8, Gk=4, k=8, S=0,
                      act=BF16, wt=E4M3, x_dist="rms", bias_std=0.0, seed=3),
    "inkling": LayerShape("inkling", T=4096, H=2048, I=512, E=256, G=1, Gk=1, k=6, S=2,
                          act=BF16, wt=BF16, x_dist="normal", bias_std=0.0, seed=4),
    "decode_nvfp4": LayerShape("decode_nvfp4", T=4, H=1536, I=512, E=128, G=8, Gk=4, k=8,
                               S=0, act=BF16, wt=NVFP4, x_dist="rms", bias_std=0.0, seed=5),
    "prefill_nvfp4": LayerShape("prefill_nvfp4", T=8192, H=1536, I=512, E=128, G=8, Gk=4, k=8,
                                S=0, act=BF16, wt=NVFP4, x_dist="rms", bias_std=0.5, seed=7),
    "decode_mxfp4": LayerShape("decode_mxfp4", T=4, H=1536, I=512, E=128, G=8, Gk=4, k=8,
                               S=0, act=BF16, wt=MXFP4, x_dist="rms", bias_std=0.0, seed=10),
    "prefill_mxfp4": LayerShape("prefill_mxfp4", T=8192, H=1536, I=512, E=128, G=8, Gk=4, k=8,
                                S=0, act=BF16, wt=MXFP4, x_dist="rms", bias_std=0.5, seed=11),
    "decode_stack": LayerShape("decode_stack", T=4, H=1536, I=512, E=128, G=8, Gk=4, k=8,
                               S=0, act=BF16, wt=BF16, x_dist="normal", bias_std=0.0, seed=6),
}
STACK_BLOCKS = 23      # MoE blocks of the 24-layer stack (layer 0 is dense)

FP8_BLOCK = 128
E4M3_MAX = 448.0


def _store(a32: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 array -> tensor in the stored element type (bf16 by torch's RNE cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    if dtype == F32:
        return t
    if dtype == BF16:
        return t.to(torch.bfloat16)
    raise ValueError(dtype)


def _encode_blocks(rng: np.random.Generator, w: np.ndarray):
    """Store one [rows, cols] expert matrix as e4m3 codes + one fp32 scale per 128x128.

    Per block: s = u * amax / 448 with u ~ U(0.5, 2), codes = e4m3(W / s) after
    clamping to +-448 (torch's cast rounds to nearest even but does not
    saturate).  The (code, scale) pair is the weight for every consumer.
    """
    rows, cols = w.shape
    rb, cb = rows // FP8_BLOCK, cols // FP8_BLOCK
    blocks = w.reshape(rb, FP8_BLOCK, cb, FP8_BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    u = rng.uniform(0.5, 2.0, size=(rb, cb)).astype(np.float32)
    s = (u * amax / np.float32(E4M3_MAX)).astype(np.float32)
    s[s == 0] = 1.0
    q = (blocks / s[:, None, :, None]).astype(np.float32)
    q = np.clip(q, -E4M3_MAX, E4M3_MAX).reshape(rows, cols)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, torch.from_numpy(s)


NVFP4_BLOCK = 16
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
E2M1_MID = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2          # rounding thresholds


def _e2m1_pack(q: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each float32 value (ties to the even code, saturating at 6;
    sign in bit 3), packed two per byte with element 2i in the low nibble.  A value on the
    midpoint between codes i and i + 1 sits above exactly i thresholds and takes i + 1
    when i is odd."""
    a = np.minimum(np.abs(q), np.float32(6.0))
    idx = np.zeros(a.shape, dtype=np.uint8)
    tie = np.zeros(a.shape, dtype=bool)
    for i, m in enumerate(E2M1_MID):                  # number of thresholds strictly below a
        idx += a > m
        if i % 2 == 1:
            tie |= a == m
    idx += tie
    codes = idx | (np.signbit(q).astype(np.uint8) << 3)
    return codes[..., 0::2] | (codes[..., 1::2] << 4)


def _encode_nvfp4(w: np.ndarray):
    """Store expert matrices [n, rows, K] as NVFP4: packed E2M1 codes [n, rows, K/2]
    (element 2i in the low nibble), E4M3 block scales [n, rows, K/16] and one fp32 scale
    per matrix [n].

    matrix scale g = amax / (6 * 448); block scale = e4m3(amax_block / (6 g)) (torch's
    round-to-nearest-even cast); code = nearest E2M1 value of w / (block scale * g), ties
    to the even code, saturating at 6.  The stored triple is the weight for every
    consumer.
    """
    n, rows, K = w.shape
    amax = np.abs(w).reshape(n, -1).max(axis=1)
    g = np.where(amax > 0, amax / (6.0 * E4M3_MAX), 1.0).astype(np.float32)
    blocks = w.reshape(n, rows, K // NVFP4_BLOCK, NVFP4_BLOCK)
    bs = (np.abs(blocks).max(axis=3) / (np.float32(6.0) * g[:, None, None])).astype(np.float32)
    bs = np.clip(bs, 0.0, E4M3_MAX)
    bcode = torch.from_numpy(bs).to(torch.float8_e4m3fn)
    den = (bcode.to(torch.float32).numpy() * g[:, None, None]).astype(np.float32)
    safe = np.where(den > 0, den, np.float32(1.0))
    q = (blocks / safe[..., None]).astype(np.float32)
    q[np.broadcast_to((den <= 0)[..., None], q.shape)] = 0.0
    packed = _e2m1_pack(q.reshape(n, rows, K))
    return torch.from_numpy(packed), bcode.view(torch.uint8), torch.from_numpy(g)


MX_BLOCK = 32


def _encode_mxfp4(w: np.ndarray):
    """Store expert matrices [n, rows, K] as MXFP4: packed E2M1 codes [n, rows, K/2]
    (element 2i in the low nibble) and E8M0 scale codes [n, rows, K/32].

    Per block of 32 inputs, the OCP Microscaling conversion: shared exponent
    X = floor(log2(amax)) - 2 (2 = exponent of E2M1's largest value, 6 = 1.5 * 2^2),
    code = nearest E2M1 value of w / 2^X, ties to the even code, saturating at 6; an
    all-zero block gets X = -127.  The stored pair is the weight for every consumer.
    """
    n, rows, K = w.shape
    blocks = w.reshape(n, rows, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=3).astype(np.float64)     # exact in float32
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.clip(np.where(amax > 0, ex - 1 - 2, -127), -127, 127)
    q = (blocks.astype(np.float64) / np.ldexp(1.0, X)[..., None]).reshape(n, rows, K).astype(np.float32)
    return torch.from_numpy(_e2m1_pack(q)), torch.from_numpy((X + 127).astype(np.uint8))


def make_norm_weight(H: int, act: str, seed: int) -> torch.Tensor:
    """Pre-MoE RMSNorm weight [H] for the decoder step: 1 + 0.1 * N(0, 1) drawn in float32
    from ``default_rng(seed)`` (its own stream, so the layer draws above are unchanged),
    stored in the activation type."""
    rng = np.random.default_rng(seed)
    return _store(np.float32(1.0) + np.float32(0.1) * rng.standard_normal(H, dtype=np.float32), act)


def make_router(E: int, H: int, act: str, seed: int, std: float = 0.05) -> torch.Tensor:
    """Router weight [E, H] ~ N(0, std) drawn in float32 from ``default_rng(seed)``, stored
    in the activation type (the decoder stack draws one per block)."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((E, H), dtype=np.float32) * np.float32(std), act)


def make_layer(shape: LayerShape) -> dict:
    """Draw one layer's inputs.  Returns CPU tensors keyed by argument name.

    Keys: x [T,H]; w_router [E,H]; router_bias [E] fp32 or None; w_gate, w_up [E,I,H];
    w_down [E,H,I] (NVFP4: packed bytes [E,I,H/2] and [E,H,I/2]); s_gate, s_up
    [E,I/128,H/128] and s_down [E,H/128,I/128] (fp8 only, else None); b_gate, b_up
    [E,I,H/16], b_down [E,H,I/16] E4M3 block scales and g_gate, g_up, g_down [E] fp32
    matrix scales (NVFP4 only, else None); sh_* the same for the S shared experts, or
    None when S == 0.
    """
    rng = np.random.default_rng(shape.seed)
    T, H, I, E, S = shape.T, shape.H, shape.I, shape.E, shape.S
    z = rng.standard_normal((T, H), dtype=np.float32)
    if shape.x_dist == "rms":
        z64 = z.astype(np.float64)
        z64 = z64 / np.sqrt(np.mean(z64 * z64, axis=1, keepdims=True))
        z = z64.astype(np.float32)
    x = _store(z, shape.act)
    w_router = _store(rng.standard_normal((E, H), dtype=np.float32) * np.float32(shape.router_std),
                      shape.act)
    bias = None
    if shape.bias_std > 0:
        bias = torch.from_numpy(rng.standard_normal(E, dtype=np.float32) * np.float32(shape.bias_std))

    fp8, nv, mx = shape.wt == E4M3, shape.wt == NVFP4, shape.wt == MXFP4
    mats = {n: [] for n in ("gate", "up", "down")}
    scales = {n: [] for n in ("gate", "up", "down")}
    gscales = {n: [] for n in ("gate", "up", "down")}
    for _e in range(E + S):
        for name, dims in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            w = rng.standard_normal(dims, dtype=np.float32) * np.float32(shape.expert_std)
            if fp8:
                c, s = _encode_blocks(rng, w)
                mats[name].append(c)
                scales[name].append(s)
            elif nv or mx:
                mats[name].append(w)             # encoded below, all experts at once
            else:
                mats[name].append(_store(w, shape.wt))

    if nv:
        for name in ("gate", "up", "down"):
            c, b, g = _encode_nvfp4(np.stack(mats[name]))
            mats[name], scales[name], gscales[name] = list(c), list(b), list(g)
    if mx:
        for name in ("gate", "up", "down"):
            c, b = _encode_mxfp4(np.stack(mats[name]))
            mats[name], scales[name] = list(c), list(b)
    out = {"x": x, "w_router": w_router, "router_bias": bias}
    for name in ("gate", "up", "down"):
        out["w_" + name] = torch.stack(mats[name][:E])
        out["sh_" + name] = torch.stack(mats[name][E:]) if S else None
        if fp8:
            out["s_" + name] = torch.stack(scales[name][:E])
            out["sh_s_" + name] = torch.stack(scales[name][E:]) if S else None
        else:
            out["s_" + name] = None
            out["sh_s_" + name] = None
        if nv or mx:
            out["b_" + name] = torch.stack(scales[name][:E])
            out["sh_b_" + name] = torch.stack(scales[name][E:]) if S else None
        if nv:
            out["g_" + name] = torch.stack(gscales[name][:E])
            out["sh_g_" + name] = torch.stack(gscales[name][E:]) if S else None
        elif mx:
            for key in ("g_", "sh_g_"):
                out[key + name] = None
        else:
            for key in ("b_", "sh_b_", "g_", "sh_g_"):
                out[key + name] = None
    return out
