"""Float64 CPU oracle of the fine-grained MoE layer (route -> permute -> SwiGLU experts -> combine).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the GPU library
and never imports it; it reads nothing but numpy arrays handed to it.

What the layer computes comes from the pages:
  * TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board", jschmied's
    comment: the config paragraph gives the Ling-3.0-tiny MoE shape (128
    experts, 8 groups of 16, 4 groups kept, hidden 1536) and says the SwiGLU
    limit lists are null (no clamp); the list "What it does not cover" says the
    router is group-limited and that the bf16 experts are computed per expert
    over the rows routed to it; the list "What #874's CUDA path now covers" describes
    checking by relative L2 against a float64 forward pass that uses identical
    expert choices.
  * HelloSun/ling30tiny model card, routing table (模型與路由): 8 experts active
    per token, 128 experts per layer; the numeric-check summary (數值檢查摘要)
    names the layer as routing plus a weighted sum of the chosen experts.
  * llama.cpp PR "Add TML Inkling architecture", PR summary: 256 experts, top-6,
    plus 2 shared experts.

Where the pages are silent the oracle takes these readings (each one is the
plainest the rest supports):
  R1  gate scores are a softmax over all E router logits;
  R2  a group's score is the largest gate score inside it (G = 1: no grouping);
  R3  ties go to the lower index, for groups and for experts;
  R4  the chosen experts' weights are renormalised to sum to 1, no extra scale;
  R5  a per-expert router bias is added to the logits before the softmax;
  R6  an expert is silu(x Wg^T) * (x Wu^T) followed by Wd, weights stored
      [out, in] row-major per expert, no clamp;
  R7  shared experts see every token with weight 1 and are added to the sum;
  R8  rows of one expert are ordered by ascending (token, slot);
  R9  block-FP8 experts are OCP e4m3 codes times one fp32 scale per 128x128
      block; activations (x, and h before the down projection) are quantised
      per token per 128 along K: scale = fp32(amax) / 448 (fp32 division),
      code = e4m3 round-to-nearest-even of fp32(v / scale), saturating at 448;
      an all-zero block gets scale 1.
  R15 NVFP4 experts (the 4-bit format TensorFold #1247 names for #874, list "What
      it does not cover"; its layout is not on the pages) are FP4 E2M1 codes
      (sign, 2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN), two per byte
      with element 2i in the low nibble, one E4M3 scale per 16 consecutive
      elements along the input dimension and one fp32 scale per expert matrix:
      weight = e2m1(code) * e4m3(block scale) * matrix scale.  Activations stay
      in their own type (no activation quantisation).
  R19 MXFP4 experts (the OCP Microscaling format gfx950's matrix cores take natively; the
      pages name 4-bit experts - NVFP4 in TensorFold #1247's list "What it does not
      cover", ROCmFP4 on the graysoft page - and give no layout): FP4 E2M1 codes, two per
      byte with element 2i in the low nibble, one E8M0 scale per 32 consecutive inputs:
      weight = e2m1(code) * 2^(scale - 127).
  R20 With MXFP4 experts the activations (x, and h before the down projection) are
      quantised per row per 32 along K to MXFP8: E8M0 shared exponent
      X = floor(log2(amax)) - 8, E4M3 elements RNE(v / 2^X) saturating at +-448; an
      all-zero block gets X = -127.  Decisions in fp32, as the kernels take them.
  R16 The decoder-layer step around the MoE block (the config paragraph of
      TensorFold #1247: 24 layers, a dense layer 0, so 23 MoE layers) is
      x_out = x + MoE(RMSNorm(x)) with RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma
      over the hidden dimension, eps = 1e-6 (no value on the pages).  The
      normalised rows are rounded to the activation type before the router and
      the experts see them, and the sum x + y is rounded to it once; the
      residual stream between layers is held in the activation type.

Every floating-point step runs in float64 except the FP8 scale/code decisions
of R9, which are taken in fp32 as the kernels take them.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

E4M3_MAX = 448.0
FP8_BLOCK = 128


def _f64(a) -> Optional[np.ndarray]:
    return None if a is None else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- routing
def router_logits(x, w_router, bias=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e])  (router projection; bias per R5)."""
    logits = _f64(x) @ _f64(w_router).T
    if bias is not None:
        logits = logits + _f64(bias)[None, :]
    return logits


def gate_scores(logits) -> np.ndarray:
    """Softmax over all E logits of each token (reading R1)."""
    logits = _f64(logits)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def _order_desc(values: np.ndarray, index: np.ndarray) -> np.ndarray:
    """Positions sorted by value descending, then by index ascending (reading R3)."""
    return np.lexsort((index, -values))


def select_experts(scores, G: int, Gk: int, k: int):
    """Group-limited top-k (TensorFold #1247, "What it does not cover": group-limited routing).

    Per token: rank the G groups by their score (R2), keep the best Gk; among
    the experts of the kept groups take the k best scores (R3 for ties).
    Returns (ids [T, k] ordered by score desc / id asc, kept groups [T, Gk] ascending).
    """
    scores = _f64(scores)
    T, E = scores.shape
    n = E // G
    ids = np.empty((T, k), dtype=np.int64)
    kept = np.empty((T, Gk), dtype=np.int64)
    for t in range(T):
        s = scores[t]
        if G > 1:
            gscore = s.reshape(G, n).max(axis=1)
            groups = np.sort(_order_desc(gscore, np.arange(G))[:Gk])
        else:
            groups = np.arange(1)
        cand = np.concatenate([np.arange(g * n, (g + 1) * n) for g in groups])
        pick = _order_desc(s[cand], cand)[:k]
        ids[t] = cand[pick]
        kept[t] = groups
    return ids, kept


def renormalise(scores, ids) -> np.ndarray:
    """w[t, j] = s[t, id_j] / sum_j' s[t, id_j']  (reading R4)."""
    scores = _f64(scores)
    sel = np.take_along_axis(scores, np.asarray(ids, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_router, bias, G: int, Gk: int, k: int):
    """Router logits -> softmax -> group-limited top-k -> renormalised weights."""
    logits = router_logits(x, w_router, bias)
    scores = gate_scores(logits)
    ids, kept = select_experts(scores, G, Gk, k)
    return ids, renormalise(scores, ids), logits


def topk_margins(logits, G: int, Gk: int, k: int):
    """Decision margins in float64 logit units, per token.

    gap_group  = Gk-th minus (Gk+1)-th best group score (max logit in group); inf if G == 1 or Gk == G.
    gap_expert = k-th minus (k+1)-th best logit among the kept groups' experts; inf if none is left out.
    A token whose min(gap_group, gap_expert) is small can be routed either way by
    rounding, so exact id comparison is restricted to tokens with a clear margin.
    """
    logits = _f64(logits)
    T, E = logits.shape
    n = E // G
    gg = np.full(T, np.inf)
    ge = np.full(T, np.inf)
    for t in range(T):
        l = logits[t]
        if G > 1:
            gmax = np.sort(l.reshape(G, n).max(axis=1))[::-1]
            if Gk < G:
                gg[t] = gmax[Gk - 1] - gmax[Gk]
            groups = _order_desc(l.reshape(G, n).max(axis=1), np.arange(G))[:Gk]
        else:
            groups = np.arange(1)
        cand = np.sort(np.concatenate([l[g * n:(g + 1) * n] for g in groups]))[::-1]
        if k < cand.size:
            ge[t] = cand[k - 1] - cand[k]
    return gg, ge


# --------------------------------------------------------------------------- permutation
def permute(ids, E: int, S: int = 0):
    """Group the T*k routed slots by expert, stable in (token, slot) order (reading R8).

    Returns offsets [E+S+1] (exclusive prefix sum of per-expert row counts; each
    shared expert owns T rows), row_token [R] (token of each row), inv [T, k]
    (row of each routed slot).  R = T*k + T*S.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.concatenate([np.bincount(flat, minlength=E), np.full(S, T, dtype=np.int64)])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    row_token = np.empty(T * k + T * S, dtype=np.int64)
    row_token[:T * k] = order // k
    for s in range(S):
        row_token[T * k + s * T:T * k + (s + 1) * T] = np.arange(T)
    inv = np.empty(T * k, dtype=np.int64)
    inv[order] = np.arange(T * k)
    return offsets, row_token, inv.reshape(T, k)


# --------------------------------------------------------------------------- FP8 (OCP e4m3)
def e4m3_values() -> np.ndarray:
    """Value of each of the 256 OCP E4M3 codes (sign, 4 exponent bits, bias 7, 3 mantissa bits;
    exponent field 0 is subnormal m/8 * 2^-6; S.1111.111 is NaN; no infinities)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        ex = (c >> 3) & 0xF
        man = c & 0x7
        if ex == 0xF and man == 0x7:
            vals[c] = np.nan
        elif ex == 0:
            vals[c] = sign * (man / 8.0) * 2.0 ** -6
        else:
            vals[c] = sign * (1.0 + man / 8.0) * 2.0 ** (ex - 7)
    return vals


def e4m3_decode(codes) -> np.ndarray:
    return e4m3_values()[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Round to nearest representable e4m3, ties to the even code, saturating at +-448.
    The sign bit follows the input's sign, so negatives that round to zero give -0 (0x80)."""
    v = np.asarray(v, dtype=np.float64)
    table = e4m3_values()
    pos_codes = np.arange(0, 0x7F)                  # 0 .. 0x7E: 0 .. 448, increasing
    pos_vals = table[pos_codes]
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(pos_vals, a, side="left"), 0, pos_vals.size - 1)
    lo = np.clip(hi - 1, 0, pos_vals.size - 1)
    dlo = a - pos_vals[lo]
    dhi = pos_vals[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (pos_codes[hi] % 2 == 0))
    mag = np.where(take_hi, pos_codes[hi], pos_codes[lo])
    sign = np.where(np.signbit(v), 0x80, 0)
    return (mag | sign).astype(np.uint8)


def quantize_act_codes(v, block: int = FP8_BLOCK):
    """Activation quantisation of reading R9, per row per `block` along the last axis,
    as stored: (codes uint8 [rows, cols], scales float32 [rows, cols / block]).

    The decisions are taken in fp32: the row values are first held in fp32 (as the
    kernels hold them), scale = fp32(amax) / 448 by one IEEE fp32 division (1 for an
    all-zero block), code = e4m3 of the fp32 quotient v / scale."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    rows, cols = v32.shape
    blocks = v32.reshape(rows, cols // block, block)
    amax = np.abs(blocks).max(axis=2)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale[amax == 0] = np.float32(1.0)
    q32 = (blocks / scale[:, :, None]).astype(np.float32)
    return e4m3_encode(q32).reshape(rows, cols), scale


def quantize_act(v, block: int = FP8_BLOCK) -> np.ndarray:
    """Activation quantisation of reading R9: the dequantised float64 values code * scale."""
    codes, scale = quantize_act_codes(v, block)
    rows, cols = codes.shape
    vals = e4m3_decode(codes).reshape(rows, cols // block, block)
    return (vals * scale[:, :, None].astype(np.float64)).reshape(rows, cols)


def dequant_blocks(codes, scales, block: int = FP8_BLOCK) -> np.ndarray:
    """[rows, cols] e4m3 codes with [rows/128, cols/128] fp32 scales -> float64 weights."""
    vals = e4m3_decode(codes)
    sc = np.repeat(np.repeat(np.asarray(scales, dtype=np.float64), block, axis=0), block, axis=1)
    return vals * sc


# --------------------------------------------------------------------------- NVFP4 (R15)
NVFP4_BLOCK = 16


def e2m1_values() -> np.ndarray:
    """Value of each of the 16 FP4 E2M1 codes: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent field 0 is subnormal m * 0.5."""
    vals = np.empty(16, dtype=np.float64)
    for c in range(16):
        sign = -1.0 if c & 0x8 else 1.0
        ex = (c >> 1) & 0x3
        man = c & 0x1
        vals[c] = sign * (man * 0.5 if ex == 0 else (1.0 + 0.5 * man) * 2.0 ** (ex - 1))
    return vals


def nvfp4_unpack(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes: element 2i in the low nibble, 2i+1 in the high."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_nvfp4(packed, block_scales, matrix_scale) -> np.ndarray:
    """[rows, K/2] packed E2M1 codes, [rows, K/16] E4M3 block scales and the fp32 scale
    of the matrix -> float64 [rows, K] weights (reading R15)."""
    vals = e2m1_values()[nvfp4_unpack(packed)]
    sc = np.repeat(e4m3_decode(block_scales), NVFP4_BLOCK, axis=-1)
    return vals * sc * float(matrix_scale)


# --------------------------------------------------------------------------- MX formats (R19, R20)
MX_BLOCK = 32


def e8m0_values() -> np.ndarray:
    """Value of each of the 256 E8M0 scale codes of the OCP Microscaling spec: 2^(c - 127),
    code 255 is NaN."""
    vals = np.ldexp(1.0, np.arange(256) - 127).astype(np.float64)
    vals[255] = np.nan
    return vals


def dequant_mxfp4(packed, scales) -> np.ndarray:
    """[rows, K/2] packed E2M1 codes (element 2i in the low nibble) and [rows, K/32] E8M0
    scale codes -> float64 [rows, K] weights (reading R19: value = e2m1 * 2^(s - 127))."""
    vals = e2m1_values()[nvfp4_unpack(packed)]
    sc = np.repeat(e8m0_values()[np.asarray(scales, dtype=np.uint8)], MX_BLOCK, axis=-1)
    return vals * sc


def quantize_mxfp8_codes(v):
    """Activation quantisation of reading R20, per row per 32 along the last axis, as
    stored: (E4M3 codes uint8 [rows, cols], E8M0 scale codes uint8 [rows, cols/32]).

    The OCP Microscaling conversion with E4M3 elements: shared exponent
    X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal, 448 = 1.75 * 2^8),
    element = E4M3 round-to-nearest-even of v / 2^X, saturating at +-448 (values from
    448 up to 512 can occur and clip); an all-zero block gets X = -127 and zero codes.
    Decisions in fp32: the values are first held in fp32, where division by 2^X is exact."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    rows, cols = v32.shape
    blocks = v32.reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2).astype(np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))          # amax = m * 2^ex, 0.5 <= m < 1
    X = np.where(amax > 0, ex - 1 - 8, -127)
    X = np.clip(X, -127, 127)
    q = blocks.astype(np.float64) / np.ldexp(1.0, X)[:, :, None]
    codes = e4m3_encode(q.astype(np.float32)).reshape(rows, cols)
    return codes, (X + 127).astype(np.uint8)


def quantize_mxfp8(v) -> np.ndarray:
    """Reading R20's activation quantisation, dequantised to float64 (code value * 2^X)."""
    codes, sc = quantize_mxfp8_codes(v)
    rows, cols = codes.shape
    vals = e4m3_decode(codes).reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    return (vals * e8m0_values()[sc][:, :, None]).reshape(rows, cols)


# --------------------------------------------------------------------------- decoder step (R16)
RMS_EPS = 1e-6


def round_bf16(v) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.  A bf16
    value has 8 significant bits: v = m * 2^e with 0.5 <= |m| < 1, so the result is
    rint(m * 2^8) * 2^(e - 8) (numpy's rint rounds halves to even).  Normal range only
    (|v| within bf16's normal exponents), which covers every activation here."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_act(v, act: str) -> np.ndarray:
    """Round to the activation type the layer stores (bf16 or fp32)."""
    if act == "bf16":
        return round_bf16(v)
    return np.asarray(v, dtype=np.float32).astype(np.float64)


def rms_norm(x, gamma, eps: float = RMS_EPS) -> np.ndarray:
    """x / sqrt(mean over the last axis of x^2 + eps) * gamma, in float64."""
    x = _f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * _f64(gamma)


def residual_layer(x, gamma, w_router, bias, experts, G: int, Gk: int, k: int,
                   act: str = "bf16", eps: float = RMS_EPS, ids=None, x_norm=None) -> dict:
    """One MoE block of the decoder step (R16): x_n = round(RMSNorm(x)); the layer runs on
    x_n; x_out = round(x + y).  `x_norm`, when given, replaces x_n (a caller that checks
    the normalisation separately runs the rest of the step on the same rows)."""
    xn = round_act(rms_norm(x, gamma, eps), act) if x_norm is None else _f64(x_norm)
    out = forward(xn, w_router, bias, experts, G, Gk, k, ids=ids)
    out["x_norm"] = xn
    out["x_out"] = round_act(_f64(x) + out["y"], act)
    return out


# --------------------------------------------------------------------------- experts
class Experts:
    """Routed and shared expert weights, decoded to float64 one expert at a time.

    Dense weights: w_gate, w_up [E, I, H], w_down [E, H, I] (any float array holding the
    exact stored values).  FP8 weights: uint8 e4m3 codes plus s_gate, s_up [E, I/128, H/128]
    and s_down [E, H/128, I/128] fp32 scales.  NVFP4 weights: packed E2M1 codes
    [E, rows, K/2] with `nv` = (b_gate, b_up, b_down, g_gate, g_up, g_down): E4M3 block
    scales [E, rows, K/16] and fp32 matrix scales [E].  Shared experts: sh_* arrays of the
    same form (`sh_nv` for NVFP4).  Only FP8 quantises activations.
    """

    def __init__(self, w_gate, w_up, w_down, s_gate=None, s_up=None, s_down=None,
                 sh_gate=None, sh_up=None, sh_down=None, sh_s_gate=None, sh_s_up=None,
                 sh_s_down=None, nv=None, sh_nv=None, mx=None, sh_mx=None):
        self.fp8 = s_gate is not None
        self.mx = mx is not None
        self.routed = (w_gate, w_up, w_down, s_gate, s_up, s_down, nv, mx)
        self.shared = (sh_gate, sh_up, sh_down, sh_s_gate, sh_s_up, sh_s_down, sh_nv, sh_mx)
        self.E = len(w_gate)
        self.S = 0 if sh_gate is None else len(sh_gate)

    @staticmethod
    def _decode(pack, e):
        wg, wu, wd, sg, su, sd, nv, mx = pack
        if mx is not None:
            bg, bu, bd = mx
            return dequant_mxfp4(wg[e], bg[e]), dequant_mxfp4(wu[e], bu[e]), dequant_mxfp4(wd[e], bd[e])
        if nv is not None:
            bg, bu, bd, gg, gu, gd = nv
            return (dequant_nvfp4(wg[e], bg[e], gg[e]), dequant_nvfp4(wu[e], bu[e], gu[e]),
                    dequant_nvfp4(wd[e], bd[e], gd[e]))
        if sg is None:
            return _f64(wg[e]), _f64(wu[e]), _f64(wd[e])
        return (dequant_blocks(wg[e], sg[e]), dequant_blocks(wu[e], su[e]),
                dequant_blocks(wd[e], sd[e]))

    @property
    def quant(self):
        """Activation quantisation of these experts: "mx" (R20), True (R9) or False."""
        return "mx" if self.mx else self.fp8

    def expert(self, e: int):
        """(Wg [I,H], Wu [I,H], Wd [H,I]) of expert e; e >= E addresses shared expert e - E."""
        if e < self.E:
            return self._decode(self.routed, e)
        return self._decode(self.shared, e - self.E)


def sigmoid(z) -> np.ndarray:
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def swiglu_expert(X, Wg, Wu, Wd, fp8=False) -> np.ndarray:
    """One SwiGLU expert on rows X (reading R6; TensorFold #1247 config paragraph: no clamp).

    h = silu(X Wg^T) * (X Wu^T), silu(z) = z * sigmoid(z);  Y = h Wd^T.
    With block-FP8 experts (fp8 True) X and h are quantised per row per 128 first
    (reading R9); with MXFP4 experts (fp8 == "mx") per row per 32 to MXFP8 (reading R20)."""
    X = _f64(X)
    quant = quantize_mxfp8 if fp8 == "mx" else quantize_act
    if fp8:
        X = quant(X)
    g = X @ Wg.T
    u = X @ Wu.T
    h = g * sigmoid(g) * u
    if fp8:
        h = quant(h)
    return h @ Wd.T


def expert_ffn(x, offsets, row_token, experts: Experts) -> np.ndarray:
    """Unweighted expert outputs in permuted row order: y_perm[r] = FFN_{expert(r)}(x[row_token[r]]).

    Every expert sees only the rows routed to it (the rows-per-expert grouping of
    TensorFold #1247, list "What it does not cover"), shared experts every token."""
    x = _f64(x)
    offsets = np.asarray(offsets, dtype=np.int64)
    row_token = np.asarray(row_token, dtype=np.int64)
    y_perm = np.zeros((int(offsets[-1]), x.shape[1]))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            Wg, Wu, Wd = experts.expert(e)
            y_perm[r0:r1] = swiglu_expert(x[row_token[r0:r1]], Wg, Wu, Wd, experts.quant)
    return y_perm


def combine(y_perm, offsets, inv, w, S: int = 0) -> np.ndarray:
    """y[t] = sum_j w[t,j] * y_perm[inv[t,j]]  +  sum_s y_perm[offsets[E+s] + t]
    (the weighted layer of the HelloSun/ling30tiny numeric-check summary; shared sum per
    the Inkling PR summary, reading R7)."""
    y_perm = _f64(y_perm)
    inv = np.asarray(inv, dtype=np.int64)
    w = _f64(w)
    T, k = inv.shape
    y = np.zeros((T, y_perm.shape[1]))
    for j in range(k):
        y += w[:, j:j + 1] * y_perm[inv[:, j]]
    E = len(offsets) - 1 - S
    for s in range(S):
        base = int(offsets[E + s])
        y += y_perm[base:base + T]
    return y


def forward(x, w_router, bias, experts: Experts, G: int, Gk: int, k: int, ids=None) -> dict:
    """The whole layer, expert-major: route, permute, run each expert on its rows, combine.

    With `ids` given (forced routing: the identical-choice comparison of TensorFold #1247
    "What #874's CUDA path now covers"), those experts are used and their weights are
    the oracle's own scores renormalised over them."""
    logits = router_logits(x, w_router, bias)
    scores = gate_scores(logits)
    if ids is None:
        ids, _ = select_experts(scores, G, Gk, k)
    ids = np.asarray(ids, dtype=np.int64)
    w = renormalise(scores, ids)
    offsets, row_token, inv = permute(ids, experts.E, experts.S)
    y_perm = expert_ffn(x, offsets, row_token, experts)
    y = combine(y_perm, offsets, inv, w, experts.S)
    return {"y": y, "ids": ids, "w": w, "logits": logits, "offsets": offsets,
            "row_token": row_token, "inv": inv, "y_perm": y_perm}


def forward_tokenmajor(x, experts: Experts, ids, w) -> np.ndarray:
    """Second formulation, no permutation: y[t] = sum_j w[t,j] FFN_{ids[t,j]}(x[t]) + sum_s FFN_s(x[t])."""
    x = _f64(x)
    ids = np.asarray(ids, dtype=np.int64)
    w = _f64(w)
    T = x.shape[0]
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(ids.shape[1]):
            Wg, Wu, Wd = experts.expert(int(ids[t, j]))
            y[t] += w[t, j] * swiglu_expert(x[t:t + 1], Wg, Wu, Wd, experts.quant)[0]
        for s in range(experts.S):
            Wg, Wu, Wd = experts.expert(experts.E + s)
            y[t] += swiglu_expert(x[t:t + 1], Wg, Wu, Wd, experts.quant)[0]
    return y


def rel_l2(a, ref) -> float:
    """||a - ref||_2 / ||ref||_2 over the whole array, in float64 (the relative L2 of
    TensorFold #1247, list "What #874's CUDA path now covers")."""
    a = _f64(a)
    ref = _f64(ref)
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))


def row_rel_l2(a, ref) -> np.ndarray:
    """Relative L2 of each row (token) of [T, H] arrays: ||a[t] - ref[t]|| / ||ref[t]||.
    A wrong row that the whole-array figure would dilute stands out here."""
    a = _f64(a)
    ref = _f64(ref)
    return np.linalg.norm(a - ref, axis=1) / np.linalg.norm(ref, axis=1)
