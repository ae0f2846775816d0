"""Shared test plumbing: move synthetic layers to the GPU, run the oracle on them,
and compare routing with the near-tie rule."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as mo
import synth

NEAR_TIE = 1e-4          # float64 logit margin below which either routing is acceptable
TOL = {"f32": 5e-3, "bf16": 5e-3, "e4m3": 2e-2, "nvfp4": 5e-3, "mxfp4": 2e-2}   # rel L2 bounds of the layer output
TOL_F32_INTERNAL = 1e-5  # fp32 layers must also be this close (no silent bf16 downcast)
# every single token's output within TOKEN_FACTOR times the layer bound: a wrong row that
# the whole-output figure would dilute (one bad (token, slot) row adds ~4e-3 in quadrature
# to an 8192-token output) fails here by orders of magnitude
TOKEN_FACTOR = 2.0

WEIGHT_KEYS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up",
               "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")
NV_KEYS = ("b_gate", "b_up", "b_down", "g_gate", "g_up", "g_down")


def np_exact(t):
    """Exact numpy copy of a CPU tensor (bf16/fp32 -> float32 values; uint8 codes as is)."""
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.float().numpy()


def oracle_experts(layer) -> mo.Experts:
    nv = sh_nv = mx = sh_mx = None
    if layer.get("b_gate") is not None and layer.get("g_gate") is None:      # MXFP4
        mx = tuple(np_exact(layer[n]) for n in ("b_gate", "b_up", "b_down"))
        if layer.get("sh_b_gate") is not None:
            sh_mx = tuple(np_exact(layer["sh_" + n]) for n in ("b_gate", "b_up", "b_down"))
    elif layer.get("b_gate") is not None:
        nv = tuple(np_exact(layer[n]) for n in NV_KEYS)
        if layer.get("sh_b_gate") is not None:
            sh_nv = tuple(np_exact(layer["sh_" + n]) for n in NV_KEYS)
    return mo.Experts(*(np_exact(layer[n]) for n in WEIGHT_KEYS), nv=nv, sh_nv=sh_nv, mx=mx,
                      sh_mx=sh_mx)


def to_device(layer, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in layer.items()}


def config_for(shape: synth.LayerShape, T=None):
    import mixture_experts_layer_route_amd as moe
    return moe.make_config(shape.T if T is None else T, shape.H, shape.I, shape.E, shape.G,
                           shape.Gk, shape.k, shape.S, shape.act, shape.wt)


def near_tie_mask(logits64, shape, tol=NEAR_TIE):
    gg, ge = mo.topk_margins(logits64, shape.G, shape.Gk, shape.k)
    return np.minimum(gg, ge) <= tol


def routing_invalid(ids_t, logits_t, G, Gk, k, tol=NEAR_TIE):
    """Why the expert ids of one token are not a routing that rounding within `tol`
    logits could produce, or None when they are.

    Valid means: k distinct ids in [0, E); some set K of Gk groups exists that contains
    every chosen expert's group, holds only groups whose score (max logit) is within
    `tol` of the Gk-th best group score, and leaves out no group more than `tol` above
    it; and no expert of K that was left out beats the lowest chosen logit by more than
    `tol`.  Among the sets K that qualify the check takes the most lenient one (extra
    groups with the lowest scores)."""
    ids_t = np.asarray(ids_t, dtype=np.int64)
    l = np.asarray(logits_t, dtype=np.float64)
    E = l.size
    n = E // G
    if ids_t.size != k or len(set(ids_t.tolist())) != k:
        return "ids are not k distinct experts"
    if ids_t.min() < 0 or ids_t.max() >= E:
        return "id out of range"
    gs = l.reshape(G, n).max(axis=1)
    thr = np.sort(gs)[::-1][Gk - 1]
    chosen_groups = set((ids_t // n).tolist())
    must = {g for g in range(G) if gs[g] > thr + tol}
    allowed = {g for g in range(G) if gs[g] >= thr - tol}
    if not chosen_groups <= allowed:
        return "a chosen expert lies in a group below the kept groups"
    base = must | chosen_groups
    if len(base) > Gk:
        return "chosen experts span more groups than are kept, or a clearly kept group was dropped"
    spare = sorted(allowed - base, key=lambda g: (gs[g], g))[:Gk - len(base)]
    kept = base | set(spare)
    cand = np.concatenate([np.arange(g * n, (g + 1) * n) for g in sorted(kept)])
    left_out = np.setdiff1d(cand, ids_t)
    if left_out.size and l[left_out].max() > l[ids_t].min() + tol:
        return "a left-out expert of the kept groups beats a chosen one"
    return None


def check_routing(gpu_ids, gpu_w, logits64, shape, w_atol=2e-6):
    """Exact ids (as sets, and order where scores differ) on tokens with a clear
    margin; validity on near-tie tokens.  Returns (near-tie mask, oracle ids)."""
    scores = mo.gate_scores(logits64)
    o_ids, _ = mo.select_experts(scores, shape.G, shape.Gk, shape.k)
    near = near_tie_mask(logits64, shape)
    gpu_ids = np.asarray(gpu_ids, dtype=np.int64)
    clear = ~near
    assert np.array_equal(np.sort(gpu_ids[clear], axis=1), np.sort(o_ids[clear], axis=1)), \
        "expert ids differ on tokens with a clear margin"
    # slot order = descending logit: exact where consecutive chosen logits differ by more
    # than the near-tie margin; where two are closer, either order is a valid ranking
    o_l = np.take_along_axis(np.asarray(logits64, dtype=np.float64), o_ids, axis=1)
    order_tie = (o_l[:, :-1] - o_l[:, 1:] <= NEAR_TIE).any(axis=1)
    strict = clear & ~order_tie
    assert np.array_equal(gpu_ids[strict], o_ids[strict]), "id order differs"
    loose = clear & order_tie
    g_l = np.take_along_axis(np.asarray(logits64, dtype=np.float64)[loose], gpu_ids[loose], axis=1)
    assert (g_l[:, 1:] - g_l[:, :-1] <= NEAR_TIE).all(), "slots not in descending logit order"
    l64 = np.asarray(logits64, dtype=np.float64)
    for t in np.nonzero(near)[0]:
        why = routing_invalid(gpu_ids[t], l64[t], shape.G, shape.Gk, shape.k)
        assert why is None, f"token {t}: {why}"
    # weights: renormalised softmax of the oracle's own scores over the GPU's ids
    w_ref = mo.renormalise(scores, gpu_ids)
    np.testing.assert_allclose(np.asarray(gpu_w, dtype=np.float64), w_ref, rtol=0, atol=w_atol)
    return near, o_ids
