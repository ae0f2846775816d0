"""Shared test plumbing: move synthetic layers to the GPU, run the oracle on them,
and compare routing with the near-tie rule."""
from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as mo
import synth

NEAR_TIE = 1e-4          # float64 logit margin below which either routing is acceptable
TOL = {"f32": 5e-3, "bf16": 5e-3, "e4m3": 2e-2, "nvfp4": 5e-3}   # rel L2 bounds of the layer output
TOL_F32_INTERNAL = 1e-5  # fp32 layers must also be this close (no silent bf16 downcast)

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
    nv = sh_nv = None
    if layer.get("b_gate") is not None:
        nv = tuple(np_exact(layer[n]) for n in NV_KEYS)
        if layer.get("sh_b_gate") is not None:
            sh_nv = tuple(np_exact(layer["sh_" + n]) for n in NV_KEYS)
    return mo.Experts(*(np_exact(layer[n]) for n in WEIGHT_KEYS), nv=nv, sh_nv=sh_nv)


def to_device(layer, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in layer.items()}


def config_for(shape: synth.LayerShape, T=None):
    import mixture_experts_layer_route_amd as moe
    return moe.make_config(shape.T if T is None else T, shape.H, shape.I, shape.E, shape.G,
                           shape.Gk, shape.k, shape.S, shape.act, shape.wt)


def near_tie_mask(logits64, shape, tol=NEAR_TIE):
    gg, ge = mo.topk_margins(logits64, shape.G, shape.Gk, shape.k)
    return np.minimum(gg, ge) <= tol


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
    n = shape.E // shape.G
    for t in np.nonzero(near)[0]:
        ids_t = gpu_ids[t]
        assert len(set(ids_t.tolist())) == shape.k
        assert len({int(e) // n for e in ids_t}) <= shape.Gk
    # weights: renormalised softmax of the oracle's own scores over the GPU's ids
    w_ref = mo.renormalise(scores, gpu_ids)
    np.testing.assert_allclose(np.asarray(gpu_w, dtype=np.float64), w_ref, rtol=0, atol=w_atol)
    return near, o_ids
