"""Wrong-row controls for the layer-output bar of the GPU parity tests.

The pages validate against a float64 forward run on the same expert choices (TensorFold
#1247, list "What #874's CUDA path now covers"), and the khronnuz/Ling-3.0-flash-exl3 card's
eight-document KL evaluation recomputes its comparisons, wrong-row controls included, in
float64 NumPy.  Here the controls run on the CPU.  The oracle's
own output, rounded once to bf16 as the kernels store it, passes both checks:
  * the whole-output relative L2;
  * the worst-token bound.
Each planted mistake fails the worst-token bound.  The mistakes are planted in the
oracle's output, never in the GPU path, and they are the kinds a grouped kernel can make:
  * a token given another token's row;
  * one (token, slot) contribution dropped;
  * one slot computed with an expert the token did not choose;
  * weights left unnormalised.
"""
import numpy as np
import pytest

from oracle import moe_oracle as mo
import synth
from tests.helpers import TOKEN_FACTOR, TOL, np_exact, oracle_experts

BAR = TOL["bf16"]


@pytest.fixture(scope="module")
def layer():
    shape = synth.LayerShape("controls", T=512, H=256, I=128, E=32, G=4, Gk=2, k=8, S=0,
                             act="bf16", wt="bf16", x_dist="rms", bias_std=0.3, seed=41)
    cpu = synth.make_layer(shape)
    x = np_exact(cpu["x"])
    ex = oracle_experts(cpu)
    out = mo.forward(x, np_exact(cpu["w_router"]), np_exact(cpu["router_bias"]), ex,
                     shape.G, shape.Gk, shape.k)
    return shape, x, ex, out


def _checks(got, ref):
    return mo.rel_l2(got, ref), float(mo.row_rel_l2(got, ref).max())


def _slot_output(x, ex, t, e):
    Wg, Wu, Wd = ex.expert(int(e))
    return mo.swiglu_expert(x[t:t + 1], Wg, Wu, Wd)[0]


def test_bf16_store_passes(layer):
    _, _, _, out = layer
    ref = out["y"]
    whole, worst = _checks(mo.round_bf16(ref), ref)
    assert whole <= BAR and worst <= TOKEN_FACTOR * BAR


def test_planted_mistakes_fail_the_token_bound(layer):
    shape, x, ex, out = layer
    ref, ids, w = out["y"], out["ids"], out["w"]
    t0, t1, j = 137, 402, 3
    cases = {}
    got = ref.copy()
    got[t0] = ref[t1]                                         # another token's row
    cases["wrong row"] = got
    got = ref.copy()
    got[t0] = ref[t0] - w[t0, j] * _slot_output(x, ex, t0, ids[t0, j])
    cases["dropped slot"] = got
    other = next(e for e in range(shape.E) if e not in set(ids[t0].tolist()))
    got = ref.copy()
    got[t0] = ref[t0] + w[t0, j] * (_slot_output(x, ex, t0, other) -
                                    _slot_output(x, ex, t0, ids[t0, j]))
    cases["wrong expert"] = got
    scale = 1.0 / w.sum(axis=1, keepdims=True)                # undo the renormalisation
    raw = mo.gate_scores(out["logits"])[np.arange(shape.T)[:, None], ids]
    cases["weights not renormalised"] = ref * (raw.sum(axis=1, keepdims=True) * scale)
    for name, got in cases.items():
        whole, worst = _checks(mo.round_bf16(got), ref)
        print(f"{name}: whole-output rel L2 {whole:.2e}, worst token {worst:.2e}")
        assert worst > TOKEN_FACTOR * BAR, name
