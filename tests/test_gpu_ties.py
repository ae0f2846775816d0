"""Exact ties through every selection path of moe_forward.

Router rows are duplicated so that logits tie bit for bit on the GPU: one row A
(scaled up, so it often leads) copied into the first expert of Gk + 1 groups, which
ties the group scores at the kept-group boundary whenever A leads; one row B copied
into k - Gk + 1 experts of the first Gk groups, which ties experts at the k-th slot
when A and B lead.  Reading R3: the lower group / expert index must win.  The GPU's
ids are compared, in order, with the oracle's selection run on the GPU's own fp32
logits (read back from the workspace), so every token is decided exactly; the
output is then checked at the layer's bar.  Paths: the decode kernels' in-block
routing (sixteen-lane rows and whole-wave selection, bf16, fp32 and NVFP4 experts),
the small-batch route+permute kernel, and the batch selection kernels (sixteen lanes
per token, and a wave per token for expert counts that are not multiples of 16)."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as mo
from tests.helpers import config_for, to_device
from tests.test_gpu_parity import _forward_check

pytestmark = pytest.mark.gpu

S_ = synth.LayerShape

CASES = [
    # name, T, H, I, E, G, Gk, k, S, act, wt, x_dist, bias_std, seed
    ("dec_rows", 4, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 0.0, 61),     # decode, 16-lane rows
    ("dec16", 16, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 0.0, 62),
    ("dec_wave", 4, 640, 256, 40, 4, 2, 6, 0, "bf16", "bf16", "rms", 0.0, 63),       # decode, wave per token
    ("dec_f32", 16, 256, 128, 16, 4, 2, 4, 0, "f32", "f32", "normal", 0.0, 64),
    ("dec_nv4", 4, 1536, 512, 128, 8, 4, 8, 0, "bf16", "nvfp4", "rms", 0.0, 65),
    ("small", 20, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 0.0, 66),       # route+permute block
    ("small_f32", 40, 256, 128, 16, 4, 2, 4, 1, "f32", "f32", "normal", 0.0, 67),
    ("rows_bf16", 300, 1536, 512, 128, 8, 4, 8, 0, "bf16", "bf16", "rms", 0.0, 68),  # batch, 16 lanes
    ("rows_f32", 300, 256, 128, 16, 4, 2, 4, 0, "f32", "f32", "normal", 0.0, 69),
    ("rows_g1", 300, 512, 128, 256, 1, 1, 6, 2, "bf16", "bf16", "normal", 0.0, 70),
    ("wave_e40", 200, 640, 256, 40, 4, 2, 6, 0, "bf16", "bf16", "rms", 0.0, 71),     # batch, wave per token
]


def tie_router(w_router, G, Gk, k):
    """Duplicate router rows (in the stored element type, so the copies are identical)."""
    wr = w_router.clone()
    E = wr.shape[0]
    n = E // G
    if G > 1:
        a = wr[0] * 4
        for g in range(min(Gk + 1, G)):
            wr[g * n] = a
        b = wr[1] * 2
        slots = [g * n + i for i in range(1, n) for g in range(Gk)]
        for e in slots[:max(0, k - Gk + 1)]:
            wr[e] = b
    else:
        a = wr[0] * 3
        for e in range(min(k + 1, E)):
            wr[e] = a
    return wr


def _boundary_ties(l, G, Gk, k):
    """Tokens whose (Gk, Gk+1)-th group scores or (k, k+1)-th kept logits are equal."""
    T, E = l.shape
    n = E // G
    gt = et = 0
    for t in range(T):
        if G > Gk:
            gs = np.sort(l[t].reshape(G, n).max(axis=1))[::-1]
            gt += gs[Gk - 1] == gs[Gk]
        kept = np.lexsort((np.arange(G), -l[t].reshape(G, n).max(axis=1)))[:Gk] if G > 1 else [0]
        cand = np.sort(np.concatenate([l[t, g * n:(g + 1) * n] for g in kept]))[::-1]
        if k < cand.size:
            et += cand[k - 1] == cand[k]
    return int(gt), int(et)


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_route_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_exact_ties_lower_index_wins(moe, case):
    print("case: ties", case[0], flush=True)
    shape = S_(*case)
    cpu = synth.make_layer(shape)
    cpu["w_router"] = tie_router(cpu["w_router"], shape.G, shape.Gk, shape.k)
    dev = to_device(cpu)
    cfg = config_for(shape)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((shape.T, shape.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((shape.T, shape.k), dtype=torch.float32, device="cuda")
    moe.forward(cfg, dev["x"], dev, ws, ids=ids, wts=wts)
    torch.cuda.synchronize()
    off, n = moe.workspace_slot(cfg, moe.WS_LOGITS)
    lg = ws[off:off + n].cpu().view(torch.float32).numpy().reshape(shape.T, shape.E)
    lg = lg.astype(np.float64)
    copy = shape.E // shape.G if shape.G > 1 else 1          # a copy of row A
    assert np.all(lg[:, 0] == lg[:, copy]), "copied rows must tie exactly"
    gt, et = _boundary_ties(lg, shape.G, shape.Gk, shape.k)
    print(f"tokens with a tie at the group boundary {gt}, at the k-th slot {et}")
    assert gt + et > 0, "the case must exercise a tie at a selection boundary"
    o_ids, _ = mo.select_experts(mo.gate_scores(lg), shape.G, shape.Gk, shape.k)
    g_ids = ids.cpu().numpy()
    bad = np.nonzero((g_ids != o_ids).any(axis=1))[0]
    assert bad.size == 0, f"tokens {bad[:8]}: gpu {g_ids[bad[:2]]} oracle {o_ids[bad[:2]]}"
    w_ref = mo.renormalise(mo.gate_scores(lg), g_ids)
    np.testing.assert_allclose(wts.cpu().numpy(), w_ref, rtol=0, atol=2e-6)
    _forward_check(moe, shape, cpu, dev)
