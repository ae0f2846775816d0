"""The C ABI library loads, exports every symbol moe.h declares, and rejects bad
arguments before touching the GPU (these calls return before any HIP call, so
they run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(moe.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(T=4, H=1536, I=512, E=128, G=8, Gk=4, k=8, S=0, act="bf16", wt="bf16")
    base.update(kw)
    return moe.make_config(**base)


def test_workspace_size_and_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(ctypes.byref(_cfg()), ctypes.byref(n)) == 0 and n.value > 0
    bad = {
        -1: [dict(T=0), dict(H=0), dict(k=0), dict(S=-1)],
        -2: [dict(E=100, G=8), dict(Gk=9), dict(k=65), dict(k=17, Gk=8), dict(H=1530),
             dict(act="f32", wt="bf16"), dict(wt="e4m3", I=500), dict(act="e4m3", wt="e4m3"),
             dict(G=128, E=128, Gk=4), dict(E=1020, G=1, Gk=1, S=8)],
    }
    for code, cases in bad.items():
        for kw in cases:
            rc = lib.moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n))
            assert rc == code, (kw, rc)
    assert lib.moe_workspace_size(None, ctypes.byref(n)) == -1
    assert lib.moe_strerror(-3) == b"workspace smaller than moe_workspace_size()"
    assert lib.moe_strerror(12345) == b"unknown status"


def test_calls_reject_null_and_small_workspace(lib):
    cfg = _cfg()
    fake = ctypes.c_void_p(1 << 40)          # never dereferenced: validation fails first
    n = ctypes.c_size_t(0)
    lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n))
    assert lib.moe_route(ctypes.byref(cfg), None, fake, None, fake, fake, None, fake, n.value,
                         None) == -1
    assert lib.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, None, fake,
                         n.value - 1, None) == -3
    assert lib.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, None,
                         ctypes.c_void_p((1 << 40) + 8), n.value, None) == -1   # misaligned ws
    assert lib.moe_permute(ctypes.byref(cfg), fake, None, fake, fake, fake, n.value, None) == -1
    w = moe.MoeWeights()
    assert lib.moe_expert_ffn(ctypes.byref(cfg), fake, fake, fake, ctypes.byref(w), fake, fake,
                              n.value, None) == -1
    assert lib.moe_forward(ctypes.byref(cfg), fake, ctypes.byref(w), fake, None, None, fake,
                           n.value, None) == -1
    w.w_router = w.w_gate = w.w_up = w.w_down = 1 << 40
    assert lib.moe_forward(ctypes.byref(cfg), fake, ctypes.byref(w), fake, None, None, fake,
                           n.value - 256, None) == -3
    cfg8 = _cfg(wt="e4m3")                   # fp8 experts need their block scales
    assert lib.moe_forward(ctypes.byref(cfg8), fake, ctypes.byref(w), fake, None, None, fake,
                           1 << 40, None) == -1
    cfg_sh = _cfg(S=2)                       # shared experts need their arrays
    assert lib.moe_expert_ffn(ctypes.byref(cfg_sh), fake, fake, fake, ctypes.byref(w), fake,
                              fake, 1 << 40, None) == -1
    assert lib.moe_combine(ctypes.byref(cfg), None, fake, fake, fake, fake, None) == -1
    cfg4 = _cfg(wt="nvfp4")                  # NVFP4 experts need block and matrix scales
    assert lib.moe_forward(ctypes.byref(cfg4), fake, ctypes.byref(w), fake, None, None, fake,
                           1 << 40, None) == -1
    assert lib.moe_expert_ffn(ctypes.byref(cfg4), fake, fake, fake, ctypes.byref(w), fake, fake,
                              1 << 40, None) == -1        # and so does the expert FFN entry


def test_forward_residual_rejects_bad_norm_arguments(lib):
    cfg = _cfg()
    fake = ctypes.c_void_p(1 << 40)
    w = moe.MoeWeights()
    w.w_router = w.w_gate = w.w_up = w.w_down = 1 << 40
    f = lib.moe_forward_residual
    assert f(ctypes.byref(cfg), fake, None, ctypes.c_float(1e-6), ctypes.byref(w), fake, None, None,
             fake, 1 << 40, None) == -1                                   # no norm weight
    for eps in (-1.0, float("nan")):
        assert f(ctypes.byref(cfg), fake, fake, ctypes.c_float(eps), ctypes.byref(w), fake, None,
                 None, fake, 1 << 40, None) == -1
    assert f(ctypes.byref(cfg), None, fake, ctypes.c_float(1e-6), ctypes.byref(w), fake, None,
             None, fake, 1 << 40, None) == -1                             # no x
    n = ctypes.c_size_t(0)
    lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n))
    assert f(ctypes.byref(cfg), fake, fake, ctypes.c_float(1e-6), ctypes.byref(w), fake, None,
             None, fake, n.value - 256, None) == -3


def test_nvfp4_supported_shapes(lib):
    n = ctypes.c_size_t(0)
    ok = [dict(wt="nvfp4"), dict(wt="nvfp4", T=1), dict(wt="nvfp4", T=16),
          dict(wt="nvfp4", S=2), dict(wt="nvfp4", H=640, I=384, E=64, G=4, Gk=2, k=4),
          dict(wt="nvfp4", T=8, H=1024, I=256, E=256, G=1, Gk=1, k=6, S=2),
          dict(wt="nvfp4", H=512, I=1024, E=32, G=1, Gk=1, k=4, S=1),
          dict(wt="nvfp4", T=3, H=512, I=256, E=256, G=64, Gk=8, k=16),
          dict(wt="nvfp4", T=12, H=2048, I=256, E=16, G=4, Gk=2, k=4),
          dict(wt="nvfp4", T=17), dict(wt="nvfp4", T=8192), dict(wt="nvfp4", T=16, H=2048)]
    for kw in ok:
        assert lib.moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n)) == 0, kw
    bad = [dict(wt="nvfp4", H=1520), dict(wt="nvfp4", I=496), dict(wt="nvfp4", act="f32"),
           dict(wt="nvfp4", H=4096), dict(wt="nvfp4", I=2048), dict(wt="nvfp4", k=8, S=25)]
    for kw in bad:
        assert lib.moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n)) == -2, kw


def test_weights_struct_matches_header():
    """The ctypes weight struct lists moe.h's fields in the header's order."""
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    body = txt[txt.index("typedef struct {", txt.index("moe_config;")):txt.index("} moe_weights;")]
    names = re.findall(r"^\s*const\s+\w+\*\s+(\w+);", body, re.M)
    assert names == [n for n, _ in moe.MoeWeights._fields_]
    cbody = txt[txt.index("typedef struct {"):txt.index("} moe_config;")]
    cnames = re.findall(r"^\s*int\d+_t\s+(\w+);", cbody, re.M)
    assert cnames == [n for n, _ in moe.MoeConfig._fields_]


def test_forward_timed_rejects_missing_events(lib):
    cfg = _cfg()
    fake = ctypes.c_void_p(1 << 40)
    w = moe.MoeWeights()
    w.w_router = w.w_gate = w.w_up = w.w_down = 1 << 40
    assert lib.moe_forward_timed(ctypes.byref(cfg), fake, ctypes.byref(w), fake, None, None, fake,
                                 1 << 40, None, None) == -1
    ev = (ctypes.c_void_p * moe.TIMED_EVENTS)(*([1 << 40] * (moe.TIMED_EVENTS - 1) + [None]))
    assert lib.moe_forward_timed(ctypes.byref(cfg), fake, ctypes.byref(w), fake, None, None, fake,
                                 1 << 40, None, ev) == -1


def test_workspace_slots_lie_inside_the_workspace(lib):
    for kw in (dict(), dict(wt="e4m3", T=2048), dict(T=8192), dict(act="f32", wt="f32", H=256, I=128,
                                                                  E=16, G=4, Gk=2, k=4)):
        cfg = _cfg(**kw)
        total = moe.workspace_size(cfg)
        spans = []
        for slot in (moe.WS_LOGITS, moe.WS_ACT_CODES, moe.WS_ACT_SCALES, moe.WS_NORM_ROWS):
            off, n = moe.workspace_slot(cfg, slot)
            assert off % 256 == 0 and off + n <= total, (kw, slot)
            if n:
                spans.append((off, off + n))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:])), kw
        T, H, E = cfg.num_tokens, cfg.hidden, cfg.num_experts
        assert moe.workspace_slot(cfg, moe.WS_LOGITS)[1] == T * E * 4
        fp8 = kw.get("wt") == "e4m3"
        assert moe.workspace_slot(cfg, moe.WS_ACT_CODES)[1] == (T * H if fp8 else 0)
        assert moe.workspace_slot(cfg, moe.WS_ACT_SCALES)[1] == (T * H // 32 if fp8 else 0)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_slot(ctypes.byref(_cfg()), 7, ctypes.byref(n), ctypes.byref(n)) == -1
    assert lib.moe_workspace_slot(ctypes.byref(_cfg()), 0, None, ctypes.byref(n)) == -1


def test_forward_noalloc_rejects_before_any_device_work(lib):
    """Validation and the scratch limit are decided on the host, before the first HIP call."""
    fake = ctypes.c_void_p(1 << 40)
    w = moe.MoeWeights()
    cfg = _cfg(T=16)
    assert lib.moe_forward_noalloc(ctypes.byref(cfg), None, ctypes.byref(w), fake, None, None,
                                   None) == -1
    w.w_router = w.w_gate = w.w_up = w.w_down = 1 << 40
    assert lib.moe_forward_noalloc(ctypes.byref(cfg), fake, ctypes.byref(w), None, None, None,
                                   None) == -1
    big = _cfg(T=8192)
    assert moe.workspace_size(big) > moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(big), fake, ctypes.byref(w), fake, None, None,
                                   None) == -5
    assert b"MOE_NOALLOC_SCRATCH_BYTES" in lib.moe_strerror(-5)
    assert moe.workspace_size(_cfg(T=256)) <= moe.NOALLOC_SCRATCH_BYTES
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(16u << 20\)", txt)
    assert moe.NOALLOC_SCRATCH_BYTES == 16 << 20
