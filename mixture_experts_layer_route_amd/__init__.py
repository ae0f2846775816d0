"""MI355X (gfx950) fine-grained MoE layer: route -> permute -> grouped SwiGLU -> combine.

Thin ctypes binding over libmoe.so (include/moe.h).  Each function marshals
torch CUDA tensors into device pointers and the current HIP stream and calls
the C entry point of the same name; every step of the layer runs in the
library's HIP kernels.  torch supplies device memory and streams only.  If the
library is missing the calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_F32, MOE_BF16, MOE_E4M3_B128, MOE_NVFP4, MOE_MXFP4 = 0, 1, 2, 3, 4
_DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_E4M3_B128, "nvfp4": MOE_NVFP4,
           "mxfp4": MOE_MXFP4}


class MoeConfig(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "router_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
        "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down",
        "b_gate", "b_up", "b_down", "g_gate", "g_up", "g_down",
        "sh_b_gate", "sh_b_up", "sh_b_down", "sh_g_gate", "sh_g_up", "sh_g_down")]


ENTRY_POINTS = ("moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn",
                "moe_combine", "moe_forward", "moe_forward_timed", "moe_forward_residual",
                "moe_workspace_slot", "moe_forward_noalloc", "moe_pager_state_layout",
                "moe_pager_reset", "moe_paged_workspace_size", "moe_forward_paged", "moe_strerror")
NOALLOC_SCRATCH_BYTES = 16 << 20   # MOE_NOALLOC_SCRATCH_BYTES
WS_LOGITS, WS_ACT_CODES, WS_ACT_SCALES, WS_NORM_ROWS = 0, 1, 2, 3   # MOE_WS_* slots
TIMED_EVENTS = 4   # MOE_TIMED_EVENTS: start/stop of the gate/up kernel, start/stop of the down kernel

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, SZ = ctypes.c_void_p, ctypes.c_size_t
    cfgp = ctypes.POINTER(MoeConfig)
    wp = ctypes.POINTER(MoeWeights)
    sig = {
        "moe_workspace_size": [cfgp, ctypes.POINTER(SZ)],
        "moe_route": [cfgp, P, P, P, P, P, P, P, SZ, P],
        "moe_permute": [cfgp, P, P, P, P, P, SZ, P],
        "moe_expert_ffn": [cfgp, P, P, P, wp, P, P, SZ, P],
        "moe_combine": [cfgp, P, P, P, P, P, P],
        "moe_forward": [cfgp, P, wp, P, P, P, P, SZ, P],
        "moe_forward_timed": [cfgp, P, wp, P, P, P, P, SZ, P, P],
        "moe_forward_residual": [cfgp, P, P, ctypes.c_float, wp, P, P, P, P, SZ, P],
        "moe_workspace_slot": [cfgp, ctypes.c_int, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "moe_forward_noalloc": [cfgp, P, wp, P, P, P, P],
        "moe_pager_state_layout": [cfgp, ctypes.c_int32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "moe_pager_reset": [cfgp, ctypes.c_int32, P, P],
        "moe_paged_workspace_size": [cfgp, ctypes.c_int32, ctypes.POINTER(SZ)],
        "moe_forward_paged": [cfgp, P, wp, wp, ctypes.c_int32, P, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.moe_strerror.argtypes = [ctypes.c_int]
    lib.moe_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


def _check(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, load_library().moe_strerror(rc).decode())


def make_config(T: int, H: int, I: int, E: int, G: int, Gk: int, k: int, S: int = 0,
                act: str = "bf16", wt: str = "bf16") -> MoeConfig:
    return MoeConfig(T, H, I, E, G, Gk, k, S, _DTYPES[act], _DTYPES[wt])


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensors only")
    if not t.is_contiguous():
        raise ValueError("contiguous tensors only")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def workspace_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


def workspace_slot(cfg: MoeConfig, slot: int):
    """(byte offset, bytes) of an inspectable workspace slot (MOE_WS_*)."""
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(load_library().moe_workspace_slot(ctypes.byref(cfg), slot, ctypes.byref(off),
                                             ctypes.byref(n)))
    return int(off.value), int(n.value)


def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    """Caller-owned scratch (torch allocation is 256-byte aligned)."""
    return torch.empty(max(workspace_size(cfg), 256), dtype=torch.uint8, device=device)


def weights_struct(w: dict) -> MoeWeights:
    """Build the weight struct from a dict of CUDA tensors (keys as in moe.h)."""
    return MoeWeights(*[_ptr(w.get(n)) for n, _ in MoeWeights._fields_])


def route(cfg, x, w_router, bias, ws, logits: Optional[torch.Tensor] = None):
    T, k = cfg.num_tokens, cfg.topk
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    wts = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(load_library().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(bias),
                                    _ptr(ids), _ptr(wts), _ptr(logits), _ptr(ws), ws.numel(),
                                    _stream()))
    return ids, wts


def permute(cfg, ids, ws):
    T, k, E, S = cfg.num_tokens, cfg.topk, cfg.num_experts, cfg.num_shared
    offsets = torch.empty(E + S + 1, dtype=torch.int32, device=ids.device)
    row_token = torch.empty(T * (k + S), dtype=torch.int32, device=ids.device)
    inv = torch.empty((T, k), dtype=torch.int32, device=ids.device)
    _check(load_library().moe_permute(ctypes.byref(cfg), _ptr(ids), _ptr(offsets), _ptr(row_token),
                                      _ptr(inv), _ptr(ws), ws.numel(), _stream()))
    return offsets, row_token, inv


def expert_ffn(cfg, x, offsets, row_token, weights: dict, ws):
    R = cfg.num_tokens * (cfg.topk + cfg.num_shared)
    y_perm = torch.empty((R, cfg.hidden), dtype=torch.float32, device=x.device)
    wst = weights_struct(weights)
    _check(load_library().moe_expert_ffn(ctypes.byref(cfg), _ptr(x), _ptr(offsets),
                                         _ptr(row_token), ctypes.byref(wst), _ptr(y_perm),
                                         _ptr(ws), ws.numel(), _stream()))
    return y_perm


def combine(cfg, y_perm, offsets, inv, wts, out_dtype):
    y = torch.empty((cfg.num_tokens, cfg.hidden), dtype=out_dtype, device=y_perm.device)
    _check(load_library().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(offsets), _ptr(inv),
                                      _ptr(wts), _ptr(y), _stream()))
    return y


def forward(cfg, x, weights: dict, ws, y: Optional[torch.Tensor] = None,
            ids: Optional[torch.Tensor] = None, wts: Optional[torch.Tensor] = None,
            wst: Optional[MoeWeights] = None):
    """The whole layer.  Returns y (and writes ids / wts when given)."""
    if y is None:
        y = torch.empty((cfg.num_tokens, cfg.hidden), dtype=x.dtype, device=x.device)
    if wst is None:
        wst = weights_struct(weights)
    _check(load_library().moe_forward(ctypes.byref(cfg), _ptr(x), ctypes.byref(wst), _ptr(y),
                                      _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(), _stream()))
    return y


def forward_noalloc(cfg, x, weights: dict, y: Optional[torch.Tensor] = None,
                    ids: Optional[torch.Tensor] = None, wts: Optional[torch.Tensor] = None,
                    wst: Optional[MoeWeights] = None):
    """The whole layer on the library's own fixed scratch (no workspace argument, no
    allocation inside the call).  Returns y (and writes ids / wts when given)."""
    if y is None:
        y = torch.empty((cfg.num_tokens, cfg.hidden), dtype=x.dtype, device=x.device)
    if wst is None:
        wst = weights_struct(weights)
    _check(load_library().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), ctypes.byref(wst),
                                              _ptr(y), _ptr(ids), _ptr(wts), _stream()))
    return y


PAGER_COUNTERS = ("calls", "refs", "lookups", "hits", "misses", "bytes_copied")


def pager_state_layout(cfg, num_slots: int):
    """(offsets of counters, key_slot, slot_key, stamp; total bytes) of a pager state."""
    offs = (ctypes.c_size_t * 4)()
    n = ctypes.c_size_t(0)
    _check(load_library().moe_pager_state_layout(ctypes.byref(cfg), num_slots, offs,
                                                 ctypes.byref(n)))
    return tuple(int(v) for v in offs), int(n.value)


def alloc_pager_state(cfg, num_slots: int, device="cuda") -> torch.Tensor:
    """A pager state, initialised (empty arena, zero counters) on the current stream."""
    _, n = pager_state_layout(cfg, num_slots)
    state = torch.empty(n, dtype=torch.uint8, device=device)
    _check(load_library().moe_pager_reset(ctypes.byref(cfg), num_slots, _ptr(state), _stream()))
    return state


def pager_tables(cfg, num_slots: int, state: torch.Tensor) -> dict:
    """Counters and residency tables of a pager state, copied to the host."""
    (oc, ok, osl, ost), _ = pager_state_layout(cfg, num_slots)
    raw = state.cpu()
    E = cfg.num_experts
    c = raw[oc:oc + 64].view(torch.int64).tolist()
    out = dict(zip(PAGER_COUNTERS, c))
    out["key_slot"] = raw[ok:ok + 4 * E].view(torch.int32).numpy().copy()
    out["slot_key"] = raw[osl:osl + 4 * num_slots].view(torch.int32).numpy().copy()
    out["stamp"] = raw[ost:ost + 8 * num_slots].view(torch.int64).numpy().copy()
    return out


def paged_workspace(cfg, num_slots: int, device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check(load_library().moe_paged_workspace_size(ctypes.byref(cfg), num_slots, ctypes.byref(n)))
    return torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device)


def forward_paged(cfg, x, host_experts: MoeWeights, resident: MoeWeights, num_slots: int,
                  state, ws, y: Optional[torch.Tensor] = None, ids: Optional[torch.Tensor] = None,
                  wts: Optional[torch.Tensor] = None):
    """The layer with its routed experts paged from pinned host memory into an arena of
    `num_slots` slots (device-side decisions).  `host_experts` holds host pointers
    (pinned tensors: use weights_struct_host), `resident` device pointers."""
    if y is None:
        y = torch.empty((cfg.num_tokens, cfg.hidden), dtype=x.dtype, device=x.device)
    _check(load_library().moe_forward_paged(ctypes.byref(cfg), _ptr(x), ctypes.byref(host_experts),
                                            ctypes.byref(resident), num_slots, _ptr(state),
                                            _ptr(y), _ptr(ids), _ptr(wts), _ptr(ws), ws.numel(),
                                            _stream()))
    return y


def weights_struct_host(w: dict) -> MoeWeights:
    """Weight struct of pinned host tensors (the paged layer's expert store)."""
    def hp(t):
        if t is None:
            return None
        if not (t.is_pinned() and t.is_contiguous()):
            raise ValueError("the expert store must be contiguous pinned host tensors")
        return t.data_ptr()
    return MoeWeights(*[hp(w.get(n)) for n, _ in MoeWeights._fields_])


def forward_residual(cfg, x, norm_weight, weights: dict, ws, x_out: Optional[torch.Tensor] = None,
                     eps: float = 1e-6, ids: Optional[torch.Tensor] = None,
                     wts: Optional[torch.Tensor] = None, wst: Optional[MoeWeights] = None):
    """The decoder step around the layer: x_out = x + MoE(RMSNorm(x) * norm_weight).
    x_out may be x itself.  Returns x_out (and writes ids / wts when given)."""
    if x_out is None:
        x_out = torch.empty_like(x)
    if wst is None:
        wst = weights_struct(weights)
    _check(load_library().moe_forward_residual(ctypes.byref(cfg), _ptr(x), _ptr(norm_weight),
                                               ctypes.c_float(eps), ctypes.byref(wst),
                                               _ptr(x_out), _ptr(ids), _ptr(wts), _ptr(ws),
                                               ws.numel(), _stream()))
    return x_out


def forward_timed(cfg, x, wst: MoeWeights, ws, y, events_array) -> None:
    """moe_forward with start/stop events attached to the gate/up and down kernel
    dispatches.  `events_array` is a ctypes array of MOE_TIMED_EVENTS hipEvent_t
    handles (timing events: torch.cuda.Event(enable_timing=True).cuda_event, or events
    created with hipEventDisableSystemFence, as bench.py does)."""
    _check(load_library().moe_forward_timed(ctypes.byref(cfg), _ptr(x), ctypes.byref(wst), _ptr(y),
                                            None, None, _ptr(ws), ws.numel(), _stream(),
                                            events_array))
