"""Python binding of libcolimoe.so: one routed MoE layer in HIP kernels for gfx950.

Argument marshalling only. Every step of the layer runs in the library's kernels;
PyTorch supplies device memory and the stream. There is no fallback path: if the
library is not built, importing any entry point raises.

Entry points (same names as the C ABI in include/coli_moe.h):
    quantize_q8_0, route, group, ffn, layer, layer_noalloc, layer_profiled,
    blob_bytes, workspace_bytes, scratch_bytes, num_stages, stage_name, strerror;
plus TimingEvents (HIP events for layer_profiled) and alloc_workspace.
Tensors must be CUDA tensors, contiguous, with the dtypes documented in the header.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcolimoe.so")

COLI_OK, COLI_E_INVALID, COLI_E_UNSUPPORTED, COLI_E_WORKSPACE, COLI_E_ALIGN, COLI_E_DEVICE = 0, -1, -2, -3, -4, -5
COLI_E_SCRATCH = -6


class ColiError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


class Cfg(C.Structure):
    """coli_moe_cfg."""
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("n_group", C.c_int32), ("topk_group", C.c_int32), ("routed_scaling_factor", C.c_float),
                ("has_shared", C.c_int32), ("wfmt", C.c_int32), ("scale_group", C.c_int32), ("topp", C.c_float)]


class _Weights(C.Structure):
    _fields_ = [("experts", C.c_void_p), ("scales", C.c_void_p), ("router_w", C.c_void_p),
                ("router_bias", C.c_void_p)]


def make_cfg(hidden, ffn, n_experts, top_k, n_group=1, topk_group=1, rsf=1.0, has_shared=False, wbits=4,
             scale_group=0, topp=0.0, **_ignored) -> Cfg:
    return Cfg(hidden, ffn, n_experts, top_k, n_group, topk_group, rsf, int(bool(has_shared)), wbits, scale_group,
               topp)


W_MXFP4 = 40  # wbits of MXFP4 weights (COLI_W_MXFP4; scale_group 32, E8M0 scale bytes)


@dataclass
class Weights:
    """Device tensors of one layer: experts uint8 [(E+S) * blob], scales fp32 [(E+S), scales_per_expert]
    (uint8 E8M0 codes for MXFP4), router_w fp32 [E, H], router_bias fp32 [E]."""
    experts: object
    scales: object
    router_w: object
    router_bias: object

    def c(self) -> _Weights:
        return _Weights(_ptr(self.experts), _ptr(self.scales), _ptr(self.router_w), _ptr(self.router_bias))


_lib = None

EXPORTS = {
    "coli_moe_blob_bytes": (C.c_size_t, [C.c_void_p]),
    "coli_moe_scales_per_expert": (C.c_size_t, [C.c_void_p]),
    "coli_moe_workspace_bytes": (C.c_size_t, [C.c_void_p, C.c_int32]),
    "coli_moe_quantize_q8_0": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "coli_moe_route": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_size_t, C.c_void_p]),
    "coli_moe_group": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_void_p]),
    "coli_moe_ffn": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_size_t, C.c_void_p]),
    "coli_tier_init": (C.c_int, [C.c_void_p]),
    "coli_tier_plan": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p]),
    "coli_moe_tier_stage": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "coli_moe_tier_workspace_bytes": (C.c_size_t, [C.c_void_p, C.c_int32, C.c_int32]),
    "coli_moe_layer_tiered": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p, C.c_void_p]),
    "coli_moe_tier_prefetch": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p,
                                         C.c_void_p, C.c_void_p]),
    "coli_moe_layer": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "coli_moe_scratch_bytes": (C.c_size_t, []),
    "coli_moe_layer_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p]),
    "coli_moe_layer_profiled": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                          C.c_void_p, C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p),
                                          C.c_int32]),
    "coli_moe_num_stages": (C.c_int, []),
    "coli_moe_stage_name": (C.c_char_p, [C.c_int32]),
    "coli_moe_strerror": (C.c_char_p, [C.c_int]),
}


def lib():
    """Load libcolimoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(quantized_moe_sigmoid_amd/build.py); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return C.c_void_p(t.data_ptr())


def _stream(stream, ref):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return C.c_void_p(stream.cuda_stream)


def _dt(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _check(rc, what):
    if rc != COLI_OK:
        raise ColiError(rc, what)


def strerror(status: int) -> str:
    return lib().coli_moe_strerror(status).decode()


def blob_bytes(cfg: Cfg) -> int:
    return int(lib().coli_moe_blob_bytes(C.byref(cfg)))


def scales_per_expert(cfg: Cfg) -> int:
    return int(lib().coli_moe_scales_per_expert(C.byref(cfg)))


def workspace_bytes(cfg: Cfg, T_max: int) -> int:
    return int(lib().coli_moe_workspace_bytes(C.byref(cfg), T_max))


def num_stages() -> int:
    return int(lib().coli_moe_num_stages())


def stage_name(i: int) -> str:
    return lib().coli_moe_stage_name(i).decode()


def alloc_workspace(cfg: Cfg, T_max: int, device="cuda"):
    import torch
    n = workspace_bytes(cfg, T_max)
    if n == 0:
        raise ColiError(COLI_E_UNSUPPORTED, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def quantize_q8_0(x, q, d, stream=None):
    import torch
    _dt(x, torch.float32, "x"), _dt(q, torch.int8, "q"), _dt(d, torch.float32, "d")
    rows, cols = x.shape
    _check(lib().coli_moe_quantize_q8_0(_ptr(x), rows, cols, _ptr(q), _ptr(d), _stream(stream, x)),
           "coli_moe_quantize_q8_0")


def route(cfg: Cfg, w: Weights, x, topk_idx, topk_w, workspace, stream=None):
    import torch
    _dt(x, torch.float32, "x"), _dt(topk_idx, torch.int32, "topk_idx"), _dt(topk_w, torch.float32, "topk_w")
    wc = w.c()
    _check(lib().coli_moe_route(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(topk_idx), _ptr(topk_w),
                                _ptr(workspace), workspace.numel(), _stream(stream, x)), "coli_moe_route")


def group(cfg: Cfg, topk_idx, T, cnt, off, perm, active, n_active, stream=None):
    import torch
    for n, t in (("topk_idx", topk_idx), ("cnt", cnt), ("off", off), ("perm", perm), ("active", active),
                 ("n_active", n_active)):
        _dt(t, torch.int32, n)
    _check(lib().coli_moe_group(C.byref(cfg), _ptr(topk_idx), T, _ptr(cnt), _ptr(off), _ptr(perm), _ptr(active),
                                _ptr(n_active), _stream(stream, topk_idx)), "coli_moe_group")


def ffn(cfg: Cfg, w: Weights, x, topk_idx, topk_w, off, perm, active, n_active, out, workspace, stream=None):
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out"), _dt(topk_w, torch.float32, "topk_w")
    wc = w.c()
    _check(lib().coli_moe_ffn(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(topk_idx), _ptr(topk_w),
                              _ptr(off), _ptr(perm), _ptr(active), _ptr(n_active), _ptr(out), _ptr(workspace),
                              workspace.numel(), _stream(stream, x)), "coli_moe_ffn")


def layer(cfg: Cfg, w: Weights, x, out, workspace, topk_idx=None, topk_w=None, stream=None):
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out")
    if topk_idx is not None:
        _dt(topk_idx, torch.int32, "topk_idx")
    if topk_w is not None:
        _dt(topk_w, torch.float32, "topk_w")
    wc = w.c()
    _check(lib().coli_moe_layer(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(out), _ptr(topk_idx),
                                _ptr(topk_w), _ptr(workspace), workspace.numel(), _stream(stream, x)),
           "coli_moe_layer")


def scratch_bytes() -> int:
    """Bytes of the fixed per-GPU scratch that layer_noalloc runs on."""
    return int(lib().coli_moe_scratch_bytes())


def layer_noalloc(cfg: Cfg, w: Weights, x, out, topk_idx=None, topk_w=None, stream=None):
    """coli_moe_layer_noalloc: the whole layer with no workspace argument, on the library's
    fixed scratch of the current device (calls on one GPU must not overlap)."""
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out")
    if topk_idx is not None:
        _dt(topk_idx, torch.int32, "topk_idx")
    if topk_w is not None:
        _dt(topk_w, torch.float32, "topk_w")
    wc = w.c()
    _check(lib().coli_moe_layer_noalloc(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(out), _ptr(topk_idx),
                                        _ptr(topk_w), _stream(stream, x)), "coli_moe_layer_noalloc")


class TimingEvents:
    """HIP events for stage timing, created with hipEventDisableSystemFence so that
    recording one does not write back and invalidate the caches (which would add
    microseconds to the stage it closes). Pass to layer_profiled; read with
    elapsed_ms(i, j) after synchronising the stream."""

    _DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import torch  # noqa: F401  (loads the HIP runtime this process already uses)
        self._hip = C.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self._hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self._hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.events = []
        for _ in range(n):
            ev = C.c_void_p()
            rc = self._hip.hipEventCreateWithFlags(C.byref(ev), self._DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.events.append(ev)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = C.c_float()
        rc = self._hip.hipEventElapsedTime(C.byref(ms), self.events[i], self.events[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.events:
            self._hip.hipEventDestroy(ev)
        self.events = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_profiled(cfg: Cfg, w: Weights, x, out, workspace, events, stream=None):
    """events: a TimingEvents(num_stages() + 1), or a list of num_stages()+1
    torch.cuda.Event(enable_timing=True)."""
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out")
    if isinstance(events, TimingEvents):
        handles = [e.value for e in events.events]
    else:
        for e in events:  # torch creates the HIP event lazily, on its first record
            if e.cuda_event == 0:
                e.record(stream if stream is not None else torch.cuda.current_stream(x.device))
        handles = [e.cuda_event for e in events]
    arr = (C.c_void_p * len(handles))(*[C.c_void_p(h) for h in handles])
    wc = w.c()
    _check(lib().coli_moe_layer_profiled(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream, x), arr, len(handles)),
           "coli_moe_layer_profiled")


# ------------------------------------------------------------------ expert tier
class _TierC(C.Structure):
    _fields_ = [("n_experts", C.c_int32), ("slots", C.c_int32), ("slot_of", C.c_void_p), ("expert_in", C.c_void_p),
                ("last_use", C.c_void_p), ("pinned", C.c_void_p), ("clock", C.c_uint64)]


class Tier:
    """Host-side state of one layer's pool of `slots` HBM expert slots (coli_tier): which
    expert each slot holds, LRU clocks, and the pinned experts (never evicted once loaded)."""

    def __init__(self, n_experts: int, slots: int, pinned=None):
        import numpy as np
        self.slot_of = np.full(n_experts, -1, np.int32)
        self.expert_in = np.full(slots, -1, np.int32)
        self.last_use = np.zeros(slots, np.uint64)
        self.pinned = None if pinned is None else np.ascontiguousarray(pinned, np.uint8)
        self.c = _TierC(n_experts, slots, self.slot_of.ctypes.data, self.expert_in.ctypes.data,
                        self.last_use.ctypes.data, None if self.pinned is None else self.pinned.ctypes.data, 0)
        _check(lib().coli_tier_init(C.byref(self.c)), "coli_tier_init")

    def plan(self, topk_idx):
        """Plan one batch from a host route [T][k]: (slot_idx [T][k], load_expert, load_slot)."""
        import numpy as np
        idx = np.ascontiguousarray(topk_idx, np.int32)
        T, k = idx.shape
        slot_idx = np.empty_like(idx)
        le = np.empty(self.c.slots, np.int32)
        ls = np.empty(self.c.slots, np.int32)
        n = C.c_int32(0)
        _check(lib().coli_tier_plan(C.byref(self.c), idx.ctypes.data, T, k, slot_idx.ctypes.data, le.ctypes.data,
                                    ls.ctypes.data, C.byref(n)), "coli_tier_plan")
        return slot_idx, le[: n.value].copy(), ls[: n.value].copy()


def tier_stage(cfg: Cfg, slots: int, host_experts, host_scales, load_expert, load_slot, slot_experts, slot_scales,
               stream=None):
    """Enqueue the host->HBM copies of a plan. host_*: CPU tensors (pinned for asynchronous
    copies), slot_*: CUDA tensors of the pool; load_*: host int32 arrays."""
    import numpy as np
    le = np.ascontiguousarray(load_expert, np.int32)
    ls = np.ascontiguousarray(load_slot, np.int32)
    assert le.shape == ls.shape
    _check(lib().coli_moe_tier_stage(C.byref(cfg), slots, C.c_void_p(host_experts.data_ptr()),
                                     C.c_void_p(host_scales.data_ptr()), le.ctypes.data, ls.ctypes.data, le.size,
                                     _ptr(slot_experts), _ptr(slot_scales), _stream(stream, slot_experts)),
           "coli_moe_tier_stage")


class HipEvent:
    """A plain HIP event (timing disabled), e.g. the copy event of layer_tiered."""

    def __init__(self):
        import torch  # noqa: F401  (the HIP runtime this process already uses)
        self._hip = C.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self._hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.handle = C.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(C.byref(self.handle), 0x2)  # hipEventDisableTiming
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def close(self):
        if self.handle:
            self._hip.hipEventDestroy(self.handle)
            self.handle = C.c_void_p()


def tier_workspace_bytes(cfg: Cfg, slots: int, T_max: int) -> int:
    return int(lib().coli_moe_tier_workspace_bytes(C.byref(cfg), slots, T_max))


def alloc_tier_workspace(cfg: Cfg, slots: int, T_max: int, device):
    import torch
    n = tier_workspace_bytes(cfg, slots, T_max)
    if n == 0:
        raise ColiError(COLI_E_INVALID, "coli_moe_tier_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def layer_tiered(cfg: Cfg, w: Weights, tier: Tier, host_experts, host_scales, pool_experts, pool_scales, x, out,
                 workspace, copy_stream, copy_event: HipEvent, topk_idx=None, topk_w=None, stream=None):
    """coli_moe_layer_tiered: route, plan, misses copied on copy_stream while the resident
    pairs compute on `stream`, then the missing pairs and the combine."""
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out")
    wc = w.c()
    _check(lib().coli_moe_layer_tiered(C.byref(cfg), C.byref(wc), C.byref(tier.c), C.c_void_p(host_experts.data_ptr()),
                                       C.c_void_p(host_scales.data_ptr()), _ptr(pool_experts), _ptr(pool_scales),
                                       _ptr(x), x.shape[0], _ptr(out), _ptr(topk_idx), _ptr(topk_w), _ptr(workspace),
                                       workspace.numel(), _stream(stream, x), C.c_void_p(copy_stream.cuda_stream),
                                       copy_event.handle), "coli_moe_layer_tiered")


def tier_prefetch(cfg: Cfg, w: Weights, tier: Tier, host_experts, host_scales, pool_experts, pool_scales, x,
                  workspace, copy_stream, stream=None) -> int:
    """coli_moe_tier_prefetch: stage the union that w's router predicts for x into that
    layer's pool on copy_stream; returns the number of experts copied."""
    import torch
    _dt(x, torch.float32, "x")
    wc = w.c()
    n = C.c_int32(0)
    _check(lib().coli_moe_tier_prefetch(C.byref(cfg), C.byref(wc), C.byref(tier.c), C.c_void_p(host_experts.data_ptr()),
                                        C.c_void_p(host_scales.data_ptr()), _ptr(pool_experts), _ptr(pool_scales),
                                        _ptr(x), x.shape[0], _ptr(workspace), workspace.numel(), _stream(stream, x),
                                        C.c_void_p(copy_stream.cuda_stream), C.byref(n)), "coli_moe_tier_prefetch")
    return n.value
