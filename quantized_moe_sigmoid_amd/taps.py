"""Test-only binding of libcolimoe_taps.so (include/coli_moe_taps.h).

The taps library is the product's HIP sources compiled with COLI_TAPS: the same
kernels, plus a write of every output row's pre-SiLU gate and up values. Only the
parity tests use it; the product binding (quantized_moe_sigmoid_amd) never loads it.
"""
from __future__ import annotations

import ctypes as C
import os

from . import EXPORTS, Cfg, ColiError, Weights, _check, _dt, _ptr, _stream

HERE = os.path.dirname(os.path.abspath(__file__))
TAPS_LIB_PATH = os.path.join(HERE, "libcolimoe_taps.so")

TAP_EXPORTS = {
    "coli_moe_layer_taps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "coli_moe_ffn_taps": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_size_t, C.c_void_p]),
}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(TAPS_LIB_PATH):
            raise RuntimeError(f"{TAPS_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(TAPS_LIB_PATH)
        for name, (res, args) in {**EXPORTS, **TAP_EXPORTS}.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def workspace_bytes(cfg: Cfg, T_max: int) -> int:
    return int(lib().coli_moe_workspace_bytes(C.byref(cfg), T_max))


def layer_taps(cfg: Cfg, w: Weights, x, out, workspace, tap, topk_idx=None, topk_w=None, stream=None):
    """coli_moe_layer_taps; tap: fp32 CUDA tensor [T*k + has_shared*T, 2F]."""
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out"), _dt(tap, torch.float32, "tap")
    wc = w.c()
    rc = lib().coli_moe_layer_taps(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(out), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(tap), _ptr(workspace), workspace.numel(), _stream(stream, x))
    if rc != 0:
        raise ColiError(rc, "coli_moe_layer_taps")


def ffn_taps(cfg: Cfg, w: Weights, x, topk_idx, topk_w, off, perm, active, n_active, out, tap, workspace,
             stream=None):
    """coli_moe_ffn_taps; tap: fp32 CUDA tensor [T*k + has_shared*T, 2F]."""
    import torch
    _dt(x, torch.float32, "x"), _dt(out, torch.float32, "out"), _dt(tap, torch.float32, "tap")
    wc = w.c()
    _check(lib().coli_moe_ffn_taps(C.byref(cfg), C.byref(wc), _ptr(x), x.shape[0], _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(off), _ptr(perm), _ptr(active), _ptr(n_active), _ptr(out), _ptr(tap),
                                   _ptr(workspace), workspace.numel(), _stream(stream, x)), "coli_moe_ffn_taps")
