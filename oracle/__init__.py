"""ctypes front end of the CPU oracle (``liboracle_coli.so`` built from coli_ref.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library never does. numpy arrays in and out.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
W_MXFP4 = 40  # wbits value of MXFP4 weights (COLI_REF_W_MXFP4)
LIB_PATH = os.path.join(HERE, "liboracle_coli.so")
SOURCES = [os.path.join(HERE, "coli_ref.c")]
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU code)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, *SOURCES, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Cfg(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("ffn", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("n_group", C.c_int32), ("topk_group", C.c_int32),
                ("rsf", C.c_float), ("has_shared", C.c_int32), ("wbits", C.c_int32),
                ("scale_group", C.c_int32), ("topp", C.c_float)]


def make_cfg(hidden, ffn, n_experts, top_k, n_group=1, topk_group=1, rsf=1.0, has_shared=False, wbits=4,
             scale_group=0, topp=0.0, **_ignored) -> Cfg:
    return Cfg(hidden, ffn, n_experts, top_k, n_group, topk_group, rsf, int(bool(has_shared)), wbits, scale_group,
               topp)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        sig = {
            "coli_ref_quantize_q8_0": [P, i64, i32, P, P],
            "coli_ref_pack": [i32, P, i64, P],
            "coli_ref_unpack": [i32, P, i64, P],
            "coli_ref_moe_route": [P, P, P, P, i32, P, P],
            "coli_ref_moe_route_scores": [P, P, P, P, i32, P, P, P],
            "coli_ref_moe_group": [P, P, i32, P, P, P, P, P],
            "coli_ref_expert_ffn": [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P],
            "coli_ref_moe_ffn": [P, P, P, P, i32, P, P, P],
            "coli_ref_moe_layer": [P, P, P, P, P, P, i32, P, P, P],
            "coli_ref_mxfp4_decode": [P, i64, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.coli_ref_row_bytes.argtypes = [i32, i32]
        L.coli_ref_row_bytes.restype = C.c_int64
        L.coli_ref_blob_bytes.argtypes = [i32, i32, i32]
        L.coli_ref_blob_bytes.restype = C.c_int64
        for name in ("coli_ref_e2m1", "coli_ref_e8m0"):
            f = getattr(L, name)
            f.argtypes = [C.c_uint32]
            f.restype = C.c_double
        L.coli_ref_threads.restype = C.c_int
        L.coli_ref_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _scales(a, wbits):
    """Scales as the oracle reads them: fp32, or E8M0 bytes for MXFP4."""
    return _c(a, np.uint8 if wbits == W_MXFP4 else np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} returned {rc}")


def threads() -> int:
    return lib().coli_ref_threads()


def set_threads(n: int) -> None:
    lib().coli_ref_set_threads(int(n))


def quantize_q8_0(x):
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    d = np.empty((rows, cols // 32), np.float32)
    _check(lib().coli_ref_quantize_q8_0(_p(x), rows, cols, _p(q), _p(d)), "quantize_q8_0")
    return q, d


def pack(q, wbits):
    q = _c(q, np.int8).ravel()
    out = np.empty(q.size * wbits // 8, np.uint8)
    _check(lib().coli_ref_pack(wbits, _p(q), q.size, _p(out)), "pack")
    return out


def unpack(b, wbits, n):
    b = _c(b, np.uint8).ravel()
    assert b.size >= n * wbits // 8
    q = np.empty(n, np.int8)
    _check(lib().coli_ref_unpack(wbits, _p(b), n, _p(q)), "unpack")
    return q


def e2m1(code: int) -> float:
    return float(lib().coli_ref_e2m1(int(code)))


def e8m0(u: int) -> float:
    return float(lib().coli_ref_e8m0(int(u)))


def mxfp4_decode(b, n):
    """E2M1 values (unscaled) of n packed MXFP4 codes."""
    b = _c(b, np.uint8).ravel()
    assert b.size >= n // 2
    v = np.empty(n, np.float64)
    _check(lib().coli_ref_mxfp4_decode(_p(b), n, _p(v)), "mxfp4_decode")
    return v


def route(cfg: Cfg, router_w, router_bias, x, scores=False):
    x = _c(x, np.float32)
    T = x.shape[0]
    k = cfg.top_k
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    s = np.empty((T, cfg.n_experts), np.float64) if scores else None
    _check(lib().coli_ref_moe_route_scores(C.byref(cfg), _p(_c(router_w, np.float32)),
                                           _p(_c(router_bias, np.float32)), _p(x), T, _p(idx), _p(w), _p(s)),
           "route")
    return (idx, w, s) if scores else (idx, w)


def group(cfg: Cfg, idx):
    idx = _c(idx, np.int32)
    T = idx.shape[0]
    E = cfg.n_experts
    cnt = np.empty(E, np.int32)
    off = np.empty(E + 1, np.int32)
    perm = np.empty(T * cfg.top_k, np.int32)
    active = np.empty(E, np.int32)
    nact = np.zeros(1, np.int32)
    _check(lib().coli_ref_moe_group(C.byref(cfg), _p(idx), T, _p(cnt), _p(off), _p(perm), _p(active),
                                    _p(nact)), "group")
    return cnt, off, perm[: off[E]].copy(), active[: nact[0]].copy()


def expert_ffn(hidden, ffn, wbits, blob, scales, xq, xd, scale_group=0):
    """All intermediates of one expert on one Q8_0 row: dict of g, u, h, hq, hd, y.
    scales: one per row (scale_group 0) or one per 64 inputs of a row (scale_group 64), fp32;
    MXFP4 (wbits W_MXFP4, scale_group 32): one E8M0 byte per 32 inputs of a row."""
    blob = _c(blob, np.uint8)
    scales = _scales(scales, wbits)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.float32)
    g = np.empty(ffn, np.float64)
    u = np.empty(ffn, np.float64)
    h = np.empty(ffn, np.float32)
    hq = np.empty(ffn, np.int8)
    hd = np.empty(ffn // 32, np.float32)
    y = np.empty(hidden, np.float64)
    _check(lib().coli_ref_expert_ffn(hidden, ffn, wbits, scale_group, _p(blob), _p(scales), _p(xq), _p(xd), _p(g), _p(u),
                                     _p(h), _p(hq), _p(hd), _p(y)), "expert_ffn")
    return dict(g=g, u=u, h=h, hq=hq, hd=hd, y=y)


def ffn(cfg: Cfg, blobs, scales, x, idx, w):
    x = _c(x, np.float32)
    T = x.shape[0]
    out = np.empty((T, cfg.hidden), np.float32)
    _check(lib().coli_ref_moe_ffn(C.byref(cfg), _p(_c(blobs, np.uint8)), _p(_scales(scales, cfg.wbits)), _p(x), T,
                                  _p(_c(idx, np.int32)), _p(_c(w, np.float32)), _p(out)), "ffn")
    return out


def layer(cfg: Cfg, blobs, scales, router_w, router_bias, x):
    x = _c(x, np.float32)
    T = x.shape[0]
    out = np.empty((T, cfg.hidden), np.float32)
    idx = np.empty((T, cfg.top_k), np.int32)
    w = np.empty((T, cfg.top_k), np.float32)
    _check(lib().coli_ref_moe_layer(C.byref(cfg), _p(_c(blobs, np.uint8)), _p(_scales(scales, cfg.wbits)),
                                    _p(_c(router_w, np.float32)), _p(_c(router_bias, np.float32)), _p(x), T,
                                    _p(out), _p(idx), _p(w)), "layer")
    return out, idx, w


def blob_bytes(hidden, ffn, wbits) -> int:
    return int(lib().coli_ref_blob_bytes(hidden, ffn, wbits))
