"""The C-ABI library loads, exports every declared symbol, and rejects bad calls on the
host before anything is enqueued (CPU only: no call here reaches a kernel)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(coli_(?:moe|tier)_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def q():
    import quantized_moe_sigmoid_amd as q
    if not os.path.exists(q.LIB_PATH):
        from quantized_moe_sigmoid_amd import build
        build.build()
    return q


def test_exports_every_declared_symbol(q):
    names = _declared()
    assert "coli_moe_layer" in names and "coli_moe_route" in names and "coli_tier_plan" in names
    L = q.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(q.EXPORTS) == set(names)


def test_host_queries(q):
    c = q.make_cfg(6144, 2048, 256, 8, 8, 4, 2.5, True, 4)
    assert q.blob_bytes(c) == 2 * 2048 * 3072 + 6144 * 1024
    assert q.blob_bytes(q.make_cfg(6144, 2048, 256, 8, 8, 4, 2.5, True, 8)) == 3 * 2048 * 6144
    assert q.blob_bytes(q.make_cfg(6144, 2048, 256, 8, 8, 4, 2.5, True, 2)) == 3 * 2048 * 6144 // 4
    mx = q.make_cfg(6144, 2048, 256, 8, 8, 4, 2.5, True, q.W_MXFP4, scale_group=32)
    assert q.blob_bytes(mx) == 3 * 2048 * 6144 // 2
    assert q.scales_per_expert(mx) == 3 * 2048 * 6144 // 32
    assert q.workspace_bytes(c, 16) > 0 and q.workspace_bytes(c, 2048) > q.workspace_bytes(c, 16)
    assert q.num_stages() == 7
    assert [q.stage_name(i) for i in range(7)][4] == "ffn_gate_up"
    assert q.stage_name(99) == ""
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert q.strerror(s)
    assert q.strerror(-77) == "unknown status"


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _w(q, experts=FAKE, scales=FAKE, rw=FAKE, rb=FAKE):
    return q._Weights(C.c_void_p(experts), C.c_void_p(scales), C.c_void_p(rw), C.c_void_p(rb))


BAD_CFGS = [
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, n_group=3, topk_group=1), -1),   # E % G
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, n_group=2, topk_group=3), -1),   # Gk > G
    (dict(hidden=256, ffn=128, n_experts=16, top_k=9, n_group=2, topk_group=1), -1),   # k > Gk*E/G
    (dict(hidden=256, ffn=128, n_experts=16, top_k=0), -1),
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, wbits=3), -1),
    (dict(hidden=160, ffn=128, n_experts=16, top_k=4), -2),                            # H % 128
    (dict(hidden=256, ffn=96, n_experts=16, top_k=4), -2),                             # F % 128
    (dict(hidden=256, ffn=128, n_experts=2048, top_k=4), -2),                          # E > 1024
    (dict(hidden=16384, ffn=128, n_experts=16, top_k=4), -2),                          # LDS of the GEMV
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, scale_group=32), -1),            # group size 64 only
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, wbits=40), -1),                  # MXFP4: scale_group 32
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, wbits=40, scale_group=64), -1),
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, topp=1.5), -1),                  # topp in [0, 1]
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, topp=-0.1), -1),
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, topp=float("nan")), -1),
]


@pytest.mark.parametrize("cfgd,want", BAD_CFGS)
def test_bad_config_rejected(q, cfgd, want):
    c = q.make_cfg(**cfgd)
    L = q.lib()
    w = _w(q)
    p = C.c_void_p(FAKE)
    assert L.coli_moe_blob_bytes(C.byref(c)) == 0
    assert L.coli_moe_scales_per_expert(C.byref(c)) == 0
    assert L.coli_moe_workspace_bytes(C.byref(c), 8) == 0
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, 8, p, None, None, p, 1 << 30, None) == want
    assert L.coli_moe_route(C.byref(c), C.byref(w), p, 8, p, p, p, 1 << 30, None) == want
    assert L.coli_moe_group(C.byref(c), p, 8, p, p, p, p, p, None) == want
    assert L.coli_moe_ffn(C.byref(c), C.byref(w), p, 8, p, p, p, p, p, p, p, p, 1 << 30, None) == want


def test_argument_errors(q):
    c = q.make_cfg(256, 128, 16, 4)
    L = q.lib()
    p = C.c_void_p(FAKE)
    ws_need = L.coli_moe_workspace_bytes(C.byref(c), 8)
    assert ws_need > 0
    w = _w(q)
    # T = 0 is a no-op
    assert L.coli_moe_layer(C.byref(c), C.byref(w), None, 0, None, None, None, None, 0, None) == 0
    # negative T, T*k too large
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, -1, p, None, None, p, ws_need, None) == -1
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, 20000, p, None, None, p, 1 << 40, None) == -2
    assert L.coli_moe_workspace_bytes(C.byref(c), 20000) == 0
    # NULL pointers
    assert L.coli_moe_layer(C.byref(c), C.byref(w), None, 8, p, None, None, p, ws_need, None) == -1
    assert L.coli_moe_layer(C.byref(c), C.byref(_w(q, experts=0)), p, 8, p, None, None, p, ws_need, None) == -1
    assert L.coli_moe_layer(C.byref(c), None, p, 8, p, None, None, p, ws_need, None) == -1
    assert L.coli_moe_layer(None, C.byref(w), p, 8, p, None, None, p, ws_need, None) == -1
    # misaligned pointers
    assert L.coli_moe_layer(C.byref(c), C.byref(_w(q, experts=FAKE + 8)), p, 8, p, None, None, p, ws_need,
                            None) == -4
    assert L.coli_moe_layer(C.byref(c), C.byref(w), C.c_void_p(FAKE + 4), 8, p, None, None, p, ws_need,
                            None) == -4
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, 8, p, None, None, C.c_void_p(FAKE + 64), ws_need,
                            None) == -4
    # workspace too small or missing
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, 8, p, None, None, p, ws_need - 1, None) == -3
    assert L.coli_moe_layer(C.byref(c), C.byref(w), p, 8, p, None, None, None, ws_need, None) == -3
    assert L.coli_moe_ffn(C.byref(c), C.byref(w), p, 8, p, p, p, p, p, p, p, p, 16, None) == -3
    assert L.coli_moe_route(C.byref(c), C.byref(w), p, 8, p, p, p, 16, None) == -3
    # quantize
    assert L.coli_moe_quantize_q8_0(p, 4, 48, p, p, None) == -2
    assert L.coli_moe_quantize_q8_0(p, -1, 64, p, p, None) == -1
    assert L.coli_moe_quantize_q8_0(p, 0, 64, None, None, None) == 0
    assert L.coli_moe_quantize_q8_0(C.c_void_p(FAKE + 4), 4, 64, p, p, None) == -4
    # profiled: wrong event count
    arr = (C.c_void_p * 3)(p, p, p)
    assert L.coli_moe_layer_profiled(C.byref(c), C.byref(w), p, 8, p, p, ws_need, None, arr, 3) == -1


def test_header_is_plain_c():
    """include/coli_moe.h compiles as C99 (no C++ or HIP types in the boundary)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_workspace_query_covers_every_smaller_batch(q):
    """The workspace for T_max tokens also covers every T <= T_max: the query never shrinks
    as T_max grows (the router's K split shrinks with T while the batch grows)."""
    for cfgd in (dict(hidden=256, ffn=128, n_experts=256, top_k=4), dict(hidden=256, ffn=128, n_experts=16, top_k=4),
                 dict(hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8, topk_group=4, has_shared=True),
                 dict(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, has_shared=True)):
        c = q.make_cfg(**cfgd)
        Tmax = min(5000, 65535 // cfgd["top_k"])
        sizes = [q.workspace_bytes(c, T) for T in range(1, Tmax + 1, 7)]
        assert all(s > 0 for s in sizes)
        assert all(a <= b for a, b in zip(sizes, sizes[1:])), cfgd


def test_taps_library_exports_only_in_test_build():
    """libcolimoe_taps.so (COLI_TAPS) exports the product symbols plus the taps entry points of
    include/coli_moe_taps.h; the product library exports no taps symbol."""
    import quantized_moe_sigmoid_amd as q
    from quantized_moe_sigmoid_amd import taps
    if not os.path.exists(taps.TAPS_LIB_PATH):
        from quantized_moe_sigmoid_amd import build
        build.build()
    src = open(os.path.join(ROOT, "include", "coli_moe_taps.h")).read()
    names = sorted(set(re.findall(r"\b(coli_moe_\w+_taps)\s*\(", src)))
    assert names == ["coli_moe_ffn_taps", "coli_moe_layer_taps"]
    T = taps.lib()
    for n in names + _declared():
        assert hasattr(T, n), n
    prod = C.CDLL(q.LIB_PATH)
    for n in names:
        assert not hasattr(prod, n), n
    assert set(taps.TAP_EXPORTS) == set(names)


def test_noalloc_rejects_on_the_host(q):
    """coli_moe_layer_noalloc validates like coli_moe_layer and rejects batches larger than the
    fixed scratch with COLI_E_SCRATCH, all before anything is enqueued (no GPU needed)."""
    L = q.lib()
    assert q.scratch_bytes() == 32 << 20
    w = _w(q)
    p = C.c_void_p(FAKE)
    glm = q.make_cfg(6144, 2048, 256, 8, 8, 4, 2.5, True, 4)
    assert q.workspace_bytes(glm, 64) <= q.scratch_bytes() < q.workspace_bytes(glm, 128)
    assert L.coli_moe_layer_noalloc(C.byref(glm), C.byref(w), p, 128, p, None, None, None) == -6
    assert L.coli_moe_layer_noalloc(C.byref(glm), C.byref(w), p, 0, p, None, None, None) == 0
    assert L.coli_moe_layer_noalloc(C.byref(glm), C.byref(w), p, -1, p, None, None, None) == -1
    assert L.coli_moe_layer_noalloc(None, C.byref(w), p, 4, p, None, None, None) == -1
    bad = q.make_cfg(160, 128, 16, 4)
    assert L.coli_moe_layer_noalloc(C.byref(bad), C.byref(w), p, 4, p, None, None, None) == -2
