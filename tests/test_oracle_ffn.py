"""Pins of the oracle's quantised expert FFN, combine and layer (CPU only)."""
import math

import numpy as np
import pytest

import refmath
import synth


def _small(wbits, H=128, F=64, E=6, has_shared=True, seed=77):
    inp = synth.layer_inputs(seed, 0, tokens=5, hidden=H, ffn=F, n_experts=E, has_shared=has_shared,
                             wbits=wbits)
    return inp


@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_expert_ffn_vs_dense_double(oracle_lib, wbits):
    """Per-block integer dots with per-block activation scales and per-row weight
    scales equal a dense float64 product of the dequantised operands."""
    H, F = 192, 96
    inp = _small(wbits, H, F, E=3)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for e in range(3):
        blob, sc = inp["blobs"][e], inp["scales"][e]
        Wg, Wu, Wd = refmath.dequant_expert(blob, sc, H, F, wbits)
        for t in range(inp["x"].shape[0]):
            r = oracle_lib.expert_ffn(H, F, wbits, blob, sc, xq[t], xd[t])
            xhat = refmath.dequant_q8(xq[t], xd[t])
            g = Wg @ xhat
            u = Wu @ xhat
            assert np.allclose(r["g"], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
            assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
            h = (refmath.silu(r["g"]) * r["u"]).astype(np.float32)
            assert np.array_equal(r["h"], h)
            hq, hd = oracle_lib.quantize_q8_0(h[None, :])
            assert np.array_equal(r["hq"], hq[0]) and np.array_equal(r["hd"], hd[0])
            y = Wd @ refmath.dequant_q8(r["hq"], r["hd"])
            assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_expert_ffn_selection_matrix_closed_form(oracle_lib):
    """int8 weights that select one input per row with scale 1: g_f = u_f = x^_f,
    h_f = silu(x^_f) x^_f, y_r = h^_r for r < F and 0 above (x^, h^ dequantised)."""
    H, F = 128, 64
    rh = H  # int8
    gate = np.zeros((F, H), np.int8)
    gate[np.arange(F), np.arange(F)] = 1
    down = np.zeros((H, F), np.int8)
    down[np.arange(F), np.arange(F)] = 1
    blob = np.concatenate([gate.view(np.uint8).ravel(), gate.view(np.uint8).ravel(),
                           down.view(np.uint8).ravel()])
    assert blob.size == 2 * F * rh + H * F
    scales = np.ones(2 * F + H, np.float32)
    x = synth.activations(21, 0, 1, H)[0]
    xq, xd = oracle_lib.quantize_q8_0(x[None, :])
    r = oracle_lib.expert_ffn(H, F, 8, blob, scales, xq[0], xd[0])
    xhat = np.array([float(xd[0, i // 32]) * int(xq[0, i]) for i in range(H)])
    for f in range(F):
        assert r["g"][f] == xhat[f] and r["u"][f] == xhat[f]
        want = xhat[f] / (1.0 + math.exp(-xhat[f])) * xhat[f]
        assert r["h"][f] == np.float32(want)
    hhat = [float(r["hd"][i // 32]) * int(r["hq"][i]) for i in range(F)]
    assert r["y"][:F].tolist() == hhat
    assert np.all(r["y"][F:] == 0.0)


@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_layer_single_expert_is_scaled_ffn(oracle_lib, wbits):
    """E = 1, k = 1: the router weight is s/s * rsf = rsf, so out = rsf * FFN(x)."""
    H, F = 128, 64
    rsf = 2.5
    inp = synth.layer_inputs(5, 0, tokens=4, hidden=H, ffn=F, n_experts=1, has_shared=False, wbits=wbits)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=F, n_experts=1, top_k=1, rsf=rsf, wbits=wbits)
    out, idx, w = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    assert np.all(idx == 0) and np.all(w == np.float32(rsf))
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for t in range(4):
        y = oracle_lib.expert_ffn(H, F, wbits, inp["blobs"][0], inp["scales"][0], xq[t], xd[t])["y"]
        assert np.array_equal(out[t], (rsf * y).astype(np.float32))


def test_layer_zero_input_gives_zero(oracle_lib):
    H, F, E = 128, 64, 8
    inp = synth.layer_inputs(6, 0, tokens=3, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=4)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=F, n_experts=E, top_k=2, n_group=2, topk_group=1, rsf=2.5,
                              has_shared=True, wbits=4)
    out, _, _ = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"],
                                 np.zeros((3, H), np.float32))
    assert np.all(out == 0.0)


@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_layer_equals_batch_union_evaluation(oracle_lib, wbits):
    """The per-token oracle equals an evaluation in batch-union order (each distinct
    expert once over its grouped pairs, then the slot-order combine), bit for bit."""
    H, F, E, k, T = 128, 64, 16, 4, 9
    inp = synth.layer_inputs(8, 0, tokens=T, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=wbits)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=F, n_experts=E, top_k=k, n_group=4, topk_group=2, rsf=2.5,
                              has_shared=True, wbits=wbits)
    out, idx, w = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    cnt, off, perm, active = oracle_lib.group(cfg, idx)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    ypair = np.zeros((T * k, H), np.float64)
    for e in active:
        for p in perm[off[e]:off[e + 1]]:
            t = p // k
            ypair[p] = oracle_lib.expert_ffn(H, F, wbits, inp["blobs"][e], inp["scales"][e], xq[t], xd[t])["y"]
    ysh = np.stack([oracle_lib.expert_ffn(H, F, wbits, inp["blobs"][E], inp["scales"][E], xq[t], xd[t])["y"]
                    for t in range(T)])
    ref = np.zeros((T, H), np.float64)
    for t in range(T):
        acc = np.zeros(H, np.float64)
        for j in range(k):
            acc = acc + np.float64(w[t, j]) * ypair[t * k + j]
        ref[t] = acc + ysh[t]
    assert np.array_equal(out, ref.astype(np.float32))


def test_layer_thread_count_invariant(oracle_lib):
    H, F, E = 256, 128, 16
    inp = synth.layer_inputs(synth.workload_seed(0), 0, tokens=8, hidden=H, ffn=F, n_experts=E,
                             has_shared=False, wbits=4)
    cfg = oracle_lib.make_cfg(**synth.WORKLOADS[0])
    n0 = oracle_lib.threads()
    try:
        oracle_lib.set_threads(1)
        a = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
        oracle_lib.set_threads(max(2, n0))
        b = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    finally:
        oracle_lib.set_threads(n0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_layer_ffn_matches_route_then_ffn(oracle_lib):
    w0 = synth.WORKLOADS[0]
    inp = synth.layer_inputs(synth.workload_seed(0), 0, tokens=8, hidden=w0["hidden"], ffn=w0["ffn"],
                             n_experts=w0["n_experts"], has_shared=False, wbits=4)
    cfg = oracle_lib.make_cfg(**w0)
    out, idx, w = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    idx2, w2 = oracle_lib.route(cfg, inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    assert np.array_equal(out, oracle_lib.ffn(cfg, inp["blobs"], inp["scales"], inp["x"], idx, w))


@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_expert_ffn_group_scales_vs_dense_double(oracle_lib, wbits):
    """One scale per 64 inputs of a row (the gs64 container): the per-block integer
    dots scaled by block and group scales equal a dense float64 product of the
    dequantised operands, s[row][i // 64] * q[row][i]."""
    H, F = 192, 128
    inp = synth.layer_inputs(78, 0, tokens=4, hidden=H, ffn=F, n_experts=2, has_shared=False, wbits=wbits,
                             scale_group=64)
    assert inp["scales"].shape == (2, 3 * F * H // 64)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for e in range(2):
        blob, sc = inp["blobs"][e], inp["scales"][e]
        Wg, Wu, Wd = refmath.dequant_expert(blob, sc, H, F, wbits, scale_group=64)
        for t in range(4):
            r = oracle_lib.expert_ffn(H, F, wbits, blob, sc, xq[t], xd[t], scale_group=64)
            xhat = refmath.dequant_q8(xq[t], xd[t])
            g, u = Wg @ xhat, Wu @ xhat
            assert np.allclose(r["g"], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
            assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
            y = Wd @ refmath.dequant_q8(r["hq"], r["hd"])
            assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_group_scales_equal_to_row_scale_reduce_to_per_row(oracle_lib):
    """Group scales that repeat each row's scale give the per-row expert."""
    H, F = 128, 64
    inp = synth.layer_inputs(79, 0, tokens=3, hidden=H, ffn=F, n_experts=1, has_shared=False, wbits=4)
    blob, sr = inp["blobs"][0], inp["scales"][0]
    sg = np.concatenate([np.repeat(sr[:F], H // 64), np.repeat(sr[F:2 * F], H // 64), np.repeat(sr[2 * F:], F // 64)])
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for t in range(3):
        a = oracle_lib.expert_ffn(H, F, 4, blob, sr, xq[t], xd[t])
        b = oracle_lib.expert_ffn(H, F, 4, blob, sg, xq[t], xd[t], scale_group=64)
        for key in ("g", "u", "y"):
            assert np.allclose(a[key], b[key], rtol=1e-13, atol=1e-13 * np.abs(a[key]).max())


def test_layer_group_scales_rejects_bad_group(oracle_lib):
    """Only 0 (per row) and 64 are group sizes; 64 must divide H and F."""
    inp = synth.layer_inputs(80, 0, tokens=2, hidden=96, ffn=64, n_experts=2, has_shared=False, wbits=4)
    for gs, H in ((32, 128), (64, 96)):
        cfg = oracle_lib.make_cfg(hidden=H, ffn=64, n_experts=2, top_k=1, wbits=4, scale_group=gs)
        with pytest.raises(ValueError):
            oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])


def test_layer_topp_is_sum_over_kept_slots(oracle_lib):
    """With adaptive top-p the layer is the weighted sum over the kept slots only (plus the
    shared expert), each evaluated by the single-expert oracle."""
    H, F, E, k = 128, 64, 8, 4
    inp = synth.layer_inputs(81, 0, tokens=6, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=4)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=F, n_experts=E, top_k=k, rsf=2.0, has_shared=True, wbits=4, topp=0.6)
    out, idx, w = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    assert np.any(idx == -1)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for t in range(6):
        acc = np.zeros(H)
        for j in range(k):
            if idx[t, j] >= 0:
                acc += float(w[t, j]) * oracle_lib.expert_ffn(H, F, 4, inp["blobs"][idx[t, j]], inp["scales"][idx[t, j]],
                                                              xq[t], xd[t])["y"]
        acc += oracle_lib.expert_ffn(H, F, 4, inp["blobs"][E], inp["scales"][E], xq[t], xd[t])["y"]
        assert np.array_equal(out[t], acc.astype(np.float32))
