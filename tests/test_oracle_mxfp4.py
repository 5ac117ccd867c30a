"""Pins of the oracle's MXFP4 expert weights (CPU only).

The pages name MXFP4 experts (JustVugg/colibri README, "Other supported models") without
spelling out the format; the oracle takes the OCP Microscaling (MX) v1.0 encodings: blocks
of 32 E2M1 codes sharing one E8M0 power-of-two scale. Pinned here against that
specification's value table, against a dense float64 product of independently decoded
weights, and against the already pinned int8 container, which an MXFP4 expert with unit
scales reduces to exactly.
"""
import math

import numpy as np
import pytest

import refmath
import synth

MX = synth.W_MXFP4


def test_e2m1_code_points_match_the_specification_table(oracle_lib):
    for c in range(16):
        v = oracle_lib.e2m1(c)
        assert v == refmath.E2M1_VALUES[c]
        assert math.copysign(1.0, v) == math.copysign(1.0, refmath.E2M1_VALUES[c])


def test_e8m0_is_a_bare_power_of_two(oracle_lib):
    assert oracle_lib.e8m0(127) == 1.0
    assert oracle_lib.e8m0(128) == 2.0
    assert oracle_lib.e8m0(0) == 2.0 ** -127
    assert oracle_lib.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle_lib.e8m0(255))


def test_mxfp4_decode_layout_matches_table_lookup(oracle_lib):
    rng = np.random.default_rng(5)
    b = rng.integers(0, 256, size=16 * 12, dtype=np.uint8)
    v = oracle_lib.mxfp4_decode(b, 32 * 12)
    assert np.array_equal(v, refmath.mxfp4_values_np(b, 32 * 12))
    # byte j of a block: code j in the low nibble, code j + 16 in the high one
    one = np.zeros(16, np.uint8)
    one[3] = 0x72  # code 2 (1.0) at position 3, code 7 (6.0) at position 19
    v = oracle_lib.mxfp4_decode(one, 32)
    assert v[3] == 1.0 and v[19] == 6.0 and np.count_nonzero(v) == 2


def test_expert_ffn_mxfp4_vs_dense_double(oracle_lib):
    """Per-block dots scaled by the activation scale and the E8M0 block scale equal a
    dense float64 product of the decoded weights."""
    H, F = 192, 128
    inp = synth.layer_inputs(82, 0, tokens=4, hidden=H, ffn=F, n_experts=2, has_shared=False, wbits=MX,
                             scale_group=32)
    assert inp["scales"].dtype == np.uint8 and inp["scales"].shape == (2, 3 * F * H // 32)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for e in range(2):
        blob, sc = inp["blobs"][e], inp["scales"][e]
        Wg, Wu, Wd = refmath.dequant_expert_mxfp4(blob, sc, H, F)
        for t in range(4):
            r = oracle_lib.expert_ffn(H, F, MX, blob, sc, xq[t], xd[t], scale_group=32)
            xhat = refmath.dequant_q8(xq[t], xd[t])
            g, u = Wg @ xhat, Wu @ xhat
            assert np.allclose(r["g"], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
            assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
            h = (refmath.silu(r["g"]) * r["u"]).astype(np.float32)
            assert np.array_equal(r["h"], h)
            y = Wd @ refmath.dequant_q8(r["hq"], r["hd"])
            assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def _as_int8_container(blob, H, F):
    """The int8 blob whose values are twice the E2M1 values (integers in [-12, 12])."""
    rh, rf = H // 2, F // 2
    parts = [(blob[: F * rh], F * H), (blob[F * rh: 2 * F * rh], F * H), (blob[2 * F * rh:], H * F)]
    return np.concatenate([(2.0 * refmath.mxfp4_values_np(p, n)).astype(np.int8).view(np.uint8) for p, n in parts])


def test_mxfp4_with_unit_scales_is_the_int8_container(oracle_lib):
    """E8M0 bytes of 127 (scale 1): every intermediate equals that of the int8 expert with
    values 2 e2m1(code) and row scales 1/2, bit for bit (both are exact rescalings by
    powers of two)."""
    H, F = 128, 96
    inp = synth.layer_inputs(83, 0, tokens=3, hidden=H, ffn=F, n_experts=1, has_shared=False, wbits=MX,
                             scale_group=32)
    blob = inp["blobs"][0]
    u1 = np.full(3 * F * H // 32, 127, np.uint8)
    b8 = _as_int8_container(blob, H, F)
    s8 = np.full(2 * F + H, 0.5, np.float32)
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for t in range(3):
        a = oracle_lib.expert_ffn(H, F, MX, blob, u1, xq[t], xd[t], scale_group=32)
        b = oracle_lib.expert_ffn(H, F, 8, b8, s8, xq[t], xd[t])
        for key in ("g", "u", "h", "hq", "hd", "y"):
            assert np.array_equal(a[key], b[key]), key


def test_layer_mxfp4_unit_scales_equal_int8_layer(oracle_lib):
    H, F, E = 128, 64, 5
    inp = synth.layer_inputs(84, 0, tokens=7, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=MX,
                             scale_group=32)
    ne = E + 1
    u1 = np.full((ne, 3 * F * H // 32), 127, np.uint8)
    b8 = np.stack([_as_int8_container(inp["blobs"][e], H, F) for e in range(ne)])
    s8 = np.full((ne, 2 * F + H), 0.5, np.float32)
    kw = dict(hidden=H, ffn=F, n_experts=E, top_k=2, rsf=1.5, has_shared=True)
    a, ia, wa = oracle_lib.layer(oracle_lib.make_cfg(**kw, wbits=MX, scale_group=32), inp["blobs"], u1,
                                 inp["router_w"], inp["router_bias"], inp["x"])
    b, ib, wb = oracle_lib.layer(oracle_lib.make_cfg(**kw, wbits=8), b8, s8, inp["router_w"], inp["router_bias"],
                                 inp["x"])
    assert np.array_equal(ia, ib) and np.array_equal(wa, wb)
    assert np.array_equal(a, b)


def test_layer_mxfp4_is_weighted_sum_of_its_experts(oracle_lib):
    """Each expert reads its own E8M0 slice (byte stride per expert)."""
    H, F, E, k = 128, 64, 6, 3
    inp = synth.layer_inputs(85, 0, tokens=5, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=MX,
                             scale_group=32)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=F, n_experts=E, top_k=k, rsf=2.0, has_shared=True, wbits=MX,
                              scale_group=32)
    out, idx, w = oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
    xq, xd = oracle_lib.quantize_q8_0(inp["x"])
    for t in range(5):
        acc = np.zeros(H, np.float64)
        for j in range(k):
            e = idx[t, j]
            r = oracle_lib.expert_ffn(H, F, MX, inp["blobs"][e], inp["scales"][e], xq[t], xd[t], scale_group=32)
            acc += float(w[t, j]) * r["y"]
        r = oracle_lib.expert_ffn(H, F, MX, inp["blobs"][E], inp["scales"][E], xq[t], xd[t], scale_group=32)
        acc += r["y"]
        assert np.array_equal(out[t], acc.astype(np.float32))


def test_mxfp4_scale_group_is_32_only(oracle_lib):
    inp = synth.layer_inputs(86, 0, tokens=2, hidden=128, ffn=64, n_experts=2, has_shared=False, wbits=MX,
                             scale_group=32)
    for wb, gs in ((MX, 0), (MX, 64), (4, 32)):
        cfg = oracle_lib.make_cfg(hidden=128, ffn=64, n_experts=2, top_k=1, wbits=wb, scale_group=gs)
        with pytest.raises(ValueError):
            oracle_lib.layer(cfg, inp["blobs"], inp["scales"], inp["router_w"], inp["router_bias"], inp["x"])
