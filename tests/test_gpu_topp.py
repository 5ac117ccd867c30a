"""Adaptive expert top-p (the --topp knob of the colibri-strix README, "Experimental resident
CUDA backend", useful-knobs paragraph) on the HIP
path against the oracle: the route with its empty slots (index -1, weight 0)
bit-exact, the grouping of a route with empty slots bit-exact, and the layer and the
FFN entry point within the parity bar, at decode sizes and past 512 pairs.
"""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_sigmoid_amd as q
    q.lib()
    return q


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


def _cfg(**kw):
    base = dict(hidden=256, ffn=128, n_experts=16, top_k=4, n_group=1, topk_group=1, rsf=1.0, has_shared=False,
                wbits=4, topp=0.7)
    base.update(kw)
    return base


ROUTE_CASES = [  # cfg kwargs, T
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 16),
    (_cfg(hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8, topk_group=4, rsf=2.5), 4),
    (_cfg(hidden=512, n_experts=40, top_k=6, n_group=5, topk_group=2, rsf=1.5, topp=0.5), 70),
    (_cfg(hidden=384, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, topp=0.3), 37),
]


def _route_inputs(cfgd, T, seed):
    # a wider router weight spreads the scores, so that top-p drops slots
    x = synth.activations(seed, 0, T, cfgd["hidden"])
    W = synth.router_weight(seed, 0, cfgd["n_experts"], cfgd["hidden"], std=0.05)
    b = synth.router_bias(seed, 0, cfgd["n_experts"])
    return x, W, b


@pytest.mark.parametrize("cfgd,T", ROUTE_CASES)
def test_route_topp_bitexact(q, orc, cfgd, T):
    import torch
    x, W, b = _route_inputs(cfgd, T, 900 + T)
    w = q.Weights(experts=None, scales=None, router_w=gu.to_dev(W), router_bias=gu.to_dev(b))
    cfg = q.make_cfg(**cfgd)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=gu.dev())
    tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=gu.dev())
    q.route(cfg, w, gu.to_dev(x), idx, tw, q.alloc_workspace(cfg, T, gu.dev()))
    torch.cuda.synchronize()
    ridx, rw = orc.route(orc.make_cfg(**cfgd), W, b, x)
    assert np.any(ridx == -1)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    twn = tw.cpu().numpy()
    assert np.all(twn[ridx == -1] == 0.0)
    assert gu.ulp_diff_f32(twn, rw).max() <= 1


@pytest.mark.parametrize("E,k,T", [(16, 4, 9), (64, 8, 300), (256, 8, 2048)])
def test_group_with_empty_slots_bitexact(q, orc, E, k, T):
    import torch
    rng = np.random.default_rng(E + T)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    keep = rng.integers(1, k + 1, size=T)
    for t in range(T):
        idx[t, keep[t]:] = -1
    cfgd = _cfg(n_experts=E, top_k=k)
    cfg = q.make_cfg(**cfgd)
    d = gu.dev()
    cnt = torch.empty(E, dtype=torch.int32, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    perm = torch.full((T * k,), -7, dtype=torch.int32, device=d)
    act = torch.empty(E, dtype=torch.int32, device=d)
    na = torch.empty(1, dtype=torch.int32, device=d)
    q.group(cfg, gu.to_dev(idx), T, cnt, off, perm, act, na)
    torch.cuda.synchronize()
    rc, ro, rp, ra = orc.group(orc.make_cfg(**cfgd), idx)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(off.cpu().numpy(), ro)
    nvalid = int(ro[-1])
    assert nvalid == int((idx >= 0).sum())
    assert np.array_equal(perm.cpu().numpy()[:nvalid], rp)
    assert int(na.item()) == ra.size
    assert np.array_equal(act.cpu().numpy()[: ra.size], ra)


LAYER_CASES = [  # cfg kwargs, T, seed
    (_cfg(), 8, 61),
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 16, 62),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          topp=0.5), 37, 63),
    # past 512 pairs (grouped GEMMs), formats and a group-scaled layer
    # (F = 1024: at F = 256 one Q8_0 flip of an h code, where the GPU's fp32 sum and the
    # oracle's fp64 sum straddle a rounding boundary, moves a token by up to ~6e-4)
    (_cfg(hidden=384, ffn=1024, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          topp=0.5), 131, 64),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, has_shared=True, wbits=8), 117, 65),
    (_cfg(hidden=512, ffn=256, n_experts=16, top_k=8, wbits=2, scale_group=64, topp=0.6), 90, 66),
    # MXFP4 weights, decode and grouped-GEMM sizes
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8, wbits=40, scale_group=32), 16, 67),
    (_cfg(hidden=512, ffn=1024, n_experts=16, top_k=8, wbits=40, scale_group=32, topp=0.6), 120, 68),
]


@pytest.mark.parametrize("cfgd,T,seed", LAYER_CASES)
def test_layer_topp_vs_oracle(q, orc, cfgd, T, seed):
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=cfgd["wbits"],
                             scale_group=cfgd.get("scale_group", 0))
    inp["router_w"] = synth.router_weight(seed, 0, cfgd["n_experts"], cfgd["hidden"], std=0.05)
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    ref, ridx, rw = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.any(ridx == -1)
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    err = gu.rel_err_per_token(out, ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("T", [21, 150])
def test_ffn_entry_with_empty_slots(q, orc, T):
    """coli_moe_ffn on the oracle's top-p route (grouped by coli_moe_group)."""
    import torch
    cfgd = _cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True)
    inp = synth.layer_inputs(71, 0, tokens=T, hidden=384, ffn=256, n_experts=24, has_shared=True, wbits=4)
    inp["router_w"] = synth.router_weight(71, 0, 24, 384, std=0.05)
    ocfg = orc.make_cfg(**cfgd)
    ridx, rw = orc.route(ocfg, inp["router_w"], inp["router_bias"], inp["x"])
    assert np.any(ridx == -1)
    ref = orc.ffn(ocfg, inp["blobs"], inp["scales"], inp["x"], ridx, rw)
    cfg = q.make_cfg(**cfgd)
    d = gu.dev()
    E, k = 24, 5
    cnt = torch.empty(E, dtype=torch.int32, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    perm = torch.empty(T * k, dtype=torch.int32, device=d)
    act = torch.empty(E, dtype=torch.int32, device=d)
    na = torch.empty(1, dtype=torch.int32, device=d)
    idx_d = gu.to_dev(ridx)
    q.group(cfg, idx_d, T, cnt, off, perm, act, na)
    out = torch.empty((T, 384), dtype=torch.float32, device=d)
    q.ffn(cfg, gu.upload_layer(inp), gu.to_dev(inp["x"]), idx_d, gu.to_dev(rw), off, perm, act, na, out,
          q.alloc_workspace(cfg, T, d))
    torch.cuda.synchronize()
    assert gu.rel_err_per_token(out.cpu().numpy(), ref).max() <= TOL
