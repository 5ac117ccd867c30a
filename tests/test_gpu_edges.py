"""Edge cases of the HIP path against the oracle.

The empty batch; the degenerate router settings of the group-limited sigmoid
router (a single expert, one expert per group, k equal to every eligible expert,
k = E); the largest expert count, group count and top-k the boundary accepts; and
the largest batch (T * k = 65535 pairs), checked on a sample of tokens that the
oracle computes one by one (tokens are independent, so the oracle's layer over the
sampled rows is the reference for those rows). Each case runs once at a decode
size (route-local grouping, GEMV kernels) and once past 512 pairs (grouping kernel,
grouped GEMMs). Bars as in the parity tests: indices bit-exact, weights within one
fp32 ulp, outputs within the per-token normwise relative error 1e-3.
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
                wbits=4)
    base.update(kw)
    return base


def _check_layer(orc, cfgd, T, seed, sample=None):
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=cfgd["wbits"])
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    rows = np.arange(T) if sample is None else np.asarray(sample)
    ref, ridx, rw = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], np.ascontiguousarray(inp["x"][rows]))
    assert np.array_equal(idx[rows], ridx)
    assert gu.ulp_diff_f32(tw[rows], rw).max() <= 1
    err = gu.rel_err_per_token(out[rows], ref)
    assert err.max() <= TOL, err.max()
    return idx, tw


def test_empty_batch_is_a_noop(q):
    """T = 0: every entry point returns success and writes nothing."""
    import torch
    cfgd = _cfg(has_shared=True, n_group=2, topk_group=1)
    cfg = q.make_cfg(**cfgd)
    inp = synth.layer_inputs(5, 0, tokens=1, hidden=256, ffn=128, n_experts=16, has_shared=True, wbits=4)
    w = gu.upload_layer(inp)
    d = gu.dev()
    x = torch.empty((0, 256), dtype=torch.float32, device=d)
    out = torch.full((4, 256), float("nan"), dtype=torch.float32, device=d)
    idx = torch.full((4, 4), -7, dtype=torch.int32, device=d)
    tw = torch.full((4, 4), float("nan"), dtype=torch.float32, device=d)
    ws = q.alloc_workspace(cfg, 1, d)
    q.layer(cfg, w, x, out[:0], ws, idx[:0], tw[:0])
    q.route(cfg, w, x, idx[:0], tw[:0], ws)
    cnt = torch.full((16,), -7, dtype=torch.int32, device=d)
    off = torch.full((17,), -7, dtype=torch.int32, device=d)
    act = torch.full((16,), -7, dtype=torch.int32, device=d)
    na = torch.full((1,), -7, dtype=torch.int32, device=d)
    perm = torch.full((4,), -7, dtype=torch.int32, device=d)
    q.group(cfg, idx[:0], 0, cnt, off, perm[:0], act, na)
    q.ffn(cfg, w, x, idx[:0], tw[:0], off, perm[:0], act, na, out[:0], ws)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(tw).all()
    for t in (idx, cnt, off, act, na, perm):
        assert (t == -7).all()


DEGENERATE = [  # cfg kwargs, (decode T, T past 512 pairs)
    # a single routed expert: every token takes it with weight rsf
    (_cfg(n_experts=1, top_k=1, rsf=2.5), (5, 600)),
    (_cfg(n_experts=1, top_k=1, rsf=2.5, has_shared=True), (7, 300)),
    # one expert per group: the group score is that expert's corrected score
    (_cfg(n_experts=8, top_k=3, n_group=8, topk_group=3, rsf=2.5, has_shared=True), (9, 200)),
    # k equal to every expert of the kept groups
    (_cfg(n_experts=16, top_k=8, n_group=4, topk_group=2, rsf=1.5), (6, 70)),
    # k = E: every expert, ordered by corrected score
    (_cfg(n_experts=8, top_k=8), (3, 80)),
]


@pytest.mark.parametrize("cfgd,Ts", DEGENERATE)
def test_degenerate_router_settings(q, orc, cfgd, Ts):
    for i, T in enumerate(Ts):
        idx, tw = _check_layer(orc, cfgd, T, 300 + 17 * i + cfgd["n_experts"])
        if cfgd["n_experts"] == 1:
            assert np.all(idx == 0) and np.all(tw == np.float32(cfgd["rsf"]))
        if cfgd["top_k"] == cfgd["n_experts"]:
            assert np.array_equal(np.sort(idx, axis=1), np.tile(np.arange(cfgd["n_experts"]), (T, 1)))


def test_largest_expert_group_and_topk_counts(q, orc):
    """E = 1024 experts in 64 groups, 8 kept, top-64 (the boundary's limits)."""
    cfgd = _cfg(hidden=128, ffn=128, n_experts=1024, top_k=64, n_group=64, topk_group=8, rsf=2.5, has_shared=True)
    for i, T in enumerate((4, 20)):   # 256 pairs (decode path), 1280 pairs (grouped GEMMs)
        _check_layer(orc, cfgd, T, 500 + i)


def test_largest_batch_sampled(q, orc):
    """T * k = 65535 pairs, the most the boundary accepts; 48 sampled tokens incl. the first and last."""
    cfgd = _cfg(hidden=128, ffn=128, n_experts=64, top_k=5, has_shared=True)
    T = 65535 // 5
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))
    _check_layer(orc, cfgd, T, 600, sample)
