"""Group-scaled weights (one fp32 scale per 64 inputs of a row, the gs64 int4
container of the JustVugg/colibri README, "2. Get the model") on the HIP path
against the oracle: decode-sized batches (GEMV kernels) and batches past 512 pairs
(grouped GEMMs), every weight format, with and without a shared expert. Bars as in
the parity tests; where every floating-point step is exact (unit scales, integer
activations with a +-127 per block) the output is bit-identical.
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
                wbits=4, scale_group=64)
    base.update(kw)
    return base


CASES = [  # cfg kwargs, T, seed
    (_cfg(), 8, 41),
    (_cfg(wbits=8), 8, 42),
    (_cfg(wbits=2), 8, 43),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 37, 44),
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 16, 45),
    (_cfg(hidden=640, ffn=384, n_experts=12, top_k=2, has_shared=True), 1, 46),
    # past 512 pairs: grouped GEMMs
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 131, 47),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=8), 117, 48),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=2), 109, 49),
    (_cfg(hidden=512, ffn=256, n_experts=8, top_k=2, has_shared=True), 300, 50),
]


@pytest.mark.parametrize("cfgd,T,seed", CASES)
def test_group_scaled_layer_vs_oracle(q, orc, cfgd, T, seed):
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=cfgd["wbits"],
                             scale_group=64)
    assert inp["scales"].shape[1] == q.scales_per_expert(q.make_cfg(**cfgd))
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    ref, ridx, rw = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    err = gu.rel_err_per_token(out, ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("wbits,T", [(4, 11), (8, 11), (2, 11), (4, 530), (8, 530), (2, 530)])
def test_group_scaled_exact_case_bitidentical(q, orc, wbits, T):
    """Unit group scales with integer activations (Q8_0 scale exactly 1) and
    selection-structured weights: every floating-point step is exact."""
    from test_gpu_parity import _exact_inputs
    H, F, E = 256, 128, 6
    x, blobs, _ = _exact_inputs(H, F, E, wbits, T, 700 + wbits)
    scales = np.ones((E, 3 * F * H // 64), np.float32)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0, wbits=wbits)
    rw = synth.router_weight(3, 0, E, H, std=0.001)
    rb = synth.router_bias(3, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, _ = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_group_scales_differ_from_row_scales(q, orc):
    """The group scales reach the kernels: scaling one 64-input group of every row
    changes the GPU output exactly as it changes the oracle's."""
    cfgd = _cfg(hidden=256, ffn=128, n_experts=4, top_k=2, has_shared=True)
    inp = synth.layer_inputs(51, 0, tokens=6, hidden=256, ffn=128, n_experts=4, has_shared=True, wbits=4,
                             scale_group=64)
    sc = inp["scales"].copy()
    sc[:, 1::4] *= 3.0   # group 1 of every gate/up row (4 groups per row of 256 inputs)
    inp2 = dict(inp, scales=sc)
    a, _, _ = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    b, _, _ = gu.run_layer(cfgd, gu.upload_layer(inp2), inp["x"])
    rb, _, _ = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], sc, inp["router_w"], inp["router_bias"], inp["x"])
    assert not np.array_equal(a, b)
    assert gu.rel_err_per_token(b, rb).max() <= TOL
