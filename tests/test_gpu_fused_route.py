"""The route of a one-token decode batch is selected inside the gate/up GEMV.

For T = 1 (decode logits kernel, E <= 512, the partials every workgroup reads at most
64 KiB) coli_moe_layer launches no selection kernel: every gate/up GEMV workgroup sums
the logit partials and selects the route with select_kernel's own device code
(sel_block), and one workgroup stores ids and weights for the down GEMV and the
combine. Larger batches take select_kernel. Either way the route the layer returns
must equal coli_moe_route's bit for bit (ids and fp32 weights), the layer output must
equal that of coli_moe_ffn run on that route and its grouping (GEMVs that read the
route) bit for bit, and both must match the oracle.
"""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3
MX = synth.W_MXFP4


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
    base = dict(hidden=256, ffn=128, n_experts=64, top_k=8, n_group=1, topk_group=1, rsf=2.5, has_shared=False,
                wbits=4, scale_group=0, topp=0.0)
    base.update(kw)
    return base


FUSED_CASES = [  # cfg kwargs, T
    (_cfg(hidden=2048, ffn=256), 1),                                   # OLMoE-scale router
    (_cfg(hidden=2048, ffn=256, has_shared=True), 1),
    (_cfg(hidden=512, n_group=8, topk_group=3, top_k=6, has_shared=True, wbits=8), 1),
    (_cfg(n_experts=128, n_group=4, topk_group=2, has_shared=True, wbits=2), 1),
    (_cfg(n_experts=128, n_group=64, topk_group=10, top_k=12), 1),    # one expert per group
    (_cfg(hidden=6144, ffn=256, n_experts=256, n_group=8, topk_group=4, has_shared=True), 1),  # GLM-scale router
    (_cfg(n_experts=256, n_group=8, topk_group=4, has_shared=True, topp=0.7), 1),                # top-p
    (_cfg(n_experts=256, top_k=64), 1),                               # k = 64
    (_cfg(n_experts=512, n_group=8, topk_group=4, has_shared=True), 1),  # two experts per thread
    (_cfg(hidden=512, n_experts=512, n_group=64, topk_group=16, top_k=16), 1),
    (_cfg(n_experts=24, n_group=8, topk_group=3, top_k=5, has_shared=True), 1),  # E not a power of two
    (_cfg(hidden=2048, ffn=256, scale_group=64), 1),                  # gs64 int4
    (_cfg(hidden=2048, ffn=256, has_shared=True, wbits=MX, scale_group=32), 1),  # MXFP4
    # selection kernel (T > 1)
    (_cfg(hidden=2048, ffn=256, has_shared=True), 4),
    (_cfg(n_experts=256, n_group=8, topk_group=4, has_shared=True, topp=0.7), 4),
    (_cfg(n_experts=512, n_group=8, topk_group=4, has_shared=True), 2),
    (_cfg(hidden=2048, ffn=256), 16),
]


def _inputs(cfgd, T, seed):
    return synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                              n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=cfgd["wbits"],
                              scale_group=cfgd["scale_group"])


@pytest.mark.parametrize("cfgd,T", FUSED_CASES)
def test_fused_route_equals_route_entry_and_unfused_ffn(q, orc, cfgd, T):
    import torch
    inp = _inputs(cfgd, T, 900 + T + cfgd["n_experts"] + cfgd["top_k"])
    w = gu.upload_layer(inp)
    cfg = q.make_cfg(**cfgd)
    d = gu.dev()
    k = cfgd["top_k"]
    x = gu.to_dev(inp["x"])
    # the layer (route selected inside the gate/up GEMV)
    out, idx, tw = gu.run_layer(cfgd, w, inp["x"])
    # the route entry point (selection kernel), then the FFN entry point on that route
    ridx = torch.empty((T, k), dtype=torch.int32, device=d)
    rtw = torch.empty((T, k), dtype=torch.float32, device=d)
    ws = q.alloc_workspace(cfg, T, d)
    q.route(cfg, w, x, ridx, rtw, ws)
    E = cfgd["n_experts"]
    cnt = torch.empty(E, dtype=torch.int32, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    perm = torch.empty(T * k, dtype=torch.int32, device=d)
    act = torch.empty(E, dtype=torch.int32, device=d)
    na = torch.empty(1, dtype=torch.int32, device=d)
    q.group(cfg, ridx, T, cnt, off, perm, act, na)
    out2 = torch.empty((T, cfgd["hidden"]), dtype=torch.float32, device=d)
    q.ffn(cfg, w, x, ridx, rtw, off, perm, act, na, out2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx, ridx.cpu().numpy())
    assert np.array_equal(tw.view(np.uint32), rtw.cpu().numpy().view(np.uint32))
    assert np.array_equal(out.view(np.uint32), out2.cpu().numpy().view(np.uint32))
    # and the oracle
    ref, oidx, ow = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.array_equal(idx, oidx)
    assert gu.ulp_diff_f32(tw, ow).max() <= 1
    assert gu.rel_err_per_token(out, ref).max() <= TOL
    if cfgd["topp"] > 0:
        assert (idx < 0).any()  # the top-p cut removed slots in this batch


@pytest.mark.parametrize("T", [1, 4])
def test_fused_route_ties_lowest_index(q, orc, T):
    """Exact ties in the selection (inside the GEMV at T = 1, the kernel at T = 4):
    identical router rows with equal bias, inside one group and across groups, and two
    identical groups; the lower index wins."""
    cfgd = _cfg(n_experts=128, n_group=4, topk_group=2, has_shared=True)
    inp = _inputs(cfgd, T, 78)
    rw, rb = inp["router_w"], inp["router_bias"]
    rb[:] = 0.0
    for e in (5, 17, 70):
        rw[e] = rw[2]
    rw[96:128] = rw[32:64]
    w = gu.upload_layer(inp)
    out, idx, tw = gu.run_layer(cfgd, w, inp["x"])
    ref, oidx, ow = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.array_equal(idx, oidx)
    assert gu.ulp_diff_f32(tw, ow).max() <= 1
    assert gu.rel_err_per_token(out, ref).max() <= TOL


def test_fused_route_batch_invariant_and_repeatable(q):
    """Token t's output and route do not depend on the other tokens of the batch, and two
    calls give the same bits (each token alone, selected inside the GEMV, against the
    batch of four, selected by the kernel)."""
    cfgd = _cfg(hidden=2048, ffn=256, has_shared=True)
    inp = _inputs(cfgd, 4, 55)
    w = gu.upload_layer(inp)
    out4, idx4, tw4 = gu.run_layer(cfgd, w, inp["x"])
    out4b, idx4b, tw4b = gu.run_layer(cfgd, w, inp["x"])
    assert np.array_equal(out4.view(np.uint32), out4b.view(np.uint32))
    for t in range(4):
        out1, idx1, tw1 = gu.run_layer(cfgd, w, inp["x"][t:t + 1])
        assert np.array_equal(idx1[0], idx4[t])
        assert np.array_equal(tw1[0].view(np.uint32), tw4[t].view(np.uint32))
        assert np.array_equal(out1[0].view(np.uint32), out4[t].view(np.uint32))


@pytest.mark.parametrize("T", [1, 4])
def test_profiled_layer_matches_layer(q, T):
    """coli_moe_layer_profiled runs the same launches as coli_moe_layer, with events
    between the stages (with one token the selection inside the gate/up GEMV): same
    output bits, and every stage's events complete."""
    import torch
    cfgd = _cfg(hidden=2048, ffn=256, has_shared=True)
    inp = _inputs(cfgd, T, 61 + T)
    w = gu.upload_layer(inp)
    out, _, _ = gu.run_layer(cfgd, w, inp["x"])
    cfg = q.make_cfg(**cfgd)
    d = gu.dev()
    x = gu.to_dev(inp["x"])
    out2 = torch.empty((T, cfgd["hidden"]), dtype=torch.float32, device=d)
    ns = q.num_stages()
    names = [q.stage_name(i) for i in range(ns)]
    ev = q.TimingEvents(ns + 1)
    stream = torch.cuda.current_stream(d)
    q.layer_profiled(cfg, w, x, out2, q.alloc_workspace(cfg, T, d), ev, stream=stream)
    stream.synchronize()
    assert np.array_equal(out.view(np.uint32), out2.cpu().numpy().view(np.uint32))
    for i in range(ns):
        assert ev.elapsed_ms(i, i + 1) >= 0.0, names[i]
    ev.close()
