"""Parity of the HIP library with the CPU oracle, element by element, on seeded inputs.

Bars: Q8_0 codes and scales, router indices, the grouping and all integer work
bit-exact; router weights within 1 fp32 ulp; layer outputs within a per-token
normwise relative error of 1e-3 (max_r |out - ref| / max_r |ref|). Where every
floating-point step is exact (integer-valued activations with unit block scale,
selection-structured weights, k = 1) the layer output must be bit-identical,
which pins every per-block int32 dot of the gate, up and down kernels.
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


# ---------------------------------------------------------------- Q8_0
@pytest.mark.parametrize("rows,cols", [(1, 32), (8, 256), (37, 6144), (3, 2048)])
def test_q8_0_bitexact(q, orc, rows, cols):
    import torch
    rng = np.random.default_rng(rows * cols)
    x = (rng.standard_normal((rows, cols)) * rng.uniform(1e-3, 1e3, (rows, 1))).astype(np.float32)
    x[0, :32] = 0.0
    if cols >= 64:
        x[0, 32:64] = np.array([127, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5] * 4, np.float32)
    xd_ = gu.to_dev(x)
    qd = torch.empty((rows, cols), dtype=torch.int8, device=gu.dev())
    dd = torch.empty((rows, cols // 32), dtype=torch.float32, device=gu.dev())
    q.quantize_q8_0(xd_, qd, dd)
    torch.cuda.synchronize()
    rq, rd = orc.quantize_q8_0(x)
    assert np.array_equal(qd.cpu().numpy(), rq)
    assert np.array_equal(dd.cpu().numpy().view(np.uint32), rd.view(np.uint32))


# ---------------------------------------------------------------- router
ROUTE_CASES = [  # cfg kwargs, T
    (dict(_cfg()), 8),
    (dict(_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8)), 1),
    (dict(_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8)), 16),
    (dict(_cfg(hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8, topk_group=4, rsf=2.5)), 4),
    (dict(_cfg(hidden=384, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5)), 37),
    (dict(_cfg(hidden=512, n_experts=40, top_k=6, n_group=5, topk_group=2, rsf=1.5)), 70),
    (dict(_cfg(hidden=256, n_experts=8, top_k=3, n_group=8, topk_group=3)), 5),
]


@pytest.mark.parametrize("cfgd,T", ROUTE_CASES)
def test_route_bitexact(q, orc, cfgd, T):
    import torch
    seed = 99 + T + cfgd["n_experts"]
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=False, wbits=4, with_blobs=False)
    w = q.Weights(experts=None, scales=None, router_w=gu.to_dev(inp["router_w"]),
                  router_bias=gu.to_dev(inp["router_bias"]))
    cfg = q.make_cfg(**cfgd)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=gu.dev())
    tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=gu.dev())
    ws = q.alloc_workspace(cfg, T, gu.dev())
    q.route(cfg, w, gu.to_dev(inp["x"]), idx, tw, ws)
    torch.cuda.synchronize()
    ridx, rw = orc.route(orc.make_cfg(**cfgd), inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert gu.ulp_diff_f32(tw.cpu().numpy(), rw).max() <= 1


def test_route_prefill_zipf_bitexact(q, orc):
    """GLM-scale router at T = 2048 with the Zipf-skewed bias."""
    import torch
    cfgd = gu.workload_cfg(3)
    T = 2048
    inp = synth.layer_inputs(synth.workload_seed(3), 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=True, wbits=4, zipf=True, with_blobs=False)
    w = q.Weights(None, None, gu.to_dev(inp["router_w"]), gu.to_dev(inp["router_bias"]))
    cfg = q.make_cfg(**cfgd)
    idx = torch.empty((T, 8), dtype=torch.int32, device=gu.dev())
    tw = torch.empty((T, 8), dtype=torch.float32, device=gu.dev())
    ws = q.alloc_workspace(cfg, T, gu.dev())
    q.route(cfg, w, gu.to_dev(inp["x"]), idx, tw, ws)
    torch.cuda.synchronize()
    ridx, rw = orc.route(orc.make_cfg(**cfgd), inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert gu.ulp_diff_f32(tw.cpu().numpy(), rw).max() <= 1


def test_route_ties_lowest_index(q, orc):
    """Identical router rows and equal bias tie exactly: the lower index wins on both sides."""
    import torch
    cfgd = _cfg(hidden=256, n_experts=32, top_k=6, n_group=4, topk_group=2)
    T = 40
    inp = synth.layer_inputs(5, 0, tokens=T, hidden=256, ffn=128, n_experts=32, has_shared=False, wbits=4,
                             with_blobs=False)
    inp["router_w"][9] = inp["router_w"][2]
    inp["router_w"][30] = inp["router_w"][2]
    inp["router_bias"][:] = 0.0
    w = q.Weights(None, None, gu.to_dev(inp["router_w"]), gu.to_dev(inp["router_bias"]))
    cfg = q.make_cfg(**cfgd)
    idx = torch.empty((T, 6), dtype=torch.int32, device=gu.dev())
    tw = torch.empty((T, 6), dtype=torch.float32, device=gu.dev())
    q.route(cfg, w, gu.to_dev(inp["x"]), idx, tw, q.alloc_workspace(cfg, T, gu.dev()))
    torch.cuda.synchronize()
    ridx, _ = orc.route(orc.make_cfg(**cfgd), inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx.cpu().numpy(), ridx)


# Decode-sized batches (H a multiple of 256, x quantised by the logits kernel): the
# selection splits each expert's rank count over several threads when E < 256 (by the
# group size), places the candidates of the kept groups by group rank, and splits the
# candidates' rank counts too. Groups of one expert, of 8 to 256 experts, one group,
# k = 64 and E = 512 (two experts per thread), against the oracle.
WAVE_CASES = [  # E, G, Gk, k, T, topp
    (64, 1, 1, 8, 3, 0.0),        # one group
    (64, 64, 8, 4, 5, 0.0),       # one expert per group: the group score is c itself
    (64, 8, 3, 6, 16, 0.0),       # one expert per lane, 8 lanes per group
    (128, 4, 2, 8, 7, 0.0),       # two experts per lane, 16 lanes per group
    (128, 64, 10, 12, 2, 0.0),    # two experts per lane, one lane per group
    (128, 2, 1, 8, 4, 0.0),       # two experts per lane, 32 lanes per group
    (256, 8, 4, 8, 16, 0.0),      # GLM-scale router
    (256, 1, 1, 64, 4, 0.0),      # k = 64: every lane holds a slot
    (512, 8, 4, 8, 9, 0.0),       # eight experts per lane
    (512, 64, 16, 16, 1, 0.0),    # eight experts per lane, one lane per group
    (256, 8, 4, 8, 16, 0.7),      # adaptive top-p
]


def _route_both(q, orc, cfgd, inp, T):
    import torch
    w = q.Weights(None, None, gu.to_dev(inp["router_w"]), gu.to_dev(inp["router_bias"]))
    cfg = q.make_cfg(**cfgd)
    k = cfgd["top_k"]
    idx = torch.empty((T, k), dtype=torch.int32, device=gu.dev())
    tw = torch.empty((T, k), dtype=torch.float32, device=gu.dev())
    q.route(cfg, w, gu.to_dev(inp["x"]), idx, tw, q.alloc_workspace(cfg, T, gu.dev()))
    torch.cuda.synchronize()
    ridx, rw = orc.route(orc.make_cfg(**cfgd), inp["router_w"], inp["router_bias"], inp["x"])
    return idx.cpu().numpy(), tw.cpu().numpy(), ridx, rw


@pytest.mark.parametrize("E,G,Gk,k,T,topp", WAVE_CASES)
def test_route_decode_select_bitexact(q, orc, E, G, Gk, k, T, topp):
    cfgd = _cfg(hidden=256, n_experts=E, top_k=k, n_group=G, topk_group=Gk, rsf=2.5, topp=topp)
    inp = synth.layer_inputs(300 + E + G + k + T, 0, tokens=T, hidden=256, ffn=128, n_experts=E, has_shared=False,
                             wbits=4, with_blobs=False)
    idx, tw, ridx, rw = _route_both(q, orc, cfgd, inp, T)
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    if topp > 0:
        assert (ridx < 0).any()  # the top-p cut removed slots in this batch


def test_route_decode_select_ties(q, orc):
    """Exact ties at decode sizes: experts with identical router rows and equal bias,
    inside one group and across groups, and two groups identical as a whole (equal group
    scores): the lower index wins every tie, as in the oracle."""
    E, G = 128, 4
    cfgd = _cfg(hidden=256, n_experts=E, top_k=8, n_group=G, topk_group=2, rsf=2.5)
    T = 16
    inp = synth.layer_inputs(77, 0, tokens=T, hidden=256, ffn=128, n_experts=E, has_shared=False, wbits=4,
                             with_blobs=False)
    rw, rb = inp["router_w"], inp["router_bias"]
    rb[:] = 0.0
    for e in (5, 17, 70):
        rw[e] = rw[2]
    rw[96:128] = rw[32:64]   # group 3 equals group 1
    idx, tw, ridx, rwt = _route_both(q, orc, cfgd, inp, T)
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rwt).max() <= 1


# ---------------------------------------------------------------- group
@pytest.mark.parametrize("E,k,T,zipf", [(16, 4, 8, False), (64, 8, 16, False), (256, 8, 2048, True),
                                        (256, 8, 1, False), (8, 8, 5, False), (1024, 8, 300, True),
                                        (24, 5, 37, False), (64, 8, 8191, True)])
def test_group_bitexact(q, orc, E, k, T, zipf):
    import torch
    rng = np.random.default_rng(E + T)
    if zipf:
        p = rng.zipf(1.3, size=E).astype(np.float64)
        p /= p.sum()
    else:
        p = np.full(E, 1.0 / E)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    cfgd = _cfg(n_experts=E, top_k=k)
    cfg = q.make_cfg(**cfgd)
    d = gu.dev()
    cnt = torch.empty(E, dtype=torch.int32, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    perm = torch.empty(T * k, dtype=torch.int32, device=d)
    act = torch.full((E,), -7, dtype=torch.int32, device=d)
    na = torch.empty(1, dtype=torch.int32, device=d)
    q.group(cfg, gu.to_dev(idx), T, cnt, off, perm, act, na)
    torch.cuda.synchronize()
    rc, ro, rp, ra = orc.group(orc.make_cfg(**cfgd), idx)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)
    assert int(na.item()) == ra.size
    assert np.array_equal(act.cpu().numpy()[: ra.size], ra)


def test_group_flags_out_of_range_ids(q):
    import torch
    cfg = q.make_cfg(**_cfg(n_experts=16, top_k=4))
    idx = np.tile(np.arange(4, dtype=np.int32), (3, 1))
    idx[1, 2] = 16
    d = gu.dev()
    na = torch.zeros(1, dtype=torch.int32, device=d)
    q.group(cfg, gu.to_dev(idx), 3, torch.empty(16, dtype=torch.int32, device=d),
            torch.empty(17, dtype=torch.int32, device=d), torch.empty(12, dtype=torch.int32, device=d),
            torch.empty(16, dtype=torch.int32, device=d), na)
    torch.cuda.synchronize()
    assert int(na.item()) == -1


# ---------------------------------------------------------------- layer
LAYER_CASES = [  # cfg kwargs, T, seed
    (gu.workload_cfg(0), 8, synth.workload_seed(0)),
    (_cfg(wbits=8), 8, 11),
    (_cfg(wbits=2), 8, 12),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 37, 13),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=8), 19, 14),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=2), 23, 15),
    (_cfg(hidden=640, ffn=384, n_experts=12, top_k=2, has_shared=True), 1, 16),
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 16, 17),
    (_cfg(hidden=256, ffn=128, n_experts=4, top_k=4), 29, 18),   # every expert gets many tokens
    # more than 512 (token, expert) pairs: the grouped-GEMM (MFMA) path, ragged token tiles
    (_cfg(hidden=256, ffn=128, n_experts=16, top_k=4), 160, 19),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 131, 20),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=8), 117, 21),
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True,
          wbits=2), 109, 22),
    (_cfg(hidden=512, ffn=256, n_experts=8, top_k=2, has_shared=True), 300, 23),  # experts with > 64 tokens
]


@pytest.mark.parametrize("cfgd,T,seed", LAYER_CASES)
def test_layer_vs_oracle(q, orc, cfgd, T, seed):
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                             n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=cfgd["wbits"])
    w = gu.upload_layer(inp)
    out, idx, tw = gu.run_layer(cfgd, w, inp["x"])
    ref, ridx, rw = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    err = gu.rel_err_per_token(out, ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("T", [21, 150])
def test_ffn_entry_matches_layer(q, orc, T):
    """coli_moe_ffn on the oracle's route (grouped by coli_moe_group) equals the oracle FFN
    (T = 150: 750 pairs, the grouped-GEMM path)."""
    import torch
    cfgd = _cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True)
    inp = synth.layer_inputs(31, 0, tokens=T, hidden=384, ffn=256, n_experts=24, has_shared=True, wbits=4)
    ocfg = orc.make_cfg(**cfgd)
    ridx, rw = orc.route(ocfg, inp["router_w"], inp["router_bias"], inp["x"])
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


# ------------------------------------------------- exact-arithmetic cases
def _exact_inputs(H, F, E, wbits, T, seed, zero_routed_down=False):
    """Integer activations with a +-127 in every block (Q8_0 scale exactly 1), unit
    weight scales, gate weights >= 0 with every gate sum >= 40 (silu(g) == g in fp32
    and fp64), up weights in [-2, 1] (sums below 2^24), and down rows that touch a
    single block each, so that every floating-point step of the layer is exact or a
    single correctly rounded operation."""
    rng = np.random.default_rng(seed)
    import oracle
    x = rng.integers(1, 128, (T, H)).astype(np.float32)
    x[:, ::32] = 127.0
    blobs, scales = [], []
    for e in range(E):
        gate = rng.integers(0, 2, (F, H)).astype(np.int8)           # 0/1 weights, positive sums
        gate[:, 0] = 1
        up = rng.integers(-2, 2, (F, H)).astype(np.int8)
        down = np.zeros((H, F), np.int8)
        if not zero_routed_down or e == E - 1:
            lo, hi = {8: (-127, 128), 4: (-8, 8), 2: (-2, 2)}[wbits]
            for r in range(H):
                b = r % (F // 32)
                down[r, 32 * b:32 * b + 32] = rng.integers(lo, hi, 32)
        blob = np.concatenate([oracle.pack(gate.ravel(), wbits), oracle.pack(up.ravel(), wbits),
                               oracle.pack(down.ravel(), wbits)])
        blobs.append(blob)
        scales.append(np.ones(2 * F + H, np.float32))
    return x, np.stack(blobs), np.stack(scales)


@pytest.mark.parametrize("wbits,T", [(4, 11), (8, 11), (2, 11), (4, 530), (8, 530), (2, 530)])
def test_layer_exact_case_bitidentical(q, orc, wbits, T):
    """T = 530 (k = 1) takes the grouped-GEMM path."""
    H, F, E = 256, 128, 6
    x, blobs, scales = _exact_inputs(H, F, E, wbits, T, 100 + wbits)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0, wbits=wbits)
    rw = synth.router_weight(3, 0, E, H, std=0.001)
    rb = synth.router_bias(3, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, rwt = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx) and np.all(tw == 1.0) and np.all(rwt == 1.0)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("H,F,T", [(512, 2048, 11), (6144, 256, 5), (6144, 2048, 3)])
def test_layer_exact_case_long_rows_bitidentical(q, orc, H, F, T):
    """The exact case at the row lengths of the GLM-scale kernels: down rows of 2048 inputs
    (one 16-byte chunk per lane over 64 lanes: the pipelined down GEMV, 8 rows per
    wavefront) and gate/up rows of 6144 inputs (three chunks per lane: the software-
    pipelined batched GEMV), int4, decode sizes."""
    print(f"exact long rows H={H} F={F} T={T}", flush=True)
    E = 6
    x, blobs, scales = _exact_inputs(H, F, E, 4, T, 400 + H // 256 + F // 256)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0, wbits=4)
    rw = synth.router_weight(5, 0, E, H, std=0.001)
    rb = synth.router_bias(5, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, _ = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("wbits,T", [(4, 13), (8, 13), (2, 13), (4, 181), (8, 181), (2, 181)])
def test_shared_expert_exact_case_bitidentical(q, orc, wbits, T):
    """Routed experts with all-zero down rows contribute exact zeros, so the output is
    the shared expert alone and must be bit-identical (k > 1, grouped router).
    T = 181 (543 pairs) takes the grouped-GEMM path."""
    H, F, E = 256, 128, 9   # 8 routed + the shared expert (the last blob)
    x, blobs, scales = _exact_inputs(H, F, E, wbits, T, 200 + wbits, zero_routed_down=True)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E - 1, top_k=3, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
                wbits=wbits)
    rw = synth.router_weight(4, 0, E - 1, H, std=0.001)
    rb = synth.router_bias(4, 0, E - 1)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, _ = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------- determinism and batch invariance
def test_layer_deterministic_and_batch_invariant(q, orc):
    cfgd = gu.workload_cfg(1)
    T = 16
    inp = synth.layer_inputs(synth.workload_seed(1), 0, tokens=T, hidden=2048, ffn=1024, n_experts=64,
                             has_shared=False, wbits=4)
    w = gu.upload_layer(inp)
    a = gu.run_layer(cfgd, w, inp["x"])
    b = gu.run_layer(cfgd, w, inp["x"])
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    # each token alone (T = 1) gives the same bits as inside the batch of 16
    for t in (0, 7, 15):
        s = gu.run_layer(cfgd, w, inp["x"][t:t + 1])
        assert np.array_equal(s[0].view(np.uint32), a[0][t:t + 1].view(np.uint32))
        assert np.array_equal(s[1], a[1][t:t + 1])


def test_zero_input_gives_zero(q):
    cfgd = _cfg(has_shared=True, n_group=2, topk_group=1)
    inp = synth.layer_inputs(9, 0, tokens=5, hidden=256, ffn=128, n_experts=16, has_shared=True, wbits=4)
    out, _, _ = gu.run_layer(cfgd, gu.upload_layer(inp), np.zeros((5, 256), np.float32))
    assert np.all(out == 0.0)
