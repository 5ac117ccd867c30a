"""The expert residency tier on the GPU: experts in pinned host RAM, a small pool of HBM
slots managed by coli_tier_plan (LRU, pinned hot store), misses copied by
coli_moe_tier_stage, and the unchanged group/FFN entry points run on the pool with the
route in slot ids. The layer output must be bit-identical to the resident layer's, batch
after batch, while experts are evicted and reloaded (JustVugg/colibri README, "Never wait
for the disk twice")."""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_moe_sigmoid_amd as q
    q.lib()
    return q


def _tiered_run(q, cfgd, slots, batches, seed, pinned=None, warm=None):
    import torch
    d = gu.dev()
    E, H = cfgd["n_experts"], cfgd["hidden"]
    S = 1 if cfgd["has_shared"] else 0
    sg = cfgd.get("scale_group", 0)
    inp = synth.layer_inputs(seed, 0, tokens=1, hidden=H, ffn=cfgd["ffn"], n_experts=E, has_shared=cfgd["has_shared"],
                             wbits=cfgd["wbits"], scale_group=sg)
    cfg = q.make_cfg(**cfgd)
    pcfg = q.make_cfg(**dict(cfgd, n_experts=slots, n_group=1, topk_group=1))  # the pool's shape
    blob, nsc = q.blob_bytes(cfg), q.scales_per_expert(cfg)
    resident = gu.upload_layer(inp)
    # slow tier: pinned host copies; fast tier: slots (+ shared) in HBM
    hb = torch.from_numpy(np.ascontiguousarray(inp["blobs"]).reshape(-1)).pin_memory()
    hs = torch.from_numpy(np.ascontiguousarray(inp["scales"]).reshape(-1)).pin_memory()
    pool_b = torch.zeros((slots + S) * blob, dtype=torch.uint8, device=d)
    pool_s = torch.zeros((slots + S) * nsc, dtype=hs.dtype, device=d)
    pool = q.Weights(pool_b, pool_s, resident.router_w, resident.router_bias)
    tier = q.Tier(E, slots, pinned)
    if S:
        q.tier_stage(cfg, slots, hb, hs, [E], [slots], pool_b, pool_s)
    loads = 0
    for bi, x_np in enumerate(batches):
        T = x_np.shape[0]
        print(f"tier batch {bi} T={T} slots={slots}", flush=True)
        x = gu.to_dev(x_np)
        ws = q.alloc_workspace(cfg, T, d)
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=d)
        tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=d)
        q.route(cfg, resident, x, idx, tw, ws)
        slot_idx, le, ls = tier.plan(idx.cpu().numpy())
        loads += le.size
        q.tier_stage(cfg, slots, hb, hs, le, ls, pool_b, pool_s)
        sidx = gu.to_dev(slot_idx)
        cnt = torch.empty(slots, dtype=torch.int32, device=d)
        off = torch.empty(slots + 1, dtype=torch.int32, device=d)
        perm = torch.empty(T * cfg.top_k, dtype=torch.int32, device=d)
        act = torch.empty(slots, dtype=torch.int32, device=d)
        na = torch.empty(1, dtype=torch.int32, device=d)
        q.group(pcfg, sidx, T, cnt, off, perm, act, na)
        out = torch.empty((T, H), dtype=torch.float32, device=d)
        q.ffn(pcfg, pool, x, sidx, tw, off, perm, act, na, out, q.alloc_workspace(pcfg, T, d))
        ref, ridx, _ = gu.run_layer(cfgd, resident, x_np)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ridx)
        # the pool holds each routed expert's bytes, and the output is the resident layer's
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), bi
    return tier, loads


@pytest.mark.parametrize("wbits,sg", [(4, 0), (40, 32)])
def test_tiered_decode_bitidentical_to_resident(q, wbits, sg):
    """Decode-sized batches (the GEMV path) through a pool of 14 slots for 32 experts: each
    batch's union (at most 12) fits beside the two pinned experts, earlier experts are
    evicted and reloaded."""
    cfgd = dict(hidden=512, ffn=256, n_experts=32, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
                wbits=wbits, scale_group=sg)
    batches = [synth.activations(500 + wbits, 0, 3, 512, index=i) for i in range(10)]
    pinned = np.zeros(32, np.uint8)
    pinned[[0, 31]] = 1
    tier, loads = _tiered_run(q, cfgd, 14, batches, 500 + wbits, pinned)
    assert loads > 14  # experts were evicted and reloaded


def test_tiered_grouped_gemm_bitidentical_to_resident(q):
    """A batch past 512 pairs (grouped GEMMs) on a pool whose slots hold the experts in a
    permuted order (a warm-up batch loads part of the union first)."""
    cfgd = dict(hidden=512, ffn=512, n_experts=24, top_k=4, n_group=1, topk_group=1, rsf=1.0, has_shared=True,
                wbits=4, scale_group=0)
    batches = [synth.activations(61, 0, 2, 512, index=0), synth.activations(61, 0, 150, 512, index=1),
               synth.activations(61, 0, 160, 512, index=2)]
    tier, _ = _tiered_run(q, cfgd, 24, batches, 61)
    assert not np.array_equal(tier.expert_in, np.arange(24))  # not the identity placement


@pytest.mark.parametrize("wbits,sg,Ts,slots", [(4, 0, (3,) * 6, 14), (40, 32, (3,) * 6, 14),
                                               (4, 0, (3, 150, 3, 150, 160, 5), 36)])
def test_layer_tiered_overlapped_bitidentical(q, wbits, sg, Ts, slots):
    """coli_moe_layer_tiered: the misses copy on a second stream while the resident pairs
    compute; batch after batch the output and the route equal the resident layer's, bit
    for bit (T >= 150: grouped GEMMs, after small batches that leave part of the union
    resident), and every batch matches the oracle: route bit-exact, weights within one
    ulp, output within the 1e-3 per-token bar."""
    import torch
    import oracle
    d = gu.dev()
    T = max(Ts)
    E = 32 if T < 100 else 36
    cfgd = dict(hidden=512, ffn=256, n_experts=E, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
                wbits=wbits, scale_group=sg)
    seed = 700 + wbits + T
    inp = synth.layer_inputs(seed, 0, tokens=1, hidden=512, ffn=256, n_experts=E, has_shared=True, wbits=wbits,
                             scale_group=sg)
    cfg = q.make_cfg(**cfgd)
    blob, nsc = q.blob_bytes(cfg), q.scales_per_expert(cfg)
    resident = gu.upload_layer(inp)
    hb = torch.from_numpy(np.ascontiguousarray(inp["blobs"]).reshape(-1)).pin_memory()
    hs = torch.from_numpy(np.ascontiguousarray(inp["scales"]).reshape(-1)).pin_memory()
    pool_b = torch.zeros((slots + 1) * blob, dtype=torch.uint8, device=d)
    pool_s = torch.zeros((slots + 1) * nsc, dtype=hs.dtype, device=d)
    tier = q.Tier(E, slots)
    q.tier_stage(cfg, slots, hb, hs, [E], [slots], pool_b, pool_s)
    cs = torch.cuda.Stream(d)
    ev = q.HipEvent()
    ws = q.alloc_tier_workspace(cfg, slots, T, d)
    loads_before = 0
    for bi, T in enumerate(Ts):
        print(f"tiered layer batch {bi} T={T} slots={slots} wbits={wbits}", flush=True)
        x_np = synth.activations(seed, 0, T, 512, index=bi)
        x = gu.to_dev(x_np)
        out = torch.full((T, 512), float("nan"), dtype=torch.float32, device=d)
        idx = torch.empty((T, 4), dtype=torch.int32, device=d)
        tw = torch.empty((T, 4), dtype=torch.float32, device=d)
        q.layer_tiered(cfg, resident, tier, hb, hs, pool_b, pool_s, x, out, ws, cs, ev, idx, tw)
        ref, ridx, rw = gu.run_layer(cfgd, resident, x_np)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(idx.cpu().numpy(), ridx)
        assert np.array_equal(tw.cpu().numpy().view(np.uint32), rw.view(np.uint32))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), bi
        oref, oidx, ow = oracle.layer(oracle.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                                      inp["router_bias"], x_np)
        assert np.array_equal(idx.cpu().numpy(), oidx), bi
        assert gu.ulp_diff_f32(tw.cpu().numpy(), ow).max() <= 1, bi
        assert gu.rel_err_per_token(got, oref).max() <= 1e-3, bi
    assert int(tier.c.clock) == len(Ts)
    ev.close()


def test_router_lookahead_prefetch_then_layer_bitidentical(q):
    """Layer B's router applied to layer A's input stages B's predicted union while A runs;
    B's tiered call (its input A's plus a small residual update) waits for those copies and
    equals the resident layer B bit for bit, and both layers match the oracle within the
    1e-3 per-token bar. The prefetch must cover part of B's union."""
    import torch
    import oracle
    d = gu.dev()
    E, slots, T = 32, 14, 3
    cfgd = dict(hidden=512, ffn=256, n_experts=E, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
                wbits=4, scale_group=0)
    cfg = q.make_cfg(**cfgd)
    blob, nsc = q.blob_bytes(cfg), q.scales_per_expert(cfg)
    lay = []
    for l in range(2):
        inp = synth.layer_inputs(800 + l, 0, tokens=1, hidden=512, ffn=256, n_experts=E, has_shared=True, wbits=4)
        hb = torch.from_numpy(np.ascontiguousarray(inp["blobs"]).reshape(-1)).pin_memory()
        hs = torch.from_numpy(np.ascontiguousarray(inp["scales"]).reshape(-1)).pin_memory()
        pb = torch.zeros((slots + 1) * blob, dtype=torch.uint8, device=d)
        ps = torch.zeros((slots + 1) * nsc, dtype=torch.float32, device=d)
        tier = q.Tier(E, slots)
        q.tier_stage(cfg, slots, hb, hs, [E], [slots], pb, ps)
        lay.append(dict(res=gu.upload_layer(inp), hb=hb, hs=hs, pb=pb, ps=ps, tier=tier, inp=inp))
    cs = torch.cuda.Stream(d)
    ev = q.HipEvent()
    ws = q.alloc_tier_workspace(cfg, slots, T, d)
    prefetched, later_loads = 0, 0
    for bi in range(6):
        print(f"lookahead batch {bi}", flush=True)
        xa_np = synth.activations(810, 0, T, 512, index=bi)
        xb_np = (xa_np + 0.3 * synth.activations(811, 0, T, 512, index=bi)).astype(np.float32)
        xa, xb = gu.to_dev(xa_np), gu.to_dev(xb_np)
        outs = []
        for l, x in ((0, xa), (1, xb)):
            L = lay[l]
            if l == 1:
                before = L["tier"].slot_of.copy()
            out = torch.full((T, 512), float("nan"), dtype=torch.float32, device=d)
            q.layer_tiered(cfg, L["res"], L["tier"], L["hb"], L["hs"], L["pb"], L["ps"], x, out, ws, cs, ev)
            if l == 1:
                later_loads += int(((L["tier"].slot_of >= 0) & (before < 0)).sum())
            outs.append(out)
            if l == 0:  # lookahead: B's router on A's input, staged while A's work drains
                prefetched += q.tier_prefetch(cfg, lay[1]["res"], lay[1]["tier"], lay[1]["hb"], lay[1]["hs"],
                                              lay[1]["pb"], lay[1]["ps"], xa, ws, cs)
        for l, x_np in ((0, xa_np), (1, xb_np)):
            ref, _, _ = gu.run_layer(cfgd, lay[l]["res"], x_np)
            torch.cuda.synchronize()
            got = outs[l].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (bi, l)
            inp = lay[l]["inp"]
            oref, _, _ = oracle.layer(oracle.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                                      inp["router_bias"], x_np)
            assert gu.rel_err_per_token(got, oref).max() <= 1e-3, (bi, l)
    ev.close()
    assert prefetched > 0
    print(f"prefetched {prefetched} experts, {later_loads} loaded on demand", flush=True)


def test_layer_tiered_union_too_large_leaves_out_and_tier_untouched(q):
    """A union larger than the pool: the call returns COLI_E_UNSUPPORTED after its route and
    the resident experts' phase; `out` keeps its contents, the tier state (maps, clocks) is
    unchanged, and the next call that fits still equals the resident layer bit for bit."""
    import torch
    import quantized_moe_sigmoid_amd as qq
    d = gu.dev()
    E, slots, T = 32, 4, 6
    cfgd = dict(hidden=512, ffn=256, n_experts=E, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
                wbits=4, scale_group=0)
    inp = synth.layer_inputs(830, 0, tokens=1, hidden=512, ffn=256, n_experts=E, has_shared=True, wbits=4)
    cfg = q.make_cfg(**cfgd)
    blob, nsc = q.blob_bytes(cfg), q.scales_per_expert(cfg)
    resident = gu.upload_layer(inp)
    hb = torch.from_numpy(np.ascontiguousarray(inp["blobs"]).reshape(-1)).pin_memory()
    hs = torch.from_numpy(np.ascontiguousarray(inp["scales"]).reshape(-1)).pin_memory()
    pool_b = torch.zeros((slots + 1) * blob, dtype=torch.uint8, device=d)
    pool_s = torch.zeros((slots + 1) * nsc, dtype=torch.float32, device=d)
    tier = q.Tier(E, slots)
    q.tier_stage(cfg, slots, hb, hs, [E], [slots], pool_b, pool_s)
    cs = torch.cuda.Stream(d)
    ev = q.HipEvent()
    ws = q.alloc_tier_workspace(cfg, slots, T, d)
    # one token first: its union (4 experts) fills the pool
    x1_np = synth.activations(830, 0, 1, 512, index=0)
    out1 = torch.empty((1, 512), dtype=torch.float32, device=d)
    q.layer_tiered(cfg, resident, tier, hb, hs, pool_b, pool_s, gu.to_dev(x1_np), out1, ws, cs, ev)
    torch.cuda.synchronize()
    before = (tier.slot_of.copy(), tier.expert_in.copy(), tier.last_use.copy(), int(tier.c.clock))
    x_np = synth.activations(830, 0, T, 512, index=1)
    out = torch.full((T, 512), float("nan"), dtype=torch.float32, device=d)
    print(f"tiered union too large T={T} slots={slots}", flush=True)
    with pytest.raises(qq.ColiError) as ei:
        q.layer_tiered(cfg, resident, tier, hb, hs, pool_b, pool_s, gu.to_dev(x_np), out, ws, cs, ev)
    assert ei.value.status == qq.COLI_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert np.array_equal(tier.slot_of, before[0]) and np.array_equal(tier.expert_in, before[1])
    assert np.array_equal(tier.last_use, before[2]) and int(tier.c.clock) == before[3]
    # a batch that fits afterwards
    out2 = torch.empty((1, 512), dtype=torch.float32, device=d)
    x2_np = synth.activations(830, 0, 1, 512, index=2)
    q.layer_tiered(cfg, resident, tier, hb, hs, pool_b, pool_s, gu.to_dev(x2_np), out2, ws, cs, ev)
    ref, _, _ = gu.run_layer(cfgd, resident, x2_np)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    ev.close()
