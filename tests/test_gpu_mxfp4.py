"""MXFP4 expert weights (E2M1 codes with one E8M0 scale per 32 inputs, the Kimi K3 /
DeepSeek V4 expert format named on the JustVugg/colibri README, "Other supported models")
on the HIP path against the oracle: decode-sized batches (generic, batched and pipelined
GEMVs) and batches past 512 pairs (grouped GEMMs), with and without a shared expert.
Bars as in the parity tests; where every floating-point step is exact (unit scales,
integer activations with a +-127 per block) the output is bit-identical.
"""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu

MX = synth.W_MXFP4
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
                wbits=MX, scale_group=32)
    base.update(kw)
    return base


CASES = [  # cfg kwargs, T, seed
    (_cfg(), 8, 91),                                                       # generic GEMV
    (_cfg(hidden=384, ffn=256, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 37, 92),
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 16, 93),          # pipelined GEMV (OLMoE shape)
    (_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 1, 94),
    (_cfg(hidden=4096, ffn=1024, n_experts=16, top_k=4, has_shared=True), 5, 95),  # batched gate/up (2 chunks)
    (_cfg(hidden=6144, ffn=2048, n_experts=32, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True), 3, 96),
    # past 512 pairs: grouped GEMMs (F >= 512 keeps Q8_0 flips of h, where the GPU's fp32
    # and the oracle's fp64 sums straddle a rounding boundary, well inside the bar)
    (_cfg(hidden=512, ffn=512, n_experts=16, top_k=4, has_shared=True), 150, 97),
    (_cfg(hidden=384, ffn=1024, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True), 117, 98),
]


@pytest.mark.parametrize("cfgd,T,seed", CASES)
def test_mxfp4_layer_vs_oracle(q, orc, cfgd, T, seed):
    print(f"mxfp4 layer H={cfgd['hidden']} F={cfgd['ffn']} E={cfgd['n_experts']} k={cfgd['top_k']} T={T}", flush=True)
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"], n_experts=cfgd["n_experts"],
                             has_shared=cfgd["has_shared"], wbits=MX, scale_group=32)
    assert inp["scales"].dtype == np.uint8
    assert inp["scales"].shape[1] == q.scales_per_expert(q.make_cfg(**cfgd))
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    ref, ridx, rw = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], inp["scales"], inp["router_w"],
                              inp["router_bias"], inp["x"])
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    err = gu.rel_err_per_token(out, ref)
    assert err.max() <= TOL, err.max()


# E2M1 codes of small integers: 0 -> 0, 1 -> 2 (1.0), 2 -> 4 (2.0); sign bit 8
_CODE = {0: 0, 1: 2, 2: 4, -1: 10, -2: 12}


def _pack_codes(c):
    """Codes [rows, n] -> packed bytes: per 32-block, byte j = code j | code (j + 16) << 4."""
    c = np.asarray(c, np.uint8).reshape(-1, 32)
    return (c[:, :16] | (c[:, 16:] << 4)).astype(np.uint8).reshape(-1)


def _exact_mx_inputs(H, F, E, T, seed):
    """Integer activations with a +-127 in every block (Q8_0 scale exactly 1), unit E8M0
    scales (byte 127), gate values in {0, 1} with every gate sum >= 40 (silu(g) == g in
    fp32 and fp64), up values in [-2, 1], and down rows that touch a single block each
    with any of the sixteen codes (half-integer values included)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(1, 128, (T, H)).astype(np.float32)
    x[:, ::32] = 127.0
    m = np.vectorize(_CODE.get)
    blobs = []
    for e in range(E):
        gate = rng.integers(0, 2, (F, H))
        gate[:, 0] = 1
        up = rng.integers(-2, 2, (F, H))
        down = np.zeros((H, F), np.int64)
        for r in range(H):
            b = r % (F // 32)
            down[r, 32 * b:32 * b + 32] = rng.integers(0, 16, 32)
        blobs.append(np.concatenate([_pack_codes(m(gate)), _pack_codes(m(up)), _pack_codes(down)]))
    scales = np.full((E, 3 * F * H // 32), 127, np.uint8)
    return x, np.stack(blobs), scales


@pytest.mark.parametrize("T", [11, 530])
def test_mxfp4_exact_case_bitidentical(q, orc, T):
    """T = 530 (k = 1) takes the grouped-GEMM path."""
    print(f"mxfp4 exact T={T}", flush=True)
    H, F, E = 256, 128, 6
    x, blobs, scales = _exact_mx_inputs(H, F, E, T, 300 + T)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0)
    rw = synth.router_weight(3, 0, E, H, std=0.001)
    rb = synth.router_bias(3, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, tw = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("T", [11, 530])
def test_mxfp4_exact_case_row_scales_bitidentical(q, orc, T):
    """The exact case with one E8M0 byte per row, varied over rows: gate 142 (2^15), up
    113 (2^-14) and down 147 (2^20) on some rows, 127 elsewhere. Every product and sum stays
    exact, so the output is bit-identical to the oracle's. The grouped GEMM (T = 530) folds
    a scale into the fp16 convert only for bytes 114..140 (e2m1 * s a normal fp16 number):
    wavefronts holding a 142, 113 or 147 row take the per-result path, the others the
    folded one, in the same launch."""
    print(f"mxfp4 exact row scales T={T}", flush=True)
    H, F, E = 256, 128, 6
    x, blobs, scales = _exact_mx_inputs(H, F, E, T, 310 + T)
    nb_h, nb_f = H // 32, F // 32
    gate = np.full((E, F, nb_h), 127, np.uint8)
    up = np.full((E, F, nb_h), 127, np.uint8)
    down = np.full((E, H, nb_f), 127, np.uint8)
    rows_f, rows_h = np.arange(F), np.arange(H)
    gate[:, ((rows_f // 32) % 2 == 1) & (rows_f % 3 == 0), :] = 142   # every other wavefront's rows
    up[:, ((rows_f // 32) % 2 == 1) & (rows_f % 5 == 1), :] = 113
    down[:, ((rows_h // 32) % 2 == 0) & (rows_h % 4 == 0), :] = 147
    scales = np.concatenate([gate.reshape(E, -1), up.reshape(E, -1), down.reshape(E, -1)], axis=1)
    assert scales.shape[1] == 3 * F * H // 32
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0)
    rw = synth.router_weight(3, 0, E, H, std=0.001)
    rb = synth.router_bias(3, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, _ = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("H,F,T", [(512, 2048, 11), (6144, 256, 5)])
def test_mxfp4_exact_case_long_rows_bitidentical(q, orc, H, F, T):
    """The exact case at GLM-scale row lengths (down rows of 2048 inputs, gate/up rows of
    6144), MXFP4, decode sizes."""
    print(f"mxfp4 exact long rows H={H} F={F} T={T}", flush=True)
    E = 6
    x, blobs, scales = _exact_mx_inputs(H, F, E, T, 320 + H // 256 + F // 256)
    cfgd = _cfg(hidden=H, ffn=F, n_experts=E, top_k=1, rsf=1.0)
    rw = synth.router_weight(3, 0, E, H, std=0.001)
    rb = synth.router_bias(3, 0, E)
    inp = dict(x=x, blobs=blobs, scales=scales, router_w=rw, router_bias=rb)
    out, idx, _ = gu.run_layer(cfgd, gu.upload_layer(inp), x)
    ref, ridx, _ = orc.layer(orc.make_cfg(**cfgd), blobs, scales, rw, rb, x)
    assert np.array_equal(idx, ridx)
    assert np.abs(ref).max() > 0
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_mxfp4_scales_reach_the_kernels(q, orc):
    """Doubling one block's scale (E8M0 byte + 1) in every row changes the GPU output
    exactly as it changes the oracle's."""
    cfgd = _cfg(hidden=256, ffn=128, n_experts=4, top_k=2, has_shared=True)
    inp = synth.layer_inputs(99, 0, tokens=6, hidden=256, ffn=128, n_experts=4, has_shared=True, wbits=MX,
                             scale_group=32)
    sc = inp["scales"].copy()
    sc[:, 2::8] += 1  # block 2 of every gate/up row (8 blocks per row of 256 inputs)
    a, _, _ = gu.run_layer(cfgd, gu.upload_layer(inp), inp["x"])
    b, _, _ = gu.run_layer(cfgd, gu.upload_layer(dict(inp, scales=sc)), inp["x"])
    rb, _, _ = orc.layer(orc.make_cfg(**cfgd), inp["blobs"], sc, inp["router_w"], inp["router_bias"], inp["x"])
    assert not np.array_equal(a, b)
    assert gu.rel_err_per_token(b, rb).max() <= TOL


@pytest.mark.parametrize("T", [21, 150])
def test_mxfp4_ffn_entry_vs_oracle(q, orc, T):
    """coli_moe_ffn on the oracle's route (grouped by coli_moe_group) with MXFP4 weights
    (T = 150: 750 pairs, the grouped-GEMM path)."""
    import torch
    cfgd = _cfg(hidden=384, ffn=512, n_experts=24, top_k=5, n_group=8, topk_group=3, rsf=2.5, has_shared=True)
    inp = synth.layer_inputs(31, 0, tokens=T, hidden=384, ffn=512, n_experts=24, has_shared=True, wbits=MX,
                             scale_group=32)
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


def test_mxfp4_empty_batch_is_a_noop(q):
    """T = 0 with MXFP4 weights: the layer and FFN entry points succeed and write nothing."""
    import torch
    cfgd = _cfg(has_shared=True, n_group=2, topk_group=1)
    cfg = q.make_cfg(**cfgd)
    inp = synth.layer_inputs(5, 0, tokens=1, hidden=256, ffn=128, n_experts=16, has_shared=True, wbits=MX,
                             scale_group=32)
    w = gu.upload_layer(inp)
    d = gu.dev()
    x = torch.empty((0, 256), dtype=torch.float32, device=d)
    out = torch.full((4, 256), float("nan"), dtype=torch.float32, device=d)
    idx = torch.full((4, 4), -7, dtype=torch.int32, device=d)
    tw = torch.full((4, 4), float("nan"), dtype=torch.float32, device=d)
    ws = q.alloc_workspace(cfg, 1, d)
    q.layer(cfg, w, x, out[:0], ws, idx[:0], tw[:0])
    off = torch.full((17,), -7, dtype=torch.int32, device=d)
    act = torch.full((16,), -7, dtype=torch.int32, device=d)
    na = torch.full((1,), -7, dtype=torch.int32, device=d)
    perm = torch.full((4,), -7, dtype=torch.int32, device=d)
    q.ffn(cfg, w, x, idx[:0], tw[:0], off, perm[:0], act, na, out[:0], ws)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(tw).all() and (idx == -7).all()


@pytest.mark.parametrize("fmt", ["mxfp4", "gs64"])
def test_deterministic_and_batch_invariant_other_scale_formats(q, fmt):
    """Run to run bit-identical, and each token alone gives the bits it gets inside the
    batch (OLMoE shape, decode path)."""
    cfgd = _cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8)
    if fmt == "gs64":
        cfgd.update(wbits=4, scale_group=64)
    T = 16
    inp = synth.layer_inputs(synth.workload_seed(1), 0, tokens=T, hidden=2048, ffn=1024, n_experts=64,
                             has_shared=False, wbits=cfgd["wbits"], scale_group=cfgd["scale_group"])
    w = gu.upload_layer(inp)
    a = gu.run_layer(cfgd, w, inp["x"])
    b = gu.run_layer(cfgd, w, inp["x"])
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    for t in (0, 7, 15):
        s = gu.run_layer(cfgd, w, inp["x"][t:t + 1])
        assert np.array_equal(s[0].view(np.uint32), a[0][t:t + 1].view(np.uint32))


def test_mxfp4_graph_replay_matches_eager(q):
    """A captured graph of MXFP4 layer calls (decode and grouped-GEMM sizes), replayed with
    eager work and synchronisations in between, reproduces the eager results bit for bit."""
    import torch
    d = gu.dev()
    runs = []
    for cfgd, T in ((_cfg(hidden=2048, ffn=1024, n_experts=64, top_k=8), 4),
                    (_cfg(hidden=512, ffn=512, n_experts=16, top_k=4, has_shared=True), 150)):
        inp = synth.layer_inputs(7, 0, tokens=T, hidden=cfgd["hidden"], ffn=cfgd["ffn"],
                                 n_experts=cfgd["n_experts"], has_shared=cfgd["has_shared"], wbits=MX,
                                 scale_group=32)
        cfg = q.make_cfg(**cfgd)
        runs.append((cfg, gu.upload_layer(inp), gu.to_dev(inp["x"]),
                     torch.empty((T, cfgd["hidden"]), dtype=torch.float32, device=d), q.alloc_workspace(cfg, T, d)))
    eager = []
    for cfg, w, x, out, ws in runs:
        q.layer(cfg, w, x, out, ws)
        eager.append(out.clone())
    torch.cuda.synchronize()
    s = torch.cuda.Stream(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for cfg, w, x, out, ws in runs:
            q.layer(cfg, w, x, out, ws, stream=s)
    for rep in range(3):
        for r in runs:
            r[3].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, r in enumerate(runs):
            assert torch.equal(r[3].view(torch.int32), eager[i].view(torch.int32)), (rep, i)
        _ = torch.randn(1000, device=d).sum().item()
