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
