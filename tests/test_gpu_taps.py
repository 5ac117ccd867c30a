"""Per-block integer dots of the gate/up kernels, bit for bit against the oracle.

The gate and up values of a row are g = s * sum_b d_b * I_b (u likewise), with I_b
the exact int32 dot of Q8_0 block b and the packed weights (colibri-strix README,
"What's implemented", integer-dot and quantization kernels items). The layer output
sees g and u only through SiLU and an 8-bit requantisation of h, so the taps build
(libcolimoe_taps.so: the same kernels compiled with COLI_TAPS) records g and u
before SiLU. Here every token's activations are integers with a +-127 in each
non-zero block (Q8_0 scale exactly 1, zero blocks scale 0) and every weight scale
is 1, so:
  - a token with ONE non-zero block b has g = I_b and u = I_b(up) exactly: each
    per-block dot is compared with the oracle's, bit for bit;
  - a token with four non-zero blocks has g = the exact integer sum of four I_b
    (below 2^24, so fp32 holds it whatever the summation order).
Weights are random bytes, i.e. every int4, int2 and E2M1 code, and every int8 value
from -128 to 127, at every position. The shapes are chosen so that each kernel
family runs: the generic, batched, register-resident and pipelined GEMVs (decode,
through coli_moe_ffn and coli_moe_layer) and the grouped GEMM (> 512 pairs).
A second group of tests compares g and u on ordinary random inputs within the fp32
summation bound.
"""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu

W_MX = synth.W_MXFP4


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    import quantized_moe_sigmoid_amd as q
    from quantized_moe_sigmoid_amd import taps
    taps.lib()
    oracle.lib()
    return q, taps, oracle


def _blobs(seed, n, H, F, wbits):
    """n expert blobs of random bytes: every code of every format at every position
    (int8: raw bytes, so -128 .. 127)."""
    nbytes = synth.blob_bytes(H, F, wbits)
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (n, nbytes), dtype=np.uint8)


def _unit_scales(n, H, F, wbits, sg):
    if wbits == W_MX:
        return np.full((n, 3 * F * H // 32), 127, np.uint8)        # E8M0 127 = 1.0
    if sg:
        return np.ones((n, 3 * F * H // sg), np.float32)
    return np.ones((n, 2 * F + H), np.float32)


def _exact_x(seed, T, H):
    """Tokens t < T/2: one non-zero block; the others: four non-zero blocks. Integer
    values in [-127, 127], each non-zero block holding a +-127."""
    rng = np.random.default_rng(seed)
    nkb = H // 32
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        nb = 1 if t < T // 2 else min(4, nkb)
        blocks = rng.choice(nkb, nb, replace=False)
        for b in blocks:
            v = rng.integers(-127, 128, 32)
            v[rng.integers(0, 32)] = 127 if rng.integers(0, 2) else -127
            x[t, 32 * b:32 * b + 32] = v
    return x


def _oracle_gu(orc, cfgd, blobs, scales, x, idx):
    """Oracle g, u (double) per tap row: pair rows t*k + j, then the shared rows P + t."""
    H, F, k, E = cfgd["hidden"], cfgd["ffn"], cfgd["top_k"], cfgd["n_experts"]
    T = x.shape[0]
    S = 1 if cfgd["has_shared"] else 0
    xq, xd = orc.quantize_q8_0(x)
    sg = cfgd.get("scale_group", 0)
    rows = {}
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e >= 0:
                rows[t * k + j] = e
        if S:
            rows[T * k + t] = E
    ref = {}
    cache = {}
    for r, e in rows.items():
        t = r // k if r < T * k else r - T * k
        key = (e, t)
        if key not in cache:
            o = orc.expert_ffn(H, F, cfgd["wbits"], blobs[e], scales[e], xq[t], xd[t], scale_group=sg)
            cache[key] = (o["g"], o["u"])
        ref[r] = cache[key]
    return ref


def _run_taps(q, taps, cfgd, blobs, scales, x, router_w, router_bias, entry):
    import torch
    d = gu.dev()
    cfg = q.make_cfg(**cfgd)
    T, H, F, k, E = x.shape[0], cfgd["hidden"], cfgd["ffn"], cfgd["top_k"], cfgd["n_experts"]
    S = 1 if cfgd["has_shared"] else 0
    w = q.Weights(gu.to_dev(np.ascontiguousarray(blobs).reshape(-1)), gu.to_dev(scales), gu.to_dev(router_w),
                  gu.to_dev(router_bias))
    xd_ = gu.to_dev(x)
    out = torch.empty((T, H), dtype=torch.float32, device=d)
    tap = torch.full((T * k + S * T, 2 * F), float("nan"), dtype=torch.float32, device=d)
    idx = torch.empty((T, k), dtype=torch.int32, device=d)
    tw = torch.empty((T, k), dtype=torch.float32, device=d)
    ws = torch.empty(taps.workspace_bytes(cfg, T), dtype=torch.uint8, device=d)
    if entry == "layer":
        taps.layer_taps(cfg, w, xd_, out, ws, tap, idx, tw)
    else:
        q.route(cfg, w, xd_, idx, tw, ws)
        cnt = torch.empty(E, dtype=torch.int32, device=d)
        off = torch.empty(E + 1, dtype=torch.int32, device=d)
        perm = torch.empty(T * k, dtype=torch.int32, device=d)
        act = torch.empty(E, dtype=torch.int32, device=d)
        na = torch.empty(1, dtype=torch.int32, device=d)
        q.group(cfg, idx, T, cnt, off, perm, act, na)
        taps.ffn_taps(cfg, w, xd_, idx, tw, off, perm, act, na, out, tap, ws)
    torch.cuda.synchronize()
    return tap.cpu().numpy(), idx.cpu().numpy()


# (H, F, wbits, scale_group, T, k, entry): the kernel each case runs is noted
EXACT_CASES = [
    (256, 128, 4, 0, 16, 4, "layer"),        # generic GEMV (8 lanes per row)
    (256, 128, 8, 0, 16, 4, "ffn"),
    (256, 128, 2, 0, 16, 4, "layer"),
    (1024, 512, 4, 0, 16, 4, "layer"),       # pipelined GEMV, 32 lanes per row
    (1024, 512, 4, 0, 16, 4, "ffn"),         # register-resident GEMV, 32 lanes per row
    (2048, 1024, 4, 0, 16, 4, "layer"),      # pipelined GEMV, 64 lanes per row
    (2048, 1024, 4, 0, 16, 4, "ffn"),        # register-resident GEMV, 64 lanes per row
    (2048, 1024, 8, 0, 16, 4, "layer"),      # batched GEMV, int8 (32-byte chunks)
    (2048, 1024, 2, 0, 16, 4, "layer"),      # batched GEMV, int2 (two blocks per chunk)
    (2048, 1024, W_MX, 32, 16, 4, "layer"),  # pipelined GEMV, MXFP4
    (2048, 1024, W_MX, 32, 16, 4, "ffn"),    # batched GEMV, MXFP4
    (2048, 1024, 4, 64, 16, 4, "layer"),     # pipelined GEMV, group scales
    (2048, 1024, 8, 64, 16, 4, "ffn"),       # batched GEMV, int8 group scales
    (6144, 2048, 4, 0, 8, 8, "layer"),       # batched GEMV, three chunks per lane (GLM-scale rows)
    (512, 256, 4, 0, 150, 4, "layer"),       # grouped GEMM (600 pairs)
    (512, 256, 8, 0, 150, 4, "layer"),
    (512, 256, 2, 0, 150, 4, "ffn"),
    (512, 256, W_MX, 32, 150, 4, "layer"),
    (512, 256, 4, 64, 150, 4, "ffn"),
]


@pytest.mark.parametrize("H,F,wbits,sg,T,k,entry", EXACT_CASES)
def test_block_dots_bitexact_full_range(env, H, F, wbits, sg, T, k, entry):
    q, taps, orc = env
    E = 8
    print(f"taps exact H={H} F={F} wbits={wbits} sg={sg} T={T} k={k} {entry}", flush=True)
    cfgd = dict(hidden=H, ffn=F, n_experts=E, top_k=k, n_group=1, topk_group=1, rsf=1.0, has_shared=True,
                wbits=wbits, scale_group=sg)
    seed = 1000 + H + F + wbits + sg + T
    blobs = _blobs(seed, E + 1, H, F, wbits)
    scales = _unit_scales(E + 1, H, F, wbits, sg)
    x = _exact_x(seed + 1, T, H)
    rw = synth.router_weight(seed, 0, E, H)
    rb = synth.router_bias(seed, 0, E)
    tap, idx = _run_taps(q, taps, cfgd, blobs, scales, x, rw, rb, entry)
    ridx, _ = orc.route(orc.make_cfg(**cfgd), rw, rb, x)
    assert np.array_equal(idx, ridx)
    ref = _oracle_gu(orc, cfgd, blobs, scales, x, ridx)
    assert len(ref) == T * k + T
    nz = 0
    for r, (g, u) in ref.items():
        assert np.array_equal(tap[r, :F].astype(np.float64), g), (r, np.abs(tap[r, :F] - g).max())
        assert np.array_equal(tap[r, F:].astype(np.float64), u), (r, np.abs(tap[r, F:] - u).max())
        nz += int(np.count_nonzero(g))
    assert nz > 0
    # the dots are not all small: the weights' extreme codes were exercised
    assert max(np.abs(g).max() for g, _ in ref.values()) > 1000


@pytest.mark.parametrize("H,F,wbits,sg,T,k,entry", [
    (2048, 1024, 4, 0, 16, 8, "layer"), (2048, 1024, 8, 0, 9, 8, "ffn"), (2048, 1024, W_MX, 32, 16, 8, "layer"),
    (6144, 2048, 4, 64, 4, 8, "layer"), (512, 256, 4, 0, 150, 4, "layer"), (512, 256, 2, 64, 150, 4, "ffn")])
def test_gate_up_random_inputs_within_fp32_bound(env, H, F, wbits, sg, T, k, entry):
    """Ordinary inputs (x ~ N(0,1), random scales): g and u agree with the oracle's fp64
    values within the fp32 summation bound, per row: |g - g_ref| <= 2e-5 * max|g_ref| (a wrong block dot moves g by
    about 1/sqrt(blocks) of its size, thousands of times more)."""
    q, taps, orc = env
    E = 12
    print(f"taps random H={H} F={F} wbits={wbits} sg={sg} T={T} {entry}", flush=True)
    cfgd = dict(hidden=H, ffn=F, n_experts=E, top_k=k, n_group=1, topk_group=1, rsf=1.0, has_shared=True,
                wbits=wbits, scale_group=sg)
    seed = 2000 + H + wbits + sg + T
    inp = synth.layer_inputs(seed, 0, tokens=T, hidden=H, ffn=F, n_experts=E, has_shared=True, wbits=wbits,
                             scale_group=sg)
    tap, idx = _run_taps(q, taps, cfgd, inp["blobs"], inp["scales"], inp["x"], inp["router_w"], inp["router_bias"],
                         entry)
    ridx, _ = orc.route(orc.make_cfg(**cfgd), inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx, ridx)
    ref = _oracle_gu(orc, cfgd, inp["blobs"], inp["scales"], inp["x"], ridx)
    for r, (g, u) in ref.items():
        for got, want in ((tap[r, :F], g), (tap[r, F:], u)):
            err = np.abs(got.astype(np.float64) - want).max()
            assert err <= 2e-5 * np.abs(want).max(), (r, err, np.abs(want).max())
