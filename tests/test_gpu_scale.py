"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Expert blobs are generated on the device (synth.device, byte-identical to the host
generator, checked here); the oracle regenerates on the host only the experts the
sampled tokens route to and evaluates those tokens one by one. Router indices are
compared for every token, layer outputs for the sampled tokens.
"""
import numpy as np
import pytest

import gpu_util as gu
import synth

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    import quantized_moe_sigmoid_amd as q
    import synth.device
    q.lib()
    synth.device.lib()
    return q, oracle


def _run(env, wl_index, T, sample, wbits=None, layer=0, scale_group=0):
    import torch
    import synth.device
    q, orc = env
    wl = gu.workload_cfg(wl_index, wbits)
    if wl["wbits"] == synth.W_MXFP4:
        scale_group = 32
    wl["scale_group"] = scale_group
    print(f"full-size {wl['name']} wbits={wl['wbits']} scale_group={scale_group} T={T}", flush=True)
    seed = synth.workload_seed(wl_index, layer)
    H, F, E, S = wl["hidden"], wl["ffn"], wl["n_experts"], 1 if wl["has_shared"] else 0
    cfg = q.make_cfg(**wl)
    blob = q.blob_bytes(cfg)
    d = gu.dev()
    blobs = torch.empty((E + S) * blob, dtype=torch.uint8, device=d)
    synth.device.fill_blobs(blobs, seed, layer, 0, E + S, blob, wl["wbits"])
    inp = synth.layer_inputs(seed, layer, tokens=T, hidden=H, ffn=F, n_experts=E, has_shared=wl["has_shared"],
                             wbits=wl["wbits"], zipf=wl.get("zipf", False), with_blobs=False,
                             scale_group=scale_group)
    w = q.Weights(blobs, gu.to_dev(inp["scales"]), gu.to_dev(inp["router_w"]), gu.to_dev(inp["router_bias"]))
    out, idx, tw = gu.run_layer(wl, w, inp["x"])
    ocfg = orc.make_cfg(**wl)
    ridx, rw = orc.route(ocfg, inp["router_w"], inp["router_bias"], inp["x"])
    assert np.array_equal(idx, ridx)
    assert gu.ulp_diff_f32(tw, rw).max() <= 1
    # the oracle on the sampled tokens, with only their experts regenerated on the host
    toks = sorted(set(int(t) for t in sample))
    need = sorted(set(int(e) for t in toks for e in ridx[t]))
    remap = {e: i for i, e in enumerate(need)}
    hb = [synth.expert_blob(seed, layer, e, H, F, wl["wbits"]) for e in need]
    hs = [inp["scales"][e] for e in need]
    if S:
        hb.append(synth.expert_blob(seed, layer, E, H, F, wl["wbits"]))
        hs.append(inp["scales"][E])
    # the device blobs equal the host generator's bytes
    for e in need[:2] + ([E] if S else []):
        got = blobs[e * blob:(e + 1) * blob].cpu().numpy()
        assert np.array_equal(got, synth.expert_blob(seed, layer, e, H, F, wl["wbits"]))
    sub = orc.make_cfg(hidden=H, ffn=F, n_experts=len(need), top_k=wl["top_k"], rsf=wl["rsf"],
                       has_shared=wl["has_shared"], wbits=wl["wbits"], scale_group=scale_group)
    sidx = np.vectorize(remap.get)(ridx[toks]).astype(np.int32)
    ref = orc.ffn(sub, np.stack(hb), np.stack(hs), inp["x"][toks], sidx, rw[toks])
    err = gu.rel_err_per_token(out[toks], ref)
    assert err.max() <= TOL, err
    assert np.all(np.isfinite(out))
    return out, idx


def test_olmoe_decode_full(env):
    for T in (1, 4, 16):
        _run(env, 1, T, range(T))


def test_glm_decode_full(env):
    for T in (1, 4, 16):
        _run(env, 2, T, range(T))


# 16 of the 2048 prefill tokens, spread over the batch (the first and the last included)
PREFILL_SAMPLE = [0, 1, 2, 131, 262, 511, 512, 777, 1023, 1024, 1300, 1536, 1801, 2000, 2046, 2047]


def test_glm_prefill_full_sampled(env):
    _, idx = _run(env, 3, 2048, PREFILL_SAMPLE)
    cnt = np.bincount(idx.ravel(), minlength=256)
    assert cnt.max() > 100 and (cnt == 0).sum() >= 1, (cnt.max(), (cnt == 0).sum())


@pytest.mark.parametrize("wbits", [8, 2])
def test_glm_verify_lowbit_full(env, wbits):
    _run(env, 4, 3, [0, 1, 2], wbits=wbits)


@pytest.mark.parametrize("fmt", ["gs64", "mxfp4"])
def test_decode_full_other_scale_formats(env, fmt):
    """Group-scaled int4 and MXFP4 weights at the OLMoE and GLM decode sizes, every token
    (GLM T = 1, 4 and 16 take different GEMV paths)."""
    kw = dict(scale_group=64) if fmt == "gs64" else dict(wbits=synth.W_MXFP4)
    _run(env, 1, 16, range(16), **kw)
    for T in (1, 4, 16):
        _run(env, 2, T, range(T), **kw)


@pytest.mark.parametrize("fmt", ["gs64", "mxfp4"])
def test_glm_prefill_full_sampled_other_scale_formats(env, fmt):
    kw = dict(scale_group=64) if fmt == "gs64" else dict(wbits=synth.W_MXFP4)
    _run(env, 3, 2048, PREFILL_SAMPLE, **kw)


@pytest.mark.parametrize("T", [1, 4])
def test_graph_replay_matches_eager(env, T):
    """A captured graph of several layer calls, replayed several times with eager work
    and synchronisations in between, reproduces the eager results bit for bit: outputs
    and routes. One token takes the selection inside the gate/up GEMV (no selection
    launch), four tokens the selection kernel."""
    import torch
    q, _ = env
    wl = gu.workload_cfg(1)
    cfg = q.make_cfg(**wl)
    d = gu.dev()
    L, k = 3, wl["top_k"]
    layers, xs, outs, idxs, tws = [], [], [], [], []
    for l in range(L):
        seed = synth.workload_seed(1, l)
        inp = synth.layer_inputs(seed, l, tokens=T, hidden=2048, ffn=1024, n_experts=64, has_shared=False, wbits=4)
        layers.append(gu.upload_layer(inp))
        xs.append(gu.to_dev(inp["x"]))
        outs.append(torch.empty((T, 2048), dtype=torch.float32, device=d))
        idxs.append(torch.empty((T, k), dtype=torch.int32, device=d))
        tws.append(torch.empty((T, k), dtype=torch.float32, device=d))
    ws = q.alloc_workspace(cfg, T, d)
    eager = []
    for l in range(L):
        q.layer(cfg, layers[l], xs[l], outs[l], ws, idxs[l], tws[l])
        eager.append((outs[l].clone(), idxs[l].clone(), tws[l].clone()))
    torch.cuda.synchronize()
    s = torch.cuda.Stream(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for l in range(L):
            q.layer(cfg, layers[l], xs[l], outs[l], ws, idxs[l], tws[l], stream=s)
    for rep in range(4):
        for l in range(L):
            outs[l].fill_(float("nan"))
            idxs[l].fill_(-7)
            tws[l].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            eo, ei, ew = eager[l]
            assert torch.equal(outs[l].view(torch.int32), eo.view(torch.int32)), (rep, l)
            assert torch.equal(idxs[l], ei), (rep, l)
            assert torch.equal(tws[l].view(torch.int32), ew.view(torch.int32)), (rep, l)
        _ = torch.randn(1000, device=d).sum().item()  # eager work between replays
