"""coli_moe_layer_noalloc (the entry point for callers that cannot allocate) against
coli_moe_layer on a caller-allocated workspace, through the C ABI: output, route and
weights bit for bit, on two calls in a row, the second with a smaller batch (the
fixed scratch then holds the first call's contents), on the GEMV path, the grouped-GEMM
path and at GLM-scale rows; and a batch larger than the scratch is rejected with
COLI_E_SCRATCH and nothing written."""
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


def _both(q, cfgd, w, x_np):
    import torch
    d = gu.dev()
    cfg = q.make_cfg(**cfgd)
    T, k = x_np.shape[0], cfgd["top_k"]
    x = gu.to_dev(x_np)
    res = []
    for noalloc in (True, False):
        out = torch.full((T, cfgd["hidden"]), float("nan"), dtype=torch.float32, device=d)
        idx = torch.full((T, k), -7, dtype=torch.int32, device=d)
        tw = torch.full((T, k), float("nan"), dtype=torch.float32, device=d)
        if noalloc:
            q.layer_noalloc(cfg, w, x, out, idx, tw)
        else:
            q.layer(cfg, w, x, out, q.alloc_workspace(cfg, T, d), idx, tw)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), tw.cpu().numpy()))
    (a, ai, aw), (b, bi, bw) = res
    assert np.all(np.isfinite(a))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ai, bi)
    assert np.array_equal(aw.view(np.uint32), bw.view(np.uint32))


@pytest.mark.parametrize("cfgd,Ts", [
    (dict(hidden=2048, ffn=1024, n_experts=64, top_k=8, n_group=1, topk_group=1, rsf=1.0, has_shared=False,
          wbits=4), (16, 3, 1)),  # the last call selects its route inside the gate/up GEMV
    (dict(hidden=256, ffn=128, n_experts=16, top_k=4, n_group=4, topk_group=2, rsf=2.5, has_shared=True,
          wbits=4), (200, 150, 5)),   # grouped GEMM (800, 600 pairs), then a decode batch
    (dict(hidden=6144, ffn=2048, n_experts=16, top_k=8, n_group=8, topk_group=4, rsf=2.5, has_shared=True,
          wbits=4), (16, 4)),
])
def test_noalloc_matches_layer_bit_for_bit(q, cfgd, Ts):
    seed = 4242 + cfgd["hidden"]
    inp = synth.layer_inputs(seed, 0, tokens=1, hidden=cfgd["hidden"], ffn=cfgd["ffn"], n_experts=cfgd["n_experts"],
                             has_shared=cfgd["has_shared"], wbits=cfgd["wbits"])
    w = gu.upload_layer(inp)
    for i, T in enumerate(Ts):
        print(f"noalloc H={cfgd['hidden']} call {i} T={T}", flush=True)
        _both(q, cfgd, w, synth.activations(seed, 0, T, cfgd["hidden"], index=i))


def test_noalloc_rejects_batch_beyond_scratch(q):
    import torch
    cfgd = dict(hidden=6144, ffn=2048, n_experts=16, top_k=8, n_group=8, topk_group=4, rsf=2.5, has_shared=True,
                wbits=4)
    cfg = q.make_cfg(**cfgd)
    T = 256
    assert q.workspace_bytes(cfg, T) > q.scratch_bytes()
    d = gu.dev()
    inp = synth.layer_inputs(7, 0, tokens=1, hidden=6144, ffn=2048, n_experts=16, has_shared=True, wbits=4,
                             with_blobs=False)
    w = q.Weights(torch.zeros(17 * q.blob_bytes(cfg), dtype=torch.uint8, device=d), gu.to_dev(inp["scales"]),
                  gu.to_dev(inp["router_w"]), gu.to_dev(inp["router_bias"]))
    x = torch.ones((T, 6144), dtype=torch.float32, device=d)
    out = torch.full((T, 6144), float("nan"), dtype=torch.float32, device=d)
    with pytest.raises(q.ColiError) as e:
        q.layer_noalloc(cfg, w, x, out)
    assert e.value.status == q.COLI_E_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
