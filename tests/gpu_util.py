"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP library, compare."""
import numpy as np

import synth


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def upload_layer(inp, blobs=None):
    """Device Weights from a synth.layer_inputs() dict (blobs may be given separately)."""
    import quantized_moe_sigmoid_amd as q
    b = inp["blobs"] if blobs is None else blobs
    return q.Weights(experts=to_dev(np.ascontiguousarray(b).reshape(-1)), scales=to_dev(inp["scales"]),
                     router_w=to_dev(inp["router_w"]), router_bias=to_dev(inp["router_bias"]))


def run_layer(cfg_dict, w, x_np, with_route=True):
    """coli_moe_layer on device; returns numpy (out, idx, w)."""
    import torch
    import quantized_moe_sigmoid_amd as q
    cfg = q.make_cfg(**cfg_dict)
    T = x_np.shape[0]
    x = to_dev(x_np)
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev())
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev()) if with_route else None
    tw = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev()) if with_route else None
    ws = q.alloc_workspace(cfg, max(T, 1), dev())
    q.layer(cfg, w, x, out, ws, idx, tw)
    torch.cuda.synchronize()
    res = (out.cpu().numpy(),)
    if with_route:
        res += (idx.cpu().numpy(), tw.cpu().numpy())
    return res


def rel_err_per_token(out, ref):
    """max_r |out - ref| / max_r |ref| for each token (0 where ref is all zero and out equals it)."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def ulp_diff_f32(a, b):
    """Distance in fp32 ulps (a, b same sign or tiny)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def workload_cfg(i, wbits=None):
    w = dict(synth.WORKLOADS[i])
    if wbits is not None:
        w["wbits"] = wbits
    return w
