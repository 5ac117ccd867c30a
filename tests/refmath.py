"""Second, independent routes to the oracle's results, used only to pin it.

Each function here computes the same mathematical object as an oracle function
by a different method: vectorised bit slicing instead of per-value unpacking,
a dense float64 matrix product on dequantised values instead of per-block
integer dots, a lexicographic sort instead of repeated arg-max selection.
"""
import numpy as np


def unpack_np(packed, wbits, n):
    """Vectorised unpack of a packed row (layout as in tests/golden/pack_layout.txt)."""
    b = np.asarray(packed, np.uint8).reshape(-1)
    if wbits == 8:
        return b[:n].view(np.int8).astype(np.int64)
    nb = n // 32
    if wbits == 4:
        blk = b[: nb * 16].reshape(nb, 16).astype(np.int64)
        lo, hi = blk & 0xF, blk >> 4
        vals = np.concatenate([lo, hi], axis=1)          # positions j and j+16
        return (np.where(vals >= 8, vals - 16, vals)).reshape(-1)
    if wbits == 2:
        blk = b[: nb * 8].reshape(nb, 8).astype(np.int64)
        fields = [(blk >> (2 * m)) & 3 for m in range(4)]  # positions j + 8m
        vals = np.concatenate(fields, axis=1)
        return (np.where(vals >= 2, vals - 4, vals)).reshape(-1)
    raise ValueError(wbits)


def row_bytes(n, wbits):
    return n * wbits // 8


def dequant_expert(blob, scales, hidden, ffn, wbits, scale_group=0):
    """Dense float64 gate, up [F, H] and down [H, F] matrices: scale[row] * q, or with
    group scales scale[row][input // scale_group] * q (scales gate[F][H/g], up, down[H][F/g])."""
    rh, rf = row_bytes(hidden, wbits), row_bytes(ffn, wbits)
    blob = np.asarray(blob, np.uint8)
    gate = unpack_np(blob[: ffn * rh], wbits, ffn * hidden).reshape(ffn, hidden)
    up = unpack_np(blob[ffn * rh: 2 * ffn * rh], wbits, ffn * hidden).reshape(ffn, hidden)
    down = unpack_np(blob[2 * ffn * rh: 2 * ffn * rh + hidden * rf], wbits, hidden * ffn).reshape(hidden, ffn)
    s = np.asarray(scales, np.float64)
    if scale_group == 0:
        return (gate * s[:ffn, None], up * s[ffn: 2 * ffn, None], down * s[2 * ffn:, None])
    g = scale_group
    ng, nd = ffn * (hidden // g), hidden * (ffn // g)
    sg = np.repeat(s[:ng].reshape(ffn, hidden // g), g, axis=1)
    su = np.repeat(s[ng: 2 * ng].reshape(ffn, hidden // g), g, axis=1)
    sd = np.repeat(s[2 * ng: 2 * ng + nd].reshape(hidden, ffn // g), g, axis=1)
    return (gate * sg, up * su, down * sd)


# OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element: the sixteen code points and
# their values, as the specification tabulates them (code 8 is negative zero).
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0)


def mxfp4_values_np(packed, n):
    """E2M1 values of n packed codes by table lookup (code j low nibble, j + 16 high)."""
    b = np.asarray(packed, np.uint8).reshape(-1)[: n // 2].reshape(-1, 16)
    codes = np.concatenate([b & 0xF, b >> 4], axis=1).reshape(-1)
    return np.asarray(E2M1_VALUES, np.float64)[codes]


def dequant_expert_mxfp4(blob, scales, hidden, ffn):
    """Dense float64 gate, up [F, H] and down [H, F] of an MXFP4 expert:
    e2m1(code) * 2^(u - 127) with one scale byte u per 32 inputs of a row."""
    rh, rf = hidden // 2, ffn // 2
    blob = np.asarray(blob, np.uint8)
    u = np.asarray(scales, np.uint8).astype(np.int64)
    pw = np.ldexp(1.0, u - 127)
    ng, nd = ffn * (hidden // 32), hidden * (ffn // 32)
    gate = mxfp4_values_np(blob[: ffn * rh], ffn * hidden).reshape(ffn, hidden)
    up = mxfp4_values_np(blob[ffn * rh: 2 * ffn * rh], ffn * hidden).reshape(ffn, hidden)
    down = mxfp4_values_np(blob[2 * ffn * rh: 2 * ffn * rh + hidden * rf], hidden * ffn).reshape(hidden, ffn)
    sg = np.repeat(pw[:ng].reshape(ffn, hidden // 32), 32, axis=1)
    su = np.repeat(pw[ng: 2 * ng].reshape(ffn, hidden // 32), 32, axis=1)
    sd = np.repeat(pw[2 * ng: 2 * ng + nd].reshape(hidden, ffn // 32), 32, axis=1)
    return gate * sg, up * su, down * sd


def dequant_q8(q, d):
    """Dequantised Q8_0 row: d[block] * q in float64."""
    q = np.asarray(q, np.float64).reshape(-1, 32)
    return (q * np.asarray(d, np.float64).reshape(-1, 1)).reshape(-1)


def router_bruteforce(x, W, bias, E, G, Gk, k, rsf):
    """Route by explicit sorting: group mask from a lexsort of group scores, then a
    lexsort of (-c, index) over the unmasked experts."""
    z = np.asarray(x, np.float64) @ np.asarray(W, np.float64).T       # [T, E]
    s = 1.0 / (1.0 + np.exp(-z))
    c = s + np.asarray(bias, np.float64)[None, :]
    T = z.shape[0]
    m = E // G
    idx = np.zeros((T, k), np.int64)
    w = np.zeros((T, k), np.float64)
    for t in range(T):
        cg = c[t].reshape(G, m)
        if m == 1:
            gs = cg[:, 0]
        else:
            srt = np.sort(cg, axis=1)
            gs = srt[:, -1] + srt[:, -2]
        gorder = np.lexsort((np.arange(G), -gs))
        keep = np.zeros(E, bool)
        for g in gorder[:Gk]:
            keep[g * m:(g + 1) * m] = True
        cand = np.nonzero(keep)[0]
        order = cand[np.lexsort((cand, -c[t, cand]))]
        idx[t] = order[:k]
        sel = s[t, idx[t]]
        w[t] = sel / sel.sum() * rsf
    return idx, w, s


def silu(v):
    return v / (1.0 + np.exp(-v))
