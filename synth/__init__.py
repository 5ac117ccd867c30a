"""Seeded synthetic inputs for the routed MoE layer.

This module holds no arithmetic of the method: it only draws numbers. Both the
CPU oracle (``oracle/``) and the HIP library are fed from here, so neither ever
produces an input for the other.

Randomness is one counter-based generator, SplitMix64 (G. Steele, D. Lea,
C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): for a
64-bit key ``k`` the i-th output word is ``mix64(k + (i + 1) * GOLDEN)`` with the
published SplitMix64 finaliser ``mix64``. Keys are derived from
``(seed, tag, layer, index)`` with the same finaliser, so any expert of any
layer can be regenerated on its own.

The large packed expert blobs are the only inputs also produced on the device
(``synth/gen_device.hip``): that kernel evaluates the same integer-only formulas
and a test checks both byte for byte. Everything with floating point (x, router
weights, bias, per-row scales) is drawn here on the host and uploaded.

Input recipe (shapes and distributions of the MoE layer workloads):
  x              ~ N(0, 1)              fp32 [T, H]   (Box-Muller in double)
  router weight  ~ N(0, 0.02)           fp32 [E, H]
  correction bias ~ N(0, 0.01)          fp32 [E]      (prefill: Zipf-skewed, see zipf_bias)
  per-row scales ~ U(0.005, 0.02)       fp32 [(E+S), 2F+H]
  int4 weights   uniform over [-8, 7]   (packed bytes are uniform random bytes)
  int2 weights   uniform over [-2, 1]   (packed bytes are uniform random bytes)
  int8 weights   ((b*255) >> 8) - 127 for a uniform byte b: values in [-127, 127]
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# stream tags
TAG_X = 1
TAG_ROUTER_W = 2
TAG_BIAS = 3
TAG_BLOB = 4
TAG_SCALE = 5
TAG_PERM = 6

# seeds of the named workloads
SEED_BASE = 0xC011B000


def workload_seed(cfg_index: int, layer: int = 0) -> int:
    """Seed of workload ``cfg_index`` (0..4), layer ``layer`` of a stacked set."""
    return (SEED_BASE + cfg_index + 7919 * layer) & 0xFFFFFFFFFFFFFFFF


def mix64(z):
    """SplitMix64 finaliser on uint64 numpy values (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def derive_key(seed: int, tag: int, layer: int = 0, index: int = 0) -> int:
    """64-bit stream key for (seed, tag, layer, index)."""
    with np.errstate(over="ignore"):
        k = mix64(np.uint64(seed & 0xFFFFFFFFFFFFFFFF))
        for v in (tag, layer, index):
            k = mix64(k ^ mix64(np.uint64(v) + GOLDEN))
    return int(k)


def words(key: int, n: int, start: int = 0) -> np.ndarray:
    """Output words start..start+n-1 of the SplitMix64 stream with state ``key``."""
    i = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + i * GOLDEN)


def uniform01(key: int, n: int, start: int = 0) -> np.ndarray:
    """Doubles in [0, 1): top 53 bits of each word times 2^-53."""
    return (words(key, n, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(key: int, n: int, std: float = 1.0) -> np.ndarray:
    """n standard-normal doubles (Box-Muller on word pairs), scaled by std."""
    m = (n + 1) // 2
    w = words(key, 2 * m)
    u1 = ((w[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = (w[1::2] >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return z[:n] * std


W_MXFP4 = 40  # wbits value of MXFP4 weights: 4-bit E2M1 codes, E8M0 scale bytes per 32 inputs


def row_bytes(n: int, wbits: int) -> int:
    """Packed bytes of one weight row with n inputs (n multiple of 32)."""
    return n // 2 if wbits == W_MXFP4 else n * wbits // 8


def blob_bytes(hidden: int, ffn: int, wbits: int) -> int:
    """Bytes of one expert blob: gate[F] | up[F] | down[H] packed rows."""
    return 2 * ffn * row_bytes(hidden, wbits) + hidden * row_bytes(ffn, wbits)


def random_bytes(key: int, nbytes: int) -> np.ndarray:
    """nbytes uniform bytes: word i supplies bytes 8i..8i+7, little-endian."""
    w = words(key, (nbytes + 7) // 8)
    return w.astype("<u8").view(np.uint8)[:nbytes].copy()


def int8_from_bytes(b: np.ndarray) -> np.ndarray:
    """Map uniform bytes to int8 weights in [-127, 127]: ((b*255) >> 8) - 127."""
    v = ((b.astype(np.int32) * 255) >> 8) - 127
    return v.astype(np.int8).view(np.uint8)


def expert_blob(seed: int, layer: int, expert: int, hidden: int, ffn: int, wbits: int) -> np.ndarray:
    """Packed blob of one expert (uint8). Index ``n_experts`` is the shared expert."""
    key = derive_key(seed, TAG_BLOB, layer, expert)
    b = random_bytes(key, blob_bytes(hidden, ffn, wbits))
    if wbits == 8:
        b = int8_from_bytes(b)
    return b


def scales_per_expert(hidden: int, ffn: int, scale_group: int = 0) -> int:
    """fp32 scales of one expert: one per row, or one per scale_group inputs of a row."""
    return 2 * ffn + hidden if scale_group == 0 else 3 * ffn * (hidden // scale_group)


def expert_scales(seed: int, layer: int, expert: int, hidden: int, ffn: int, scale_group: int = 0,
                  wbits: int = 4) -> np.ndarray:
    """fp32 scales of one expert, U(0.005, 0.02): per row gate[F], up[F], down[H]; or with
    group scales gate[F][H/g], up[F][H/g], down[H][F/g]. MXFP4 (scale_group 32): E8M0
    bytes uniform over 119..122 (2^-8 .. 2^-5, so |w| <= 6 * 2^-5, the range of the
    integer formats' weights), same order."""
    key = derive_key(seed, TAG_SCALE, layer, expert)
    if wbits == W_MXFP4:
        return (119 + (words(key, scales_per_expert(hidden, ffn, scale_group)) & 3)).astype(np.uint8)
    u = uniform01(key, scales_per_expert(hidden, ffn, scale_group))
    return (0.005 + 0.015 * u).astype(np.float32)


def activations(seed: int, layer: int, tokens: int, hidden: int, index: int = 0) -> np.ndarray:
    """x ~ N(0, 1), fp32 [T, H]."""
    key = derive_key(seed, TAG_X, layer, index)
    return normal(key, tokens * hidden).astype(np.float32).reshape(tokens, hidden)


def router_weight(seed: int, layer: int, n_experts: int, hidden: int, std: float = 0.02) -> np.ndarray:
    """Router weight ~ N(0, std), fp32 [E, H]."""
    key = derive_key(seed, TAG_ROUTER_W, layer)
    return normal(key, n_experts * hidden, std).astype(np.float32).reshape(n_experts, hidden)


def router_bias(seed: int, layer: int, n_experts: int, std: float = 0.01) -> np.ndarray:
    """Correction bias ~ N(0, std), fp32 [E]."""
    key = derive_key(seed, TAG_BIAS, layer)
    return normal(key, n_experts, std).astype(np.float32)


def zipf_bias(seed: int, layer: int, n_experts: int, s: float = 1.1, beta: float = 0.07) -> np.ndarray:
    """Zipf-skewed correction bias: beta * ln(r_e^(-s)) = -beta * s * ln(r_e), with r a
    seeded random permutation of the ranks 1..E. An additive bias acts on selection
    like a log-prior, so this skews routing along a Zipf law; beta = 0.07 gives
    per-expert counts from 0 up to several hundred at T = 2048 (GLM-scale shapes)."""
    key = derive_key(seed, TAG_PERM, layer)
    order = np.argsort(words(key, n_experts), kind="stable")
    rank = np.empty(n_experts, dtype=np.float64)
    rank[order] = np.arange(1, n_experts + 1, dtype=np.float64)
    return (-beta * s * np.log(rank)).astype(np.float32)


def layer_inputs(seed: int, layer: int, *, tokens: int, hidden: int, ffn: int, n_experts: int,
                 has_shared: bool, wbits: int, zipf: bool = False, with_blobs: bool = True,
                 x_index: int = 0, scale_group: int = 0) -> dict:
    """All host-side inputs of one layer. Blobs are [E+S, blob_bytes] uint8."""
    ne = n_experts + (1 if has_shared else 0)
    d = {
        "x": activations(seed, layer, tokens, hidden, x_index),
        "router_w": router_weight(seed, layer, n_experts, hidden),
        "router_bias": zipf_bias(seed, layer, n_experts) if zipf else router_bias(seed, layer, n_experts),
        "scales": np.stack([expert_scales(seed, layer, e, hidden, ffn, scale_group, wbits) for e in range(ne)]),
    }
    if with_blobs:
        d["blobs"] = np.stack([expert_blob(seed, layer, e, hidden, ffn, wbits) for e in range(ne)])
    return d


# The named workloads: shapes only (sizes, formats, router settings).
WORKLOADS = {
    0: dict(name="tiny", hidden=256, ffn=128, n_experts=16, top_k=4, n_group=1, topk_group=1,
            rsf=1.0, has_shared=False, wbits=4, tokens=(8,), layers=1),
    1: dict(name="olmoe_decode", hidden=2048, ffn=1024, n_experts=64, top_k=8, n_group=1, topk_group=1,
            rsf=1.0, has_shared=False, wbits=4, tokens=(1, 4, 16), layers=8),
    2: dict(name="glm_decode", hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8, topk_group=4,
            rsf=2.5, has_shared=True, wbits=4, tokens=(1, 4, 16), layers=8),
    3: dict(name="glm_prefill", hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8, topk_group=4,
            rsf=2.5, has_shared=True, wbits=4, tokens=(2048,), layers=1, zipf=True),
    4: dict(name="glm_verify_lowbit", hidden=6144, ffn=2048, n_experts=256, top_k=8, n_group=8,
            topk_group=4, rsf=2.5, has_shared=True, wbits=(8, 2), tokens=(3,), layers=1),
}
