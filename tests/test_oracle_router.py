"""Pins of the oracle's sigmoid noaux_tc router and batch-union grouping (CPU only)."""
import numpy as np
import pytest

from goldens import load
import refmath
import synth


def _cfg(oracle_lib, E, G, Gk, k, rsf, H=32):
    return oracle_lib.make_cfg(hidden=H, ffn=32, n_experts=E, top_k=k, n_group=G, topk_group=Gk, rsf=rsf)


@pytest.mark.parametrize("case", sorted(load("router_cases.txt")))
def test_router_golden(oracle_lib, case):
    c = load("router_cases.txt")[case]
    E, G, Gk, k = (int(c[n][0]) for n in ("E", "G", "Gk", "k"))
    rsf = float(c["rsf"][0])
    z = np.array([float(v) for v in c["z"]], np.float32)
    W = np.zeros((E, 32), np.float32)
    W[np.arange(E), np.arange(E)] = 1.0
    x = np.zeros((1, 32), np.float32)
    x[0, :E] = z
    bias = np.array([float(v) for v in c["bias"]], np.float32)
    idx, w, s = oracle_lib.route(_cfg(oracle_lib, E, G, Gk, k, rsf), W, bias, x, scores=True)
    assert idx[0].tolist() == [int(v) for v in c["idx"]]
    if "w" in c:
        assert w[0].tolist() == [float(v) for v in c["w"]]
    # the scores are the sigmoid of the logits, bias excluded
    assert np.allclose(s[0], 1.0 / (1.0 + np.exp(-z.astype(np.float64))), rtol=0, atol=1e-15)
    # weights are proportional to the unbiased scores and sum to rsf
    sel = s[0, idx[0]]
    assert np.allclose(w[0], sel / sel.sum() * rsf, rtol=1e-7, atol=0)


ROUTER_SHAPES = [  # E, G, Gk, k, H
    (16, 1, 1, 4, 64), (64, 1, 1, 8, 128), (256, 8, 4, 8, 256), (32, 4, 2, 6, 96),
    (24, 8, 3, 5, 32), (8, 8, 3, 3, 32), (32, 4, 1, 8, 64),
]


@pytest.mark.parametrize("E,G,Gk,k,H", ROUTER_SHAPES)
def test_router_bruteforce(oracle_lib, E, G, Gk, k, H):
    seed = 1234 + E + 7 * G + k
    x = synth.activations(seed, 0, 37, H)
    W = synth.router_weight(seed, 0, E, H)
    bias = synth.router_bias(seed, 0, E, std=0.05)
    rsf = 2.5
    idx, w = oracle_lib.route(_cfg(oracle_lib, E, G, Gk, k, rsf, H), W, bias, x)
    bidx, bw, _ = refmath.router_bruteforce(x, W, bias, E, G, Gk, k, rsf)
    assert np.array_equal(idx, bidx)
    ulp = np.spacing(np.abs(bw).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(w.astype(np.float64) - bw) <= ulp)
    # sum of weights is rsf within a few fp32 ulps
    assert np.all(np.abs(w.astype(np.float64).sum(1) - rsf) <= k * np.spacing(np.float32(rsf)))
    # distinct experts, all inside the kept groups, in non-increasing c
    assert all(len(set(r)) == k for r in idx.tolist())


def test_router_plain_topk_special_case(oracle_lib):
    """G = 1 and zero bias: the route is the top-k of the logits (sigmoid is monotone),
    i.e. numpy's stable descending argsort of x @ W^T."""
    E, H, k, T = 64, 128, 8, 50
    x = synth.activations(5, 0, T, H)
    W = synth.router_weight(5, 0, E, H)
    idx, w = oracle_lib.route(_cfg(oracle_lib, E, 1, 1, k, 1.0, H), W, np.zeros(E, np.float32), x)
    z = x.astype(np.float64) @ W.astype(np.float64).T
    want = np.argsort(-z, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, want)


def test_router_duplicate_rows_lower_index_first(oracle_lib):
    E, H, k = 32, 64, 6
    x = synth.activations(9, 0, 40, H)
    W = synth.router_weight(9, 0, E, H)
    bias = np.zeros(E, np.float32)
    W[17] = W[4]
    W[30] = W[4]
    idx, _ = oracle_lib.route(_cfg(oracle_lib, E, 1, 1, k, 1.0, H), W, bias, x)
    hit = 0
    for row in idx.tolist():
        # an identical twin is routed only after its lower-index copy
        if 17 in row:
            hit += 1
            assert 4 in row and row.index(4) < row.index(17)
        if 30 in row:
            assert 17 in row and row.index(17) < row.index(30)
    assert hit > 0


def test_router_all_eligible(oracle_lib):
    """k = Gk * E/G: every expert of the kept groups is routed."""
    E, G, Gk, H = 32, 8, 2, 64
    k = Gk * E // G
    x = synth.activations(3, 0, 20, H)
    W = synth.router_weight(3, 0, E, H)
    bias = synth.router_bias(3, 0, E)
    idx, _ = oracle_lib.route(_cfg(oracle_lib, E, G, Gk, k, 1.0, H), W, bias, x)
    for row in idx.tolist():
        groups = sorted({e // (E // G) for e in row})
        assert len(groups) == Gk
        assert sorted(row) == [e for g in groups for e in range(g * E // G, (g + 1) * E // G)]


def test_router_rejects_bad_config(oracle_lib):
    x = np.zeros((1, 32), np.float32)
    W = np.zeros((8, 32), np.float32)
    b = np.zeros(8, np.float32)
    for E, G, Gk, k in [(8, 3, 1, 1), (8, 2, 3, 1), (8, 2, 1, 5), (8, 1, 1, 0)]:
        with pytest.raises(ValueError):
            oracle_lib.route(_cfg(oracle_lib, E, G, Gk, k, 1.0), W[:E], b[:E], x)


def test_group_golden(oracle_lib):
    c = load("group_case.txt")["three_tokens"]
    E, k = int(c["E"][0]), int(c["k"][0])
    idx = np.array([int(v) for v in c["idx"]], np.int32).reshape(-1, k)
    cnt, off, perm, active = oracle_lib.group(_cfg(oracle_lib, E, 1, 1, k, 1.0), idx)
    for name, got in (("cnt", cnt), ("off", off), ("perm", perm), ("active", active)):
        assert got.tolist() == [int(v) for v in c[name]], name


@pytest.mark.parametrize("E,k,T", [(16, 4, 8), (64, 8, 16), (256, 8, 2048), (256, 8, 1), (8, 8, 5)])
def test_group_invariants(oracle_lib, E, k, T):
    rng = np.random.default_rng(E * 1000 + T)
    skew = rng.zipf(1.5, size=E).astype(np.float64)
    p = skew / skew.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    cnt, off, perm, active = oracle_lib.group(_cfg(oracle_lib, E, 1, 1, k, 1.0), idx)
    flat = idx.ravel()
    assert cnt.sum() == T * k == off[-1]
    assert np.array_equal(cnt, np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    # a stable sort of the pair ids by expert
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    assert np.array_equal(active, np.nonzero(cnt)[0])


# ---------------------------------------------------------------- adaptive expert top-p
def _topp_inputs(seed, T, E, H):
    x = synth.activations(seed, 0, T, H)
    W = synth.router_weight(seed, 0, E, H, std=0.05)
    b = synth.router_bias(seed, 0, E)
    return x, W, b


@pytest.mark.parametrize("E,G,Gk,k,p", [(16, 1, 1, 4, 0.7), (64, 1, 1, 8, 0.5), (32, 4, 2, 6, 0.75),
                                        (256, 8, 4, 8, 0.7), (8, 8, 3, 3, 0.3)])
def test_router_topp_bruteforce(oracle_lib, E, G, Gk, k, p):
    """The kept slots are the shortest prefix of the plain route (descending c) whose
    scores sum to at least p of the k slots' sum, recomputed here from the plain route
    and its scores; kept weights renormalised over the kept slots, dropped slots -1 / 0."""
    T, H, rsf = 24, 64, 2.5
    x, W, b = _topp_inputs(300 + E + k, T, E, H)
    plain = oracle_lib.make_cfg(hidden=H, ffn=32, n_experts=E, top_k=k, n_group=G, topk_group=Gk, rsf=rsf)
    idx0, w0, s = oracle_lib.route(plain, W, b, x, scores=True)
    cfg = oracle_lib.make_cfg(hidden=H, ffn=32, n_experts=E, top_k=k, n_group=G, topk_group=Gk, rsf=rsf, topp=p)
    idx, w = oracle_lib.route(cfg, W, b, x)
    dropped_any = False
    for t in range(T):
        st = s[t, idx0[t]]                      # scores of the plain slots, slot order
        cum = np.cumsum(st)                     # sequential float64 sums
        m = int(np.argmax(cum >= np.float64(np.float32(p)) * cum[-1])) + 1
        assert 1 <= m <= k
        assert np.array_equal(idx[t, :m], idx0[t, :m]) and np.all(idx[t, m:] == -1)
        want = ((st[:m] / cum[m - 1]) * np.float64(np.float32(rsf))).astype(np.float32)
        assert np.array_equal(w[t, :m], want) and np.all(w[t, m:] == 0.0)
        # kept share reaches p; without the last kept slot it does not
        assert cum[m - 1] >= p * cum[-1] * (1 - 1e-12)
        if m > 1:
            assert cum[m - 2] < np.float64(np.float32(p)) * cum[-1]
        assert abs(float(w[t, :m].astype(np.float64).sum()) - rsf) <= 4 * m * np.spacing(np.float32(rsf))
        dropped_any |= m < k
    assert dropped_any


def test_router_topp_one_and_zero_are_plain(oracle_lib):
    """topp = 0 (off) gives the plain route; topp = 1 keeps every slot."""
    T, E, H, k = 16, 32, 64, 6
    x, W, b = _topp_inputs(321, T, E, H)
    base = dict(hidden=H, ffn=32, n_experts=E, top_k=k, n_group=4, topk_group=2, rsf=1.5)
    idx0, w0 = oracle_lib.route(oracle_lib.make_cfg(**base), W, b, x)
    for p in (0.0, 1.0):
        idx, w = oracle_lib.route(oracle_lib.make_cfg(**base, topp=p), W, b, x)
        assert np.array_equal(idx, idx0) and np.array_equal(w, w0)


def test_group_skips_empty_slots(oracle_lib):
    """Index -1 (a dropped top-p slot) belongs to no expert; the grouping of the other
    pairs is the stable sort of their ids by expert."""
    E, k, T = 16, 4, 50
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    keep = rng.integers(1, k + 1, size=T)
    for t in range(T):
        idx[t, keep[t]:] = -1
    cnt, off, perm, active = oracle_lib.group(_cfg(oracle_lib, E, 1, 1, k, 1.0), idx)
    flat = idx.ravel()
    valid = np.nonzero(flat >= 0)[0]
    assert off[-1] == valid.size == cnt.sum()
    assert np.array_equal(cnt, np.bincount(flat[valid], minlength=E))
    assert np.array_equal(perm, valid[np.argsort(flat[valid], kind="stable")])
    assert np.array_equal(active, np.nonzero(cnt)[0])
