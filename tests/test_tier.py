"""The expert tier's host planner (coli_tier_plan): LRU over HBM slots with a pinned hot
store, each expert of the batch union loaded once (JustVugg/colibri README, "Never wait for
the disk twice"). CPU only: checked against an independent Python LRU and its rules."""
import numpy as np
import pytest


@pytest.fixture(scope="module")
def q():
    import quantized_moe_sigmoid_amd as q
    q.lib()
    return q


class RefLRU:
    """Plain reference: misses in ascending expert order take the lowest empty slot, else
    evict the least recently used slot (lowest index on ties) outside the union and not pinned."""

    def __init__(self, E, S, pinned=None):
        self.E, self.S = E, S
        self.holder = [-1] * S
        self.last = [0] * S
        self.clock = 0
        self.pinned = set() if pinned is None else {e for e in range(E) if pinned[e]}

    def plan(self, idx):
        union = sorted({int(e) for e in np.asarray(idx).ravel() if e >= 0})
        where = {e: s for s, e in enumerate(self.holder) if e >= 0}
        misses = [e for e in union if e not in where]
        empties = [s for s in range(self.S) if self.holder[s] < 0]
        cands = sorted((self.last[s], s) for s in range(self.S)
                       if self.holder[s] >= 0 and self.holder[s] not in union and self.holder[s] not in self.pinned)
        victims = (empties + [s for _, s in cands])[: len(misses)]
        if len(victims) < len(misses):
            raise ValueError("does not fit")
        self.clock += 1
        loads = []
        for e, s in zip(misses, victims):
            self.holder[s] = e
            loads.append((e, s))
        where = {e: s for s, e in enumerate(self.holder) if e >= 0}
        for e in union:
            self.last[where[e]] = self.clock
        slot_idx = np.vectorize(lambda e: -1 if e < 0 else where[int(e)], otypes=[np.int32])(np.asarray(idx))
        return slot_idx.astype(np.int32), loads


def test_plan_matches_reference_lru_over_random_batches(q):
    rng = np.random.default_rng(3)
    E, S, k = 40, 14, 4
    pinned = np.zeros(E, np.uint8)
    pinned[[3, 17]] = 1
    t = q.Tier(E, S, pinned)
    ref = RefLRU(E, S, pinned)
    total_loads = 0
    for step in range(200):
        T = int(rng.integers(0, 4))
        idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
        if T and step % 5 == 0:
            idx[0, -1] = -1  # an empty slot (adaptive top-p) passes through
        try:
            want_idx, want_loads = ref.plan(idx)
        except ValueError:
            import quantized_moe_sigmoid_amd as qq
            with pytest.raises(qq.ColiError):
                t.plan(idx)
            continue
        slot_idx, le, ls = t.plan(idx)
        assert list(zip(le.tolist(), ls.tolist())) == want_loads
        assert np.array_equal(slot_idx, want_idx)
        total_loads += len(le)
        # the state: the slot of every loaded expert holds it
        for s, e in enumerate(t.expert_in):
            if e >= 0:
                assert t.slot_of[e] == s
        assert (t.slot_of >= 0).sum() == (t.expert_in >= 0).sum()
    assert total_loads > S  # evictions happened


def test_hits_load_nothing_and_union_is_loaded_once(q):
    t = q.Tier(16, 8)
    idx = np.array([[1, 5, 9], [5, 1, 2], [9, 2, 1]], np.int32)
    slot_idx, le, ls = t.plan(idx)
    assert sorted(le.tolist()) == [1, 2, 5, 9] and le.tolist() == sorted(le.tolist())
    assert ls.tolist() == [0, 1, 2, 3]  # empty slots, lowest first
    assert np.array_equal(t.expert_in[slot_idx], idx)  # the remapped route names the same experts
    slot_idx2, le2, _ = t.plan(idx[::-1].copy())
    assert le2.size == 0 and np.array_equal(t.expert_in[slot_idx2], idx[::-1])


def test_lru_victim_and_pins(q):
    E, S = 8, 3
    pinned = np.zeros(E, np.uint8)
    pinned[0] = 1
    t = q.Tier(E, S, pinned)
    t.plan(np.array([[0, 1, 2]], np.int32))    # slots: 0->e0 (pinned), 1->e1, 2->e2
    t.plan(np.array([[1]], np.int32))          # e1 used more recently than e2
    _, le, ls = t.plan(np.array([[3]], np.int32))
    assert le.tolist() == [3] and ls.tolist() == [2]  # e2 is the LRU non-pinned slot
    _, le, ls = t.plan(np.array([[4]], np.int32))
    assert ls.tolist() == [1]                          # e1 now; e0 is pinned and stays
    assert t.slot_of[0] == 0


def test_union_too_large_or_bad_ids_leave_the_state_unchanged(q):
    import quantized_moe_sigmoid_amd as qq
    t = q.Tier(10, 3)
    t.plan(np.array([[0, 1]], np.int32))
    before = (t.slot_of.copy(), t.expert_in.copy(), t.last_use.copy(), t.c.clock)
    with pytest.raises(qq.ColiError) as ei:
        t.plan(np.array([[2, 3, 4, 5]], np.int32))
    assert ei.value.status == qq.COLI_E_UNSUPPORTED
    for bad in (10, -2):
        with pytest.raises(qq.ColiError) as ei:
            t.plan(np.array([[1, bad]], np.int32))
        assert ei.value.status == qq.COLI_E_INVALID
    after = (t.slot_of, t.expert_in, t.last_use, t.c.clock)
    for a, b in zip(before, after):
        assert np.array_equal(a, b)


def test_stage_rejects_bad_plans_before_copying(q):
    """Validation happens on the host before any copy is enqueued (no GPU needed)."""
    import ctypes as C
    import quantized_moe_sigmoid_amd as qq
    cfg = q.make_cfg(256, 128, 16, 4, has_shared=True)
    L = q.lib()
    p = C.c_void_p(0x1000)
    le = (C.c_int32 * 2)(3, 16)
    ls = (C.c_int32 * 2)(0, 5)  # the shared expert (16) must go to slot `slots` = 4
    assert L.coli_moe_tier_stage(C.byref(cfg), 4, p, p, le, ls, 2, p, p, None) == qq.COLI_E_INVALID
    ls2 = (C.c_int32 * 2)(4, 4)  # routed expert into the shared slot
    assert L.coli_moe_tier_stage(C.byref(cfg), 4, p, p, le, ls2, 2, p, p, None) == qq.COLI_E_INVALID
    assert L.coli_moe_tier_stage(C.byref(cfg), 4, p, p, le, ls, 0, p, p, None) == qq.COLI_OK  # nothing to copy


def test_tiered_entry_points_reject_bad_arguments_on_the_host(q):
    """No GPU call is reached: every check happens before anything is enqueued."""
    import ctypes as C
    import quantized_moe_sigmoid_amd as qq
    cfg = q.make_cfg(256, 128, 16, 4, has_shared=True)
    L = q.lib()
    assert L.coli_moe_tier_workspace_bytes(C.byref(cfg), 8, 16) > 0
    assert L.coli_moe_tier_workspace_bytes(C.byref(cfg), 0, 16) == 0     # no slots
    assert L.coli_moe_tier_workspace_bytes(C.byref(cfg), 17, 16) == 0    # more slots than experts
    assert L.coli_moe_tier_workspace_bytes(C.byref(cfg), 3, 16) == 0     # k = 4 > slots
    t = q.Tier(16, 8)
    p = C.c_void_p(0x1000)
    w = q.Weights(None, None, None, None).c()
    args = lambda tier, T, ws_bytes: (C.byref(cfg), C.byref(w), tier, p, p, p, p, p, T, p, None, None, p, ws_bytes,
                                      None, p, p)
    fn = L.coli_moe_layer_tiered
    assert fn(*args(None, 4, 1 << 30)) == qq.COLI_E_INVALID                # no tier state
    assert fn(*args(C.byref(t.c), 0, 0)) == qq.COLI_OK                      # T = 0 is a no-op
    assert fn(*args(C.byref(t.c), -1, 1 << 30)) == qq.COLI_E_INVALID
    assert fn(*args(C.byref(t.c), 4, 16)) == qq.COLI_E_WORKSPACE            # workspace too small
    t2 = q.Tier(12, 8)
    assert fn(*args(C.byref(t2.c), 4, 1 << 30)) == qq.COLI_E_INVALID        # tier of another layer shape
    assert int(t.c.clock) == 0


def test_inconsistent_state_is_rejected(q):
    import quantized_moe_sigmoid_amd as qq
    t = q.Tier(8, 3)
    t.plan(np.array([[1, 2]], np.int32))
    t.expert_in[0] = 7          # slot 0 claims expert 7, whose slot_of is -1
    with pytest.raises(qq.ColiError) as ei:
        t.plan(np.array([[1]], np.int32))
    assert ei.value.status == qq.COLI_E_INVALID
    t.expert_in[0] = 1
    t.slot_of[5] = 9            # out of range
    with pytest.raises(qq.ColiError):
        t.plan(np.array([[1]], np.int32))
