"""Host logic of the expert slot pools (no GPU): the per-layer LFU decisions of
w4_pool_plan against an independent Python model of the rule, and the error
cases.  The rule (the anyesh.me page, "Streaming without touching a single GPU
kernel": a per-layer LFU cache over expert slots): hits stay; a miss takes the
lowest empty slot, else the slot whose expert the call does not request with
the fewest uses (one use per call that requests it), then the least recently
used, then the lowest index."""

import numpy as np
import pytest


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


class ModelLFU:
    def __init__(self, E, S):
        self.E, self.S = E, S
        self.owner = [-1] * S
        self.last = [0] * S
        self.uses = [0] * E
        self.calls = 0
        self.hits = self.misses = 0

    def request(self, ids):
        self.calls += 1
        order = list(dict.fromkeys(int(i) for i in ids))
        wanted = set(order)
        misses = []
        for e in order:
            self.uses[e] += 1
            if e in self.owner:
                self.last[self.owner.index(e)] = self.calls
                self.hits += 1
                continue
            self.misses += 1
            empty = [s for s in range(self.S) if self.owner[s] < 0]
            if empty:
                v = empty[0]
            else:
                cands = [s for s in range(self.S) if self.owner[s] not in wanted]
                v = min(cands, key=lambda s: (self.uses[self.owner[s]], self.last[s], s))
            self.owner[v] = e
            self.last[v] = self.calls
            misses.append((e, v))
        slot_of = np.full(self.E, -1, dtype=np.int32)
        for s, e in enumerate(self.owner):
            if e >= 0:
                slot_of[e] = s
        return slot_of, misses


@pytest.mark.parametrize("E,S,per_call,seed", [(128, 32, 8, 0), (128, 32, 32, 1), (40, 8, 5, 2),
                                               (16, 16, 16, 3), (10, 3, 2, 4)])
def test_lfu_matches_model(w4, E, S, per_call, seed):
    rng = np.random.default_rng(seed)
    L = 3
    pool = w4.w4_pool_create(L, E, S, [4096, 512])
    models = [ModelLFU(E, S) for _ in range(L)]
    try:
        for call in range(60):
            layer = int(rng.integers(0, L))
            # skewed choices (some experts far more popular), with repeats
            p = rng.dirichlet(np.full(E, 0.3))
            ids = rng.choice(E, size=per_call, p=p)
            got_slots, got_misses = w4.w4_pool_plan(pool, layer, ids, E)
            want_slots, want_misses = models[layer].request(ids)
            assert got_misses == want_misses, (call, layer)
            assert np.array_equal(got_slots, want_slots), (call, layer)
            # every requested expert is resident, each in its own slot
            assert np.all(got_slots[ids] >= 0)
            res = got_slots[got_slots >= 0]
            assert len(set(res.tolist())) == res.size and res.max() < S
        h, m, b = w4.w4_pool_stats(pool)
        assert (h, m, b) == (sum(x.hits for x in models), sum(x.misses for x in models), 0)
    finally:
        w4.w4_pool_destroy(pool)


def test_lfu_keeps_frequent_experts(w4):
    """Three slots; expert 0 requested every call stays resident, and a
    once-used expert is evicted before a twice-used one."""
    pool = w4.w4_pool_create(1, 10, 3, [16])
    try:
        w4.w4_pool_plan(pool, 0, [0, 1, 2], 10)
        w4.w4_pool_plan(pool, 0, [0, 2], 10)          # uses: 0:2, 1:1, 2:2
        slot_of, misses = w4.w4_pool_plan(pool, 0, [0, 3], 10)
        assert misses == [(3, 1)]                    # expert 1 (one use) goes
        assert slot_of[0] == 0 and slot_of[2] == 2 and slot_of[1] == -1
        h, m, _ = w4.w4_pool_stats(pool)
        assert (h, m) == (3, 4)
    finally:
        w4.w4_pool_destroy(pool)


def test_pool_errors_leave_state_unchanged(w4):
    pool = w4.w4_pool_create(2, 8, 2, [16, 32])
    try:
        w4.w4_pool_plan(pool, 1, [3, 4], 8)
        with pytest.raises(w4.W4Error) as e:
            w4.w4_pool_plan(pool, 1, [0, 1, 2], 8)     # 3 distinct experts, 2 slots
        assert e.value.status == w4.W4_ERR_UNSUPPORTED
        with pytest.raises(w4.W4Error) as e:
            w4.w4_pool_plan(pool, 1, [0, 8], 8)        # id out of range
        assert e.value.status == w4.W4_ERR_INVALID_ARG
        slot_of, misses = w4.w4_pool_plan(pool, 1, [4, 3, 4], 8)
        assert misses == [] and slot_of[3] == 0 and slot_of[4] == 1
        assert w4.lib.w4_pool_plan(pool, 2, None, 0, None, None, None) == w4.W4_ERR_INVALID_ARG  # layer
    finally:
        w4.w4_pool_destroy(pool)
    h = w4.ctypes.c_void_p()
    for args in [(0, 8, 2, 1), (1, 8, 0, 1), (1, 8, 2, 0), (1, 8, 2, 9)]:
        pb = (w4.ctypes.c_int64 * 9)(*([16] * 9))
        assert w4.lib.w4_pool_create(*args, pb, w4.ctypes.byref(h)) == w4.W4_ERR_INVALID_ARG
    pb = (w4.ctypes.c_int64 * 1)(24)                     # not a multiple of 16
    assert w4.lib.w4_pool_create(1, 8, 2, 1, pb, w4.ctypes.byref(h)) == w4.W4_ERR_ALIGNMENT
