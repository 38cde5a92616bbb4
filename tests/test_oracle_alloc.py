"""Pins of the allocator model against hand-derived histories (CPU).

Expected index streams below are worked out by hand from the policy the model
states (lowest free index first, all-or-nothing, generation bumped on free)."""

import numpy as np

from oracle import alloc_model as am


def test_hand_history():
    m = am.AllocModel(8)
    st, h, idx = m.alloc(3)
    assert st == am.OK and idx == [0, 1, 2] and h == [am.handle(1, i) for i in (0, 1, 2)]
    assert m.free_handles([h[1]]) == am.OK                 # block 1 back, generation 2
    st, h2, idx2 = m.alloc(2)
    assert idx2 == [1, 3] and h2 == [am.handle(2, 1), am.handle(1, 3)]
    assert m.free_handles([h[1]]) == am.STALE              # old handle of block 1
    assert m.free_handles([h2[0], h2[0]]) == am.STALE      # duplicate in one call
    assert m.n_used == 4 and m.n_free == 4                 # nothing changed
    st, _, _ = m.alloc(5)
    assert st == am.NOMEM and m.n_free == 4                # all or nothing
    st, h3, idx3 = m.alloc(4)
    assert idx3 == [4, 5, 6, 7] and m.n_free == 0
    assert m.alloc(1)[0] == am.NOMEM
    assert m.alloc(0) == (am.OK, [], [])
    assert m.alloc(-1)[0] == am.INVALID
    # a mixed call with one stale handle frees nothing
    assert m.free_handles([h3[0], h[1]]) == am.STALE and m.n_free == 0
    assert m.free_handles([am.handle(1, 8)]) == am.INVALID  # index out of range
    assert m.free_handles(h3 + [h[0]]) == am.OK and m.n_free == 5
    st, _, idx4 = m.alloc(5)
    assert idx4 == [0, 4, 5, 6, 7]


def test_generation_wraps_past_zero():
    m = am.AllocModel(1)
    m.gen[0] = (1 << 32) - 1
    st, h, _ = m.alloc(1)
    assert h == [am.handle((1 << 32) - 1, 0)]
    assert m.free_handles(h) == am.OK
    assert m.gen[0] == 1                                   # 0 is skipped
    assert m.free_handles(h) == am.STALE


def test_random_histories_keep_invariants():
    rng = np.random.default_rng(0)
    m = am.AllocModel(64)
    live = {}
    for step in range(3000):
        if rng.random() < 0.5:
            n = int(rng.integers(0, 12))
            free_before = sorted(m.free)
            st, h, idx = m.alloc(n)
            if n <= len(free_before):
                assert st == am.OK and idx == free_before[:n]
                for hh, i in zip(h, idx):
                    live[i] = hh
            else:
                assert st == am.NOMEM and sorted(m.free) == free_before
        elif live:
            keys = list(live)
            pick = [keys[int(i)] for i in rng.choice(len(keys), size=min(len(keys), int(rng.integers(1, 5))), replace=False)]
            hs = [live[i] for i in pick]
            if rng.random() < 0.2:
                hs.append(hs[0])                           # duplicate -> all rejected
                assert m.free_handles(hs) == am.STALE
            else:
                assert m.free_handles(hs) == am.OK
                for i in pick:
                    del live[i]
        assert m.n_free + m.n_used == 64
        assert set(live) == set(range(64)) - m.free
