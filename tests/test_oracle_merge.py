"""Split + merge equals the single pass: 1024 seeded cases (CPU).

A deterministic host merge oracle over 1,024 cases is what llama.cpp PR 2
(Summary) validates its page-run merge with; here the cases check the oracle's
own merge against its single-pass softmax.  Cases include empty chunks, chunks
whose keys are all masked for the row, logits of extreme magnitude and rows
with no visible key at all (merged result 0, lse -inf)."""

import numpy as np

from oracle import attention


def _case(rng, i):
    D = 8
    L = int(rng.integers(0, 65))
    n_vis = int(rng.integers(0, L + 1)) if i % 7 else L        # visible prefix
    if i % 53 == 0:
        n_vis = 0                                               # all masked
    mag = [1e-3, 1.0, 30.0, 1e3, 1e5][i % 5]
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D)) * [1.0, 1e-6, 1e6][i % 3]
    n_cut = int(rng.integers(0, 6))
    cuts = sorted([0, L] + [int(x) for x in rng.integers(0, L + 1, size=n_cut)])  # repeats = empty chunks
    return q, k, v, n_vis, mag, cuts


def test_1024_merge_cases():
    rng = np.random.default_rng(20260401)
    for i in range(1024):
        q, k, v, n_vis, mag, cuts = _case(rng, i)
        full_o, full_l = attention.attend_one(q, k, v, [n_vis], mag)
        po, pl = [], []
        for c in range(len(cuts) - 1):
            k0, k1 = cuts[c], cuts[c + 1]
            n = max(0, min(n_vis, k1) - k0)
            o, l = attention.attend_one(q, k[k0:k1], v[k0:k1], [n], mag)
            po.append(o)
            pl.append(l)
        mo, ml = attention.merge(po, pl)
        if n_vis == 0:
            assert np.all(mo == 0) and np.all(np.isneginf(ml)), i
            assert np.all(full_o == 0) and np.all(np.isneginf(full_l)), i
            continue
        scale = np.abs(full_o).max()
        assert np.max(np.abs(mo - full_o)) <= 1e-12 * scale, (i, np.max(np.abs(mo - full_o)) / scale)
        assert abs(ml[0] - full_l[0]) <= 1e-12 * (1 + abs(full_l[0])), i


def test_merge_special_cases():
    o = np.arange(12, dtype=np.float64).reshape(1, 3, 4)
    l = np.array([[0.5, -np.inf, 2.0]])
    mo, ml = attention.merge(o, l)                      # single part: identity
    assert np.array_equal(mo[np.isfinite(l[0])], o[0][np.isfinite(l[0])])
    assert np.all(mo[1] == 0) and np.isneginf(ml[1])
    # two parts, one empty: the empty part has no weight
    mo, ml = attention.merge([o[0], np.full((3, 4), 99.0)], [l[0], np.full(3, -np.inf)])
    assert np.array_equal(mo[0], o[0, 0]) and ml[0] == 0.5
    # equal lse: plain average, lse + ln 2
    mo, ml = attention.merge([np.ones((1, 4)), 3 * np.ones((1, 4))], [np.zeros(1), np.zeros(1)])
    assert np.all(mo == 2.0) and abs(ml[0] - np.log(2)) < 1e-15
    # huge lse values do not overflow
    mo, ml = attention.merge([np.ones((1, 2)), -np.ones((1, 2))], [np.array([1e300]), np.array([1e300 - 1e290])])
    assert np.all(np.isfinite(mo)) and np.all(mo == 1.0)
