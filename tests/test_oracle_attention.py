"""Pins of the oracle's attention, gather and merge (CPU)."""

import numpy as np
import pytest

from oracle import attention, pool_model, quant
from paged_kv_attention_walk_amd import synth
from oracle_checks import (HKV, HQ, D, check_against_brute_force, check_against_sdpa,
                           check_paged_equals_contiguous, random_sequence_case)


def _decoded_cases(seed, n, lens=(1, 2, 5, 17, 40), kinds=("f16", "bf16", "q8_0", "q4_0")):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        L = int(lens[i % len(lens)])
        T = 1 + i % 8
        kind = kinds[i % len(kinds)]
        scale = [1 / 16, 1.0, 0.37][i % 3]
        q, kb, vb = random_sequence_case(rng, L, T, kind, kind)
        out.append((q, quant.decode(kb, kind), quant.decode(vb, kind), L, scale))
    return out


def test_against_sdpa_library_routine():
    check_against_sdpa(attention.decode_sequence, _decoded_cases(1, 24, lens=(1, 3, 16, 33, 48, 100, 300)))


def test_against_brute_force_tiny():
    cases = _decoded_cases(2, 6, lens=(1, 4, 7, 12))
    check_against_brute_force(attention.decode_sequence, cases)


def test_gather_recovers_logical_rows():
    rng = np.random.default_rng(3)
    for P in (16, 48, 64, 128, 256, 512):
        lens = [int(x) for x in rng.integers(0, 3 * P, size=4)]
        w = synth.make_workload("g", lens, 1, "q4_0", "q4_0", P, table="shuffled", seed=P)
        cont = synth.contiguous_from_table(w["k_pool"], w["block_table"], lens, max(lens + [1]))
        for s, L in enumerate(lens):
            got = pool_model.gather_rows(w["k_pool"], w["block_table"][s], L)
            assert np.array_equal(got, cont[s, :, :L])


def test_paged_equals_contiguous_exact():
    check_paged_equals_contiguous(attention.paged_decode, attention.contiguous_decode)


def test_constant_v_rows_give_v():
    # V rows built from codes directly (not by quantising): every row the same.
    rng = np.random.default_rng(4)
    for kind in ("q4_0", "q8_0", "f16", "bf16"):
        L, T = 37, 3
        q, kb, _ = random_sequence_case(rng, L, T, kind, kind)
        one = synth.encode(rng.standard_normal((1, 256)).astype(np.float32), kind)[0]
        vb = np.broadcast_to(one, (HKV, L, one.shape[0])).copy()
        k, v = quant.decode(kb, kind), quant.decode(vb, kind)
        out, _ = attention.decode_sequence(q, k, v, L, 1 / 16)
        target = quant.decode(one[None], kind)[0]
        assert np.max(np.abs(out - target[None, None, :])) <= 4 * np.finfo(np.float64).eps * np.abs(target).max()


def test_single_key_returns_its_v_row():
    rng = np.random.default_rng(5)
    q, kb, vb = random_sequence_case(rng, 1, 1, "q8_0", "q4_0")
    k, v = quant.decode(kb, "q8_0"), quant.decode(vb, "q4_0")
    out, lse = attention.decode_sequence(q, k, v, 1, 1 / 16)
    for h in range(HQ):
        assert np.array_equal(out[0, h], v[h // 6, 0])
        assert lse[0, h] == (q[0, h].astype(np.float64) @ k[h // 6, 0]) / 16


def test_zero_query_gives_mean_of_visible_rows():
    rng = np.random.default_rng(6)
    L, T = 29, 4
    _, kb, vb = random_sequence_case(rng, L, T, "f16", "f16")
    k, v = quant.decode(kb, "f16"), quant.decode(vb, "f16")
    q = np.zeros((T, HQ, D), np.float32)
    out, lse = attention.decode_sequence(q, k, v, L, 1 / 16)
    for t in range(T):
        n = L - T + t + 1
        for h in range(HQ):
            np.testing.assert_allclose(out[t, h], v[h // 6, :n].mean(0), rtol=0, atol=1e-15)
            assert abs(lse[t, h] - np.log(n)) < 1e-14


def test_gqa_identical_queries_identical_outputs():
    rng = np.random.default_rng(7)
    L, T = 50, 2
    _, kb, vb = random_sequence_case(rng, L, T, "q4_0", "q4_0")
    k, v = quant.decode(kb, "q4_0"), quant.decode(vb, "q4_0")
    q = rng.standard_normal((T, HQ, D)).astype(np.float32)
    for g in range(HKV):
        q[:, 6 * g:6 * g + 6] = q[:, 6 * g:6 * g + 1]
    out, _ = attention.decode_sequence(q, k, v, L, 1 / 16)
    for g in range(HKV):
        for h in range(6 * g, 6 * g + 6):
            assert np.array_equal(out[:, h], out[:, 6 * g])
    assert not np.array_equal(out[:, 0], out[:, 6])


@pytest.mark.parametrize("T", [4, 8])
def test_causal_decomposition(T):
    rng = np.random.default_rng(8)
    L = 45
    q, kb, vb = random_sequence_case(rng, L, T, "bf16", "bf16")
    k, v = quant.decode(kb, "bf16"), quant.decode(vb, "bf16")
    out, lse = attention.decode_sequence(q, k, v, L, 1 / 16)
    for t in range(T):
        Lt = L - T + t + 1
        o1, l1 = attention.decode_sequence(q[t:t + 1], k[:, :Lt], v[:, :Lt], Lt, 1 / 16)
        assert np.max(np.abs(o1[0] - out[t])) <= 1e-12 * np.abs(out).max()
        assert np.max(np.abs(l1[0] - lse[t])) <= 1e-12 * np.abs(lse).max()


def test_empty_and_short_sequences():
    rng = np.random.default_rng(9)
    w = synth.make_workload("e", [0, 2, 5], 4, "q4_0", "q4_0", 16, seed=9)
    out, lse = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q4_0", "q4_0",
                                      w["block_table"], w["seq_lens"])
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    # L = 2, T = 4: tokens 0 and 1 see no key; token 2 sees key 0; token 3 keys 0..1
    assert np.all(out[1, :2] == 0) and np.all(np.isneginf(lse[1, :2]))
    assert np.all(np.isfinite(lse[1, 2:])) and np.all(np.isfinite(lse[2]))
    # eight tokens over five stored rows: tokens 0..2 see nothing, token 3 key 0
    w = synth.make_workload("e8", [5], 8, "q8_0", "q8_0", 16, seed=10)
    out, lse = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q8_0",
                                      w["block_table"], w["seq_lens"])
    assert np.all(out[0, :3] == 0) and np.all(np.isneginf(lse[0, :3])) and np.all(np.isfinite(lse[0, 3:]))
    v0 = quant.decode(pool_model.gather_rows(w["v_pool"], w["block_table"][0], 1), "q8_0")[:, 0]
    for h in range(24):
        assert np.array_equal(out[0, 3, h], v0[h // 6])          # a single visible key returns its V row


def test_corrupt_table_gives_nan_for_that_sequence_only():
    w = synth.make_workload("c", [20, 40, 9], 1, "q8_0", "q8_0", 16, seed=10)
    bt = w["block_table"].copy()
    bt[1, 1] = w["n_blocks"] + 5
    out, lse = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q8_0", bt, w["seq_lens"])
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    assert np.all(np.isfinite(out[0])) and np.all(np.isfinite(out[2]))
    bt = w["block_table"].copy()
    bt[0, 0] = -1
    out, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q8_0", bt, w["seq_lens"])
    assert np.all(np.isnan(out[0])) and np.all(np.isfinite(out[1]))
    # a length beyond the table row is corrupt too
    lens = w["seq_lens"].copy()
    lens[2] = 16 * w["block_table"].shape[1] + 1
    out, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q8_0", w["block_table"], lens)
    assert np.all(np.isnan(out[2]))


def test_planted_high_score_key_dominates():
    # a key aligned with q and a large scale: the output approaches that key's
    # V row; the residual is bounded by the other keys' total weight.
    rng = np.random.default_rng(12)
    L = 64
    kx = rng.standard_normal((HKV, L, D)).astype(np.float32) * 0.1
    q = rng.standard_normal((1, HQ, D)).astype(np.float32)
    j = 23
    for h in range(HQ):
        kx[h // 6, j] = q[0, h // 6 * 6]
    k = quant.decode(synth.encode(kx, "f16"), "f16")
    v = quant.decode(synth.encode(rng.standard_normal((HKV, L, D)).astype(np.float32), "f16"), "f16")
    out, _ = attention.decode_sequence(q, k, v, L, 1.0)
    for g in range(HKV):
        h = 6 * g
        s = q[0, h].astype(np.float64) @ k[g].T
        w_other = np.exp(np.delete(s, j) - s[j]).sum()
        assert np.max(np.abs(out[0, h] - v[g, j])) <= 2 * w_other * np.abs(v[g]).max() + 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_split_merge_equals_single_pass_quick(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 90))
    T = int(rng.integers(1, 9))
    q, kb, vb = random_sequence_case(rng, L, T, "q4_0", "q8_0")
    k, v = quant.decode(kb, "q4_0"), quant.decode(vb, "q8_0")
    cuts = sorted(set([0, L] + [int(x) for x in rng.integers(0, L + 1, size=3)]))
    a, al = attention.decode_sequence(q, k, v, L, 1 / 16)
    b, bl = attention.chunked_decode_sequence(q, k, v, L, 1 / 16, cuts)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1e-300, np.abs(a).max())
    fin = np.isfinite(al)
    assert np.array_equal(fin, np.isfinite(bl))
    assert np.max(np.abs(al[fin] - bl[fin]), initial=0) <= 1e-12 * (1 + np.abs(al[fin]).max(initial=0))
