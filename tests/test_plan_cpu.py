"""The split-K partition (pa_split_plan, the host computation pa_decode uses
with pa_decode_ext.seq_lens_host): properties the partition must have, a
model of the rule written from its description, and the headline workload's
figures.  Runs on the host only (no device)."""

import numpy as np
import pytest

from paged_kv_attention_walk_amd import binding as pb

GRANULE = 128          # 32-key tiles x 4 waves of a workgroup
N_KV = 4


def _n_chunks(L, cap, chunk):
    return 1 if (L <= 0 or L > cap) else -(-L // chunk)


def _granule(c):
    c = -(-c // GRANULE) * GRANULE
    return min(max(c, GRANULE), 1 << 30)


def _model(lens, cap, n_cu, wgs):
    """The rule as stated: slots = CUs x resident workgroups; item target =
    slots - 4 n_seq when 8 n_seq <= slots (one round), else slots / 2, or 2
    slots when the batch is ragged (the longest valid sequence above 1.5
    times a slot's share 4 sum(L) / slots); capped at 4 per CU; chunk =
    ceil(4 sum(valid L) / target) rounded up to the granule; in the
    one-round case the shortest of the four granule steps from
    ceil(4 sum L / budget) up whose items fit the budget (target + 4 n_seq),
    if shorter.  Returns (chunk, target)."""
    n = len(lens)
    slots = n_cu * wgs
    per = N_KV * n
    cap_t = n_cu * 4
    valid = [L for L in lens if 0 < L <= cap]
    total = sum(valid)
    one_round = 2 * per <= slots
    target = slots - per if one_round else slots // 2
    target = max(1, min(target, cap_t))
    if not one_round and valid and 2 * max(valid) * slots > 3 * N_KV * total:
        target = min(2 * slots, cap_t)
    chunk = _granule(-(-(total * N_KV) // target))
    if one_round and total > 0:
        budget = target + per
        c0 = _granule(-(-(total * N_KV) // budget))
        for k in range(4):
            ck = c0 + GRANULE * k
            if ck < chunk and N_KV * sum(_n_chunks(L, cap, ck) for L in lens) <= budget:
                chunk = ck
                break
    return chunk, target


def _check_partition(lens, cap, chunk, items, first):
    assert chunk % GRANULE == 0 and chunk >= GRANULE
    nc = [_n_chunks(int(L), cap, chunk) for L in lens]
    assert first[0] == 0 and list(np.diff(first)) == nc          # every sequence has >= 1 chunk
    assert items == N_KV * sum(nc)
    for L, c in zip(lens, nc):                                  # chunks tile [0, L) exactly
        if 0 < L <= cap:
            assert (c - 1) * chunk < L <= c * chunk


def test_many_stream_serving_workload_is_split():
    # 128 streams of 513..8193 positions: chunks of about half a slot's share
    # (2176 positions), 1280 items over two rounds of 512 resident workgroups,
    # rather than one chunk per stream (the longest stream would set the time)
    from paged_kv_attention_walk_amd import synth
    w = synth.config5()
    chunk, items, first = pb.split_plan(w["seq_lens"], w["block_table"].shape[1] * 64, 256, 2)
    assert (chunk, items) == (2176, 1280)
    assert int(np.max(np.diff(first))) > 1


def test_even_many_sequence_batch_keeps_one_chunk_per_head():
    # 200 x 4096: more (sequence, head) pairs than a round holds, but even
    # lengths: one chunk each already balances, so the batch is not split
    chunk, items, first = pb.split_plan([4096] * 200, 4096, 256, 2)
    assert items == 800 and chunk >= 4096


def test_headline_ragged_workload():
    # 131072 + 7 x 8192, 16-position pages: one round of resident workgroups,
    # 512 items of 1536 positions on 256 compute units x 2 workgroups (one
    # workgroup per compute unit would give 256 items of 3072)
    lens = [131072] + [8192] * 7
    chunk, items, first = pb.split_plan(lens, 131072, 256, 1)
    assert (chunk, items) == (3072, 256)
    assert list(first) == [0, 43, 46, 49, 52, 55, 58, 61, 64]
    chunk, items, first = pb.split_plan(lens, 131072, 256, 2)
    assert (chunk, items) == (1536, 512)
    assert list(first) == [0, 86, 92, 98, 104, 110, 116, 122, 128]


@pytest.mark.parametrize("n_cu,wgs", [(256, 2), (256, 1), (304, 2), (80, 2), (256, 3)])
def test_random_batches_match_model_and_partition(n_cu, wgs):
    rng = np.random.default_rng(1000 + n_cu + wgs)
    for _ in range(200):
        n = int(rng.integers(1, 257))
        cap = int(rng.choice([4096, 65536, 262144]))
        lens = rng.integers(0, cap + 1, size=n)
        if rng.random() < 0.3:
            lens[rng.integers(0, n)] = -5                       # corrupt: one empty chunk
        if rng.random() < 0.3:
            lens[rng.integers(0, n)] = cap + 7
        chunk, items, first = pb.split_plan(lens, cap, n_cu, wgs)
        m_chunk, target = _model([int(x) for x in lens], cap, n_cu, wgs)
        assert chunk == m_chunk
        _check_partition([int(x) for x in lens], cap, chunk, items, first)
        slots = n_cu * wgs
        assert items <= target + N_KV * n                       # within the split grid
        if 2 * N_KV * n <= slots:
            assert items <= slots                               # one round of resident workgroups


def test_all_empty_and_single_key():
    chunk, items, first = pb.split_plan([0, 0, 0], 1024, 256, 2)
    assert (chunk, items, list(first)) == (128, 12, [0, 1, 2, 3])
    chunk, items, first = pb.split_plan([1], 16, 256, 2)
    assert (chunk, items, list(first)) == (128, 4, [0, 1])


def test_limits_and_errors():
    chunk, items, first = pb.split_plan([], 16, 256, 2)
    assert (chunk, items) == (0, 0)
    with pytest.raises(pb.PaError):
        pb.split_plan([5] * 257, 1024, 256, 2)                  # past the host plan's batch limit
    with pytest.raises(pb.PaError):
        pb.split_plan([5], 0, 256, 2)
    with pytest.raises(pb.PaError):
        pb.split_plan([5], 16, 0, 2)
