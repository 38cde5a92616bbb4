"""GPU tests of the pool: append scatter and the block-table gather hook are
bit-exact against the oracle's byte model; multi-step append + decode equals
decoding freshly uploaded rows; moving every page between steps changes
nothing (bitwise)."""

import numpy as np
import pytest
import torch

from oracle import attention, pool_model
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity, run

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,P", [("q4_0", 16), ("q8_0", 48), ("bf16", 64), ("f16", 512)])
def test_debug_gather_bitexact(kind, P):
    w = synth.make_workload(f"gather_{kind}", [3 * P + 5, 1, 2 * P], 1, kind, kind, P, seed=61, n_blocks=12)
    log(f"[case] debug gather {kind} P={P}")
    dk = dev(w["k_pool"])
    dbt = dev(w["block_table"])
    rb = synth.ROW_BYTES[kind]
    for s, L in enumerate(w["seq_lens"]):
        L = int(L)
        dst = torch.zeros((4, max(L, 1), rb), dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        pb.debug_gather(dk, rb, dbt, w["block_table"].shape[1], w["k_pool"].shape[0], s, L, P, dst, err)
        torch.cuda.synchronize()
        ref = pool_model.gather_rows(w["k_pool"], w["block_table"][s], L)
        assert np.array_equal(dst.cpu().numpy()[:, :L], ref)
        assert int(err.item()) == 0
    # an out-of-range entry: rows of that page are 0xFF and the error bit is set
    bt = w["block_table"].copy()
    bt[0, 1] = 999
    dst = torch.zeros((4, 3 * P + 5, rb), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pb.debug_gather(dk, rb, dev(bt), bt.shape[1], w["k_pool"].shape[0], 0, 3 * P + 5, P, dst, err)
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    assert np.all(d[:, P:2 * P] == 0xFF) and int(err.item()) & pb.DEVERR_TABLE


def test_append_scatter_bitexact():
    P, kind, nb = 64, "bf16", 10
    rb = synth.ROW_BYTES[kind]
    log("[case] append scatter")
    kp = torch.zeros((nb, 4, P, rb), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((nb, 4, P, rb), dtype=torch.uint8, device="cuda")
    pool = pb.Pool(nb, P, kind, k_pool=kp, v_pool=vp, max_append_rows=7)   # several staging batches
    _, idx = pool.alloc(6)
    rng = np.random.default_rng(7)
    n = 40
    blocks = rng.choice(idx, size=n).astype(np.int32)
    slots = rng.integers(0, P, size=n).astype(np.int32)
    blocks[5], slots[5] = blocks[2], slots[2]           # a repeated destination: the later row wins
    krows = rng.integers(0, 256, size=(n, 4, rb), dtype=np.uint8)
    vrows = rng.integers(0, 256, size=(n, 4, rb), dtype=np.uint8)
    assert pool.append_kv(blocks, slots, krows, vrows) == pb.OK
    torch.cuda.synchronize()
    refk = pool_model.scatter_rows(np.zeros((nb, 4, P, rb), np.uint8), blocks, slots, krows)
    refv = pool_model.scatter_rows(np.zeros((nb, 4, P, rb), np.uint8), blocks, slots, vrows)
    assert np.array_equal(kp.cpu().numpy(), refk)
    assert np.array_equal(vp.cpu().numpy(), refv)
    # errors: unallocated block, slot out of range -> nothing written
    free_block = [b for b in range(nb) if b not in set(idx.tolist())][0]
    before = kp.cpu().numpy().copy()
    assert pool.append_kv([idx[0], free_block], [0, 0], krows[:2], vrows[:2]) == pb.ERR_INVALID
    assert pool.append_kv([idx[0]], [P], krows[:1], vrows[:1]) == pb.ERR_INVALID
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), before)
    pool.destroy()


def test_multistep_append_then_decode_equals_fresh_upload():
    """Resident pages across steps (colibri#372, Validation): warm every stream
    at length 1, then append one row per stream per step; each step's decode
    over the resident pool must equal the decode of a freshly uploaded pool
    holding the same rows, bit for bit."""
    P, kind, n_seq, steps = 64, "bf16", 6, 70
    rb = synth.ROW_BYTES[kind]
    nb = n_seq * 3
    log("[case] multi-step append + decode")
    kp = torch.zeros((nb, 4, P, rb), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((nb, 4, P, rb), dtype=torch.uint8, device="cuda")
    pool = pb.Pool(nb, P, kind, k_pool=kp, v_pool=vp, max_seqs=n_seq, max_blocks_per_seq=3)
    rng = np.random.default_rng(9)
    host_k = np.zeros((nb, 4, P, rb), np.uint8)
    host_v = np.zeros((nb, 4, P, rb), np.uint8)
    table = np.full((n_seq, 3), -1, np.int32)
    lens = np.zeros(n_seq, np.int32)
    extra = np.array([0, 1, 2, 0, 1, 2])                 # ragged: some streams append 2 rows a step
    for step in range(steps):
        blocks, slots, rows_k, rows_v = [], [], [], []
        for s in range(n_seq):
            for _ in range(1 + (extra[s] if step % 5 == 0 else 0)):
                L = int(lens[s])
                if L >= 3 * P:
                    continue
                if L % P == 0:
                    _, ix = pool.alloc(1)
                    table[s, L // P] = ix[0]
                blocks.append(table[s, L // P])
                slots.append(L % P)
                rows_k.append(synth.random_rows((4,), kind, seed=1000 * step + 10 * s + len(blocks)))
                rows_v.append(synth.random_rows((4,), kind, seed=7 + 1000 * step + 10 * s + len(blocks)))
                lens[s] += 1
        rk, rv = np.stack(rows_k), np.stack(rows_v)
        assert pool.append_kv(blocks, slots, rk, rv) == pb.OK
        host_k = pool_model.scatter_rows(host_k, blocks, slots, rk)
        host_v = pool_model.scatter_rows(host_v, blocks, slots, rv)
        if step % 10 != 9:
            continue
        q = synth.normal((n_seq, 1, 24, 256), seed=step)
        w = synth.Workload(q=q, k_pool=host_k, v_pool=host_v, block_table=table.copy(), seq_lens=lens.copy(),
                           n_qtok=1, k_kind=kind, v_kind=kind, page_size=P, scale=1 / 16)
        resident, _, _ = run(w, dk=kp, dv=vp)
        fresh, _, _ = run(w)
        assert np.array_equal(resident.view(np.uint32), fresh.view(np.uint32)), step
        parity(resident, attention.paged_decode(q, host_k, host_v, kind, kind, table, lens, 1 / 16)[0],
               what=f"multi-step {step}")
    pool.destroy()


def test_rotate_every_page_between_steps():
    """Moving every page to another pool slot and rewriting the table (the
    pages' rotate debug mode, llama.cpp PR 2, KV-streaming commit) leaves the
    output bitwise unchanged."""
    w = synth.make_workload("rotate", [3000, 100, 1234], 2, "q8_0", "q8_0", 16, seed=71, n_blocks=300)
    log("[case] rotate pages")
    base, _, _ = run(w)
    rng = np.random.default_rng(3)
    k, v, bt = w["k_pool"], w["v_pool"], w["block_table"]
    for rep in range(3):
        perm = rng.permutation(k.shape[0])            # page i moves to perm[i]
        k2 = np.empty_like(k)
        v2 = np.empty_like(v)
        k2[perm] = k
        v2[perm] = v
        bt2 = np.where(bt >= 0, perm[np.clip(bt, 0, None)], bt).astype(np.int32)
        k, v, bt = k2, v2, bt2
        w2 = dict(w)
        w2.update(k_pool=k, v_pool=v, block_table=bt)
        got, _, _ = run(synth.Workload(w2))
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32)), rep


def test_append_scatter_mixed_types_bitexact():
    # K and V pools of different encodings: each row lands with its own size
    P, nb = 16, 6
    kv = pb.kv_type("q8_0", "q4_0")
    rbk, rbv = synth.ROW_BYTES["q8_0"], synth.ROW_BYTES["q4_0"]
    log("[case] append scatter K=q8_0 V=q4_0")
    kp = torch.zeros((nb, 4, P, rbk), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((nb, 4, P, rbv), dtype=torch.uint8, device="cuda")
    pool = pb.Pool(nb, P, kv, k_pool=kp, v_pool=vp, max_append_rows=5)
    _, idx = pool.alloc(4)
    rng = np.random.default_rng(9)
    n = 23
    blocks = rng.choice(idx, size=n).astype(np.int32)
    slots = rng.integers(0, P, size=n).astype(np.int32)
    krows = rng.integers(0, 256, size=(n, 4, rbk), dtype=np.uint8)
    vrows = rng.integers(0, 256, size=(n, 4, rbv), dtype=np.uint8)
    assert pool.append_kv(blocks, slots, krows, vrows) == pb.OK
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), pool_model.scatter_rows(np.zeros((nb, 4, P, rbk), np.uint8), blocks, slots, krows))
    assert np.array_equal(vp.cpu().numpy(), pool_model.scatter_rows(np.zeros((nb, 4, P, rbv), np.uint8), blocks, slots, vrows))
    pool.destroy()


@pytest.mark.parametrize("nbytes", [16, 16 * 97, 1 << 20, (1 << 24) + 16 * 13])
def test_read_bandwidth_probe_reads_every_word_once(nbytes):
    # the probe folds what it reads with xor: the xor of its output words is the
    # xor of every 32-bit word of the buffer exactly when each is read once
    rng = np.random.default_rng(nbytes)
    host = rng.integers(-2**31, 2**31 - 1, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    log(f"[case] read probe over {nbytes} bytes")
    src = torch.from_numpy(host).cuda()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((32 * n_cu,), 0, dtype=torch.int32, device="cuda")
    pb.read_bandwidth_probe(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("wgs,u,slice_", [(1, 1, False), (4, 16, False), (32, 2, False), (2, 8, True), (16, 4, True),
                                          (8, 16, True)])
def test_read_bandwidth_probe_ex_reads_every_word_once(wgs, u, slice_):
    # every register-load configuration of the probe reads each word once
    nbytes = (1 << 22) + 16 * 77
    rng = np.random.default_rng(wgs * 100 + u)
    host = rng.integers(-2**31, 2**31 - 1, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    log(f"[case] read probe ex wgs={wgs} loads={u} slice={slice_}")
    src = torch.from_numpy(host).cuda()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros((4 * wgs * n_cu,), dtype=torch.int32, device="cuda")
    pb.read_bandwidth_probe_ex(src, sink, wgs, u, pb.PROBE_SLICE if slice_ else 0)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("slice_", [False, True])
def test_read_bandwidth_probe_ex_direct_to_lds_runs(slice_):
    # the direct-to-LDS loads discard the data (each wave overwrites one LDS
    # slot), so only completion is checked
    src = torch.ones((1 << 20) // 4 + 4 * 13, dtype=torch.int32, device="cuda")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros((4 * 8 * n_cu,), dtype=torch.int32, device="cuda")
    log(f"[case] read probe ex direct to LDS slice={slice_}")
    pb.read_bandwidth_probe_ex(src, sink, 8, 8, pb.PROBE_LDS | (pb.PROBE_SLICE if slice_ else 0))
    torch.cuda.synchronize()
