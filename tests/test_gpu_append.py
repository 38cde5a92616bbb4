"""GPU tests of pa_append_kv_device (device rows encoded into pages on the
device): every written byte equals the oracle's encoder followed by its
scatter model, bytes no row names stay untouched, bad destinations are
skipped and reported, and decode over pages filled this way matches the
oracle."""

import numpy as np
import pytest
import torch

from oracle import attention, encode, pool_model
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity, run

pytestmark = pytest.mark.gpu

ROW_BYTES = {"f16": 512, "bf16": 512, "q8_0": 272, "q4_0": 144}


def _source_rows(n, seed, src):
    """[n][4][256] float32 rows: N(0,1) at per-row magnitudes from 1e-4 to
    3000, a zero row, and rows with the rounding cases of the encoders
    (halves, a value just below a half, the float32 product that lands on a
    half, the fp16 rounding edges).  Returns (values for the device in the
    source type, the same values widened to float32)."""
    rng = np.random.default_rng(seed)
    mags = np.array([1e-4, 0.05, 1.0, 40.0, 3000.0], np.float32)
    x = rng.standard_normal((n, 4, 256)).astype(np.float32) * mags[rng.integers(0, len(mags), size=n)][:, None, None]
    if n > 4:
        x[1] = 0.0
        blk = np.zeros(32, np.float32)
        blk[:8] = [2.5, -2.5, 0.5, -0.5, np.float32(0.5) - np.float32(2.0 ** -25), 126.5, -7.5, 3.5]
        blk[8] = np.float32(7.5) - np.float32(2.0 ** -21)
        blk[31] = 127.0
        x[2, :, :] = np.tile(blk, 8)
        x[3, 0, :] = np.resize(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65519.0, 2.0 ** -25, 2.0 ** -24,
                                         1 + 2.0 ** -8, -(1 + 3 * 2.0 ** -8)], np.float32), 256)
        x[3, 1, :32] = np.float32(7.5) - np.float32(2.0 ** -21)
        x[3, 1, 31] = 381.0
    if src == "f32":
        return torch.from_numpy(x), x
    if src == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
        return t, encode.widen_bf16(t.view(torch.int16).numpy().view(np.uint16))
    h = np.clip(x, -60000, 60000).astype(np.float16)
    return torch.from_numpy(h), encode.widen_f16(h.view(np.uint16))


def _pool(nb, P, k, v, seed):
    rng = np.random.default_rng(seed)
    hk = rng.integers(0, 256, size=(nb, 4, P, ROW_BYTES[k]), dtype=np.uint8)
    hv = rng.integers(0, 256, size=(nb, 4, P, ROW_BYTES[v]), dtype=np.uint8)
    kp, vp = dev(hk), dev(hv)
    pool = pb.Pool(nb, P, pb.kv_type(k, v), k_pool=kp, v_pool=vp)
    return pool, kp, vp, hk, hv


PAIRS = [("f16", "f16"), ("bf16", "bf16"), ("q8_0", "q8_0"), ("q4_0", "q4_0"),
         ("q8_0", "q4_0"), ("f16", "q4_0"), ("q4_0", "bf16")]


@pytest.mark.parametrize("src", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("kv", PAIRS, ids=lambda p: f"K{p[0]}-V{p[1]}")
def test_append_device_bitexact(kv, src):
    k, v = kv
    nb, P, n = 12, 16, 37
    log(f"[case] device append K={k} V={v} src={src} n={n}")
    pool, kp, vp, hk, hv = _pool(nb, P, k, v, seed=5)
    rng = np.random.default_rng(17)
    dest = rng.choice(nb * P, size=n, replace=False)
    blocks, slots = (dest // P).astype(np.int32), (dest % P).astype(np.int32)
    dk_src, xk = _source_rows(n, 23, src)
    dv_src, xv = _source_rows(n, 29, src)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool.append_kv_device(dev(blocks), dev(slots), dk_src.cuda(), dv_src.cuda(), src, err_word=err)
    torch.cuda.synchronize()
    refk = pool_model.scatter_rows(hk, blocks, slots, encode.encode(xk, k))
    refv = pool_model.scatter_rows(hv, blocks, slots, encode.encode(xv, v))
    gk, gv = kp.cpu().numpy(), vp.cpu().numpy()
    assert int(err.item()) == 0
    bad = np.argwhere(gk != refk)
    assert bad.size == 0, f"K bytes differ at {bad[:5].tolist()}"
    bad = np.argwhere(gv != refv)
    assert bad.size == 0, f"V bytes differ at {bad[:5].tolist()}"
    pool.destroy()


@pytest.mark.parametrize("kv", [("q4_0", "q4_0"), ("q8_0", "bf16")], ids=lambda p: f"K{p[0]}-V{p[1]}")
def test_append_device_many_rows(kv):
    # thousands of workgroups, every destination of a 64-page pool but one
    k, v = kv
    nb, P = 64, 64
    n = nb * P - 1
    log(f"[case] device append many rows K={k} V={v} n={n}")
    pool, kp, vp, hk, hv = _pool(nb, P, k, v, seed=6)
    dest = np.random.default_rng(3).permutation(nb * P)[:n]
    blocks, slots = (dest // P).astype(np.int32), (dest % P).astype(np.int32)
    dk_src, xk = _source_rows(n, 31, "f32")
    dv_src, xv = _source_rows(n, 37, "f32")
    pool.append_kv_device(dev(blocks), dev(slots), dk_src.cuda(), dv_src.cuda(), "f32")
    torch.cuda.synchronize()
    assert pool.device_error() == 0
    assert np.array_equal(kp.cpu().numpy(), pool_model.scatter_rows(hk, blocks, slots, encode.encode(xk, k)))
    assert np.array_equal(vp.cpu().numpy(), pool_model.scatter_rows(hv, blocks, slots, encode.encode(xv, v)))
    pool.destroy()


def test_append_device_bad_destinations_are_skipped():
    nb, P = 6, 32
    log("[case] device append with out-of-range destinations")
    pool, kp, vp, hk, hv = _pool(nb, P, "q8_0", "q4_0", seed=8)
    blocks = np.array([-1, nb, 0, 2, 5, 3], np.int32)
    slots = np.array([0, 0, P, -1, 7, 31], np.int32)
    good = np.array([False, False, False, False, True, True])
    dk_src, xk = _source_rows(6, 41, "f32")
    dv_src, xv = _source_rows(6, 43, "f32")
    pool.append_kv_device(dev(blocks), dev(slots), dk_src.cuda(), dv_src.cuda(), "f32")
    torch.cuda.synchronize()
    assert pool.device_error() & pb.DEVERR_APPEND
    assert pool.device_error() == 0                                  # read-and-clear
    refk = pool_model.scatter_rows(hk, blocks[good], slots[good], encode.encode(xk[good], "q8_0"))
    refv = pool_model.scatter_rows(hv, blocks[good], slots[good], encode.encode(xv[good], "q4_0"))
    assert np.array_equal(kp.cpu().numpy(), refk)
    assert np.array_equal(vp.cpu().numpy(), refv)
    # all rows valid: no error bit
    g = torch.from_numpy(good)
    pool.append_kv_device(dev(blocks[good]), dev(slots[good]), dk_src[g].contiguous().cuda(),
                          dv_src[g].contiguous().cuda(), "f32")
    torch.cuda.synchronize()
    assert pool.device_error() == 0
    pool.destroy()


@pytest.mark.parametrize("kv", [("q4_0", "q4_0"), ("bf16", "bf16"), ("q8_0", "q4_0")], ids=lambda p: f"K{p[0]}-V{p[1]}")
def test_fill_by_device_append_then_decode(kv):
    """The serving flow: K/V rows leave a projection as float32 on the device,
    a device append encodes them into pages taken from the allocator, and
    decode reads them back through the block table."""
    k, v = kv
    P, lens, T = 64, [700, 64, 1, 2049, 130], 2
    need = [(L + P - 1) // P for L in lens]
    nb = sum(need) + 3
    log(f"[case] fill by device append, decode K={k} V={v} lens={lens}")
    kp = torch.zeros((nb, 4, P, ROW_BYTES[k]), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((nb, 4, P, ROW_BYTES[v]), dtype=torch.uint8, device="cuda")
    pool = pb.Pool(nb, P, pb.kv_type(k, v), k_pool=kp, v_pool=vp, max_seqs=8, max_blocks_per_seq=max(need))
    table = np.full((len(lens), max(need)), -1, np.int32)
    blocks, slots = [], []
    for s, L in enumerate(lens):
        _, ix = pool.alloc(need[s])
        table[s, :need[s]] = ix
        for pos in range(L):
            blocks.append(table[s, pos // P])
            slots.append(pos % P)
    blocks, slots = np.array(blocks, np.int32), np.array(slots, np.int32)
    n = len(blocks)
    rng = np.random.default_rng(71)
    xk = rng.standard_normal((n, 4, 256)).astype(np.float32)
    xv = rng.standard_normal((n, 4, 256)).astype(np.float32)
    pool.append_kv_device(dev(blocks), dev(slots), dev(xk), dev(xv), "f32")
    torch.cuda.synchronize()
    assert pool.device_error() == 0
    hk = pool_model.scatter_rows(np.zeros((nb, 4, P, ROW_BYTES[k]), np.uint8), blocks, slots, encode.encode(xk, k))
    hv = pool_model.scatter_rows(np.zeros((nb, 4, P, ROW_BYTES[v]), np.uint8), blocks, slots, encode.encode(xv, v))
    assert np.array_equal(kp.cpu().numpy(), hk) and np.array_equal(vp.cpu().numpy(), hv)
    q = synth.normal((len(lens), T, 24, 256), seed=72)
    w = synth.Workload(q=q, k_pool=hk, v_pool=hv, block_table=table, seq_lens=np.array(lens, np.int32),
                       n_qtok=T, k_kind=k, v_kind=v, page_size=P, scale=1 / 16)
    out, _, err = run(w, dk=kp, dv=vp)
    assert err == 0
    ref, _ = attention.paged_decode(q, hk, hv, k, v, table, np.array(lens, np.int32), 1 / 16)
    parity(out, ref, what=f"device-appended K={k} V={v}")
    pool.destroy()
