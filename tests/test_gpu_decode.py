"""GPU parity of pa_decode against the float64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import attention
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import TOL, dev, log, parity, run, workspace

pytestmark = pytest.mark.gpu

KINDS = ("f16", "bf16", "q8_0", "q4_0")


def _oracle(w, scale=None, bt=None, lens=None):
    return attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"],
                                  w["block_table"] if bt is None else bt,
                                  w["seq_lens"] if lens is None else lens,
                                  w["scale"] if scale is None else scale)


ENGINES = ["mfma", "valu"]


@pytest.mark.parametrize("engine", ENGINES)
def test_config1_parity(engine):
    w = synth.config1()
    log(f"[case] config1 f16 1x1024 p16 shuffled, {engine}")
    out, lse, err = run(w, lse=True, engine=engine)
    ref, rlse = _oracle(w)
    assert err == 0
    parity(out, ref, what="config1")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_small_ragged_parity(kind, T, engine):
    # several chunks per sequence (the plan's granule is 128 keys), ragged
    # tails, empty and shorter-than-T sequences, pages of 48 positions
    lens = [0, 2, 63, 64, 65, 700, 1500, 3001]
    w = synth.make_workload(f"small_{kind}_{T}", lens, T, kind, kind, 48, table="shuffled", seed=11 + T)
    log(f"[case] small ragged {kind} T={T} P=48 lens={lens} {engine}")
    out, lse, err = run(w, lse=True, engine=engine)
    ref, rlse = _oracle(w)
    assert err == 0
    parity(out, ref, what=f"small {kind} T={T}")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-3


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("kind", KINDS)
def test_unscaled_data_scale_one(kind, engine):
    # logits of order 16 exercise the max subtraction (config 1 data barely do)
    w = synth.make_workload(f"unscaled_{kind}", [333, 2048, 17], 2, kind, kind, 16, seed=21, scale=1.0)
    log(f"[case] unscaled {kind} {engine}")
    out, _, err = run(w, engine=engine)
    ref, _ = _oracle(w)
    parity(out, ref, what=f"unscaled {kind}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mag", [1e-3, 30.0])
def test_value_magnitudes(kind, mag, engine):
    # small block scales (f16 products near the subnormal range) and large ones
    w = synth.make_workload(f"mag_{kind}", [700, 90, 2500], 2, kind, kind, 32, seed=23,
                            value_scale=mag, q_scale=1.0 / mag, scale=1.0 / 16)
    log(f"[case] magnitude {mag} {kind} {engine}")
    out, _, err = run(w, engine=engine)
    parity(out, _oracle(w)[0], what=f"magnitude {mag} {kind}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("P", [16, 48, 128, 256, 512])
def test_paged_equals_contiguous_bitwise(P, engine):
    lens = [5 * P + 3, 2 * P, 1, 9 * P - 1]
    for kind in ("q4_0", "bf16", "q8_0", "f16"):
        T = {16: 2, 48: 5, 128: 8, 256: 3, 512: 6}[P]
        w = synth.make_workload(f"pc_{kind}_{P}", lens, T, kind, kind, P, table="shuffled", seed=P)
        log(f"[case] paged==contiguous {kind} P={P} T={T} {engine}")
        kc = synth.contiguous_from_table(w["k_pool"], w["block_table"], lens, w["block_table"].shape[1] * P)
        vc = synth.contiguous_from_table(w["v_pool"], w["block_table"], lens, w["block_table"].shape[1] * P)
        a, al, _ = run(w, lse=True, engine=engine)
        b, bl, _ = run(w, contiguous=True, kc=kc, vc=vc, lse=True, engine=engine)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert np.array_equal(al.view(np.uint32), bl.view(np.uint32))
        parity(a, _oracle(w)[0], what=f"pc {kind} P={P}")
        # three repeats are identical
        for _ in range(2):
            c, _, _ = run(w, engine=engine)
            assert np.array_equal(a.view(np.uint32), c.view(np.uint32))


def test_round_robin_vs_shuffled_bitwise():
    lens = [4096, 1000, 2500]
    a = synth.make_workload("rr", lens, 1, "q4_0", "q4_0", 16, table="round_robin", seed=3)
    log("[case] round robin vs shuffled placement")
    # same logical rows, different page placement
    kc = synth.contiguous_from_table(a["k_pool"], a["block_table"], lens, 4096)
    vc = synth.contiguous_from_table(a["v_pool"], a["block_table"], lens, 4096)
    oa, _, _ = run(a)
    ob, _, _ = run(a, contiguous=True, kc=kc, vc=vc)
    assert np.array_equal(oa.view(np.uint32), ob.view(np.uint32))
    parity(oa, _oracle(a)[0], what="round robin")


@pytest.mark.parametrize("engine", ENGINES)
def test_corrupt_table_and_length(engine):
    w = synth.make_workload("corrupt", [100, 900, 40, 3000], 2, "q8_0", "q8_0", 16, seed=31)
    log(f"[case] corrupt table entry / length {engine}")
    bt = w["block_table"].copy()
    bt[1, 3] = w["n_blocks"] + 7          # out of range
    bt[3, 100] = -5
    out, _, err = run(w, dbt=dev(bt), engine=engine)
    assert err & pb.DEVERR_TABLE
    ref, _ = _oracle(w, bt=bt)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[3]))
    parity(out[[0, 2]], ref[[0, 2]], what="intact sequences")
    lens = w["seq_lens"].copy()
    lens[2] = 16 * w["block_table"].shape[1] + 1
    lens[0] = -3
    out, _, err = run(w, dlens=dev(lens), engine=engine)
    assert err & pb.DEVERR_LENGTH
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(out[2]))
    parity(out[[1, 3]], _oracle(w)[0][[1, 3]], what="intact after bad lengths")


def test_registered_pool_path_without_ext():
    # pa_decode with ext == NULL: the pool is found from k_pool
    w = synth.make_workload("noext", [777, 64, 1], 1, "q4_0", "q4_0", 16, seed=41, n_blocks=80)
    log("[case] pa_decode without ext")
    dk, dv = dev(w["k_pool"]), dev(w["v_pool"])
    nb = w["k_pool"].shape[0]
    pool = pb.Pool(nb, 16, "q4_0", k_pool=dk, v_pool=dv, max_seqs=8, max_blocks_per_seq=w["block_table"].shape[1])
    out = torch.empty((3, 1, 24, 256), device="cuda")
    pb.decode(dev(w["q"]), dk, dv, dev(w["block_table"]), dev(w["seq_lens"]), 1, "q4_0", 16, out)
    assert pool.device_error() == 0
    torch.cuda.synchronize()
    parity(out.cpu().numpy(), _oracle(w)[0], what="no-ext path")
    pool.destroy()


def test_lse_matches_oracle_and_merge_of_halves():
    w = synth.make_workload("lse", [5000, 130], 4, "f16", "f16", 64, seed=51)
    log("[case] lse output")
    out, lse, _ = run(w, lse=True)
    ref, rlse = _oracle(w)
    parity(out, ref, what="lse case out")
    fin = np.isfinite(rlse)
    assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-4 * max(1.0, np.abs(rlse[fin]).max())


MIXED = [(k, v) for k in KINDS for v in KINDS if k != v]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("T", [1, 4, 7])
@pytest.mark.parametrize("kv", MIXED, ids=lambda p: f"K{p[0]}-V{p[1]}")
def test_mixed_types_parity(kv, T, engine):
    # K and V pools of different encodings (every off-diagonal pair)
    k, v = kv
    lens = [0, 3, 64, 129, 1000, 2047]
    w = synth.make_workload(f"mixed_{k}_{v}_{T}", lens, T, k, v, 48, table="shuffled", seed=61 + T)
    log(f"[case] mixed K={k} V={v} T={T} P=48 lens={lens} {engine}")
    out, lse, err = run(w, lse=True, engine=engine)
    ref, rlse = _oracle(w)
    assert err == 0
    parity(out, ref, what=f"mixed K={k} V={v} T={T}")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-3


@pytest.mark.parametrize("kv", [("q8_0", "q4_0"), ("f16", "q4_0"), ("q4_0", "bf16")], ids=lambda p: f"K{p[0]}-V{p[1]}")
@pytest.mark.parametrize("P", [16, 256])
def test_mixed_paged_equals_contiguous_bitwise(kv, P):
    k, v = kv
    lens = [3 * P + 5, P, 7 * P - 2]
    w = synth.make_workload(f"mpc_{k}_{v}_{P}", lens, 1, k, v, P, table="shuffled", seed=70 + P)
    log(f"[case] mixed paged==contiguous K={k} V={v} P={P}")
    cap = w["block_table"].shape[1] * P
    kc = synth.contiguous_from_table(w["k_pool"], w["block_table"], lens, cap)
    vc = synth.contiguous_from_table(w["v_pool"], w["block_table"], lens, cap)
    a, al, _ = run(w, lse=True)
    b, bl, _ = run(w, contiguous=True, kc=kc, vc=vc, lse=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(al.view(np.uint32), bl.view(np.uint32))
    parity(a, _oracle(w)[0], what=f"mixed pc K={k} V={v} P={P}")


def _plant_v_block(w, s, pos, d, code):
    """Sets V block 0 of sequence s's row `pos` (every KV head) to scale d and
    all 32 codes `code` (stored code for Q8_0; code + 8 nibbles for Q4_0)."""
    P = w["page_size"]
    page = int(w["block_table"][s][pos // P])
    v = w["v_pool"]
    dbytes = np.float16(d).tobytes()
    for h in range(4):
        row = v[page, h, pos % P]
        row[0:2] = np.frombuffer(dbytes, np.uint8)
        if w["v_kind"] == "q8_0":
            row[2:34] = np.uint8(code & 0xFF)
        else:
            nib = code + 8
            row[2:18] = np.uint8(nib | (nib << 4))


@pytest.mark.parametrize("v_kind,d_ok,d_over,code", [("q8_0", 515.5, 600.0, 127), ("q4_0", 8188.0, 9000.0, -8)])
def test_v_values_at_the_f16_range_limit(v_kind, d_ok, d_over, code):
    # The matrix-core path forms a quantised V value code x d as an f16 pair:
    # exact up to |code x d| = 65504, the f16 range (rows encoded from data in
    # the f16 range never exceed it).  At the limit the output matches the
    # oracle; past it the rows that see the value are non-finite (documented
    # in pa.h), the other sequence is unaffected, and the fp32 vector path
    # still matches the oracle.
    for d, finite in ((d_ok, True), (d_over, False)):
        w = synth.make_workload(f"vlimit_{v_kind}", [40, 70], 1, "q8_0", v_kind, 16, table="shuffled", seed=31)
        _plant_v_block(w, 0, 5, d, code)
        ref, _ = _oracle(w)
        log(f"[case] V {v_kind} value {code} x {d} = {abs(code) * d:.0f} (finite expected: {finite})")
        out, _, err = run(w)
        assert err == 0
        if finite:
            parity(out, ref, what=f"V {v_kind} at the f16 limit")
        else:
            assert not np.isfinite(out[0]).all()
            parity(out[1:], ref[1:], what=f"V {v_kind} past the limit, other sequence")
        out_v, _, err = run(w, engine="valu")
        assert err == 0
        parity(out_v, ref, what=f"V {v_kind} value {abs(code) * d:.0f}, fp32 vector path")


@pytest.mark.parametrize("qv,finite", [(40000.0, True), (50000.0, False)])
def test_q_at_the_f16_range_limit(qv, finite):
    # q x scale x log2(e) is split into f16 hi + lo for F16 / Q8_0 / Q4_0 K:
    # within the f16 range the result matches the oracle, past it the query
    # row's outputs are non-finite; the fp32 vector path matches either way
    w = synth.make_workload("qlimit", [40, 33], 1, "q8_0", "q8_0", 16, table="shuffled", seed=32,
                            scale=1.0, value_scale=1e-3)
    w["q"][0, 0, 7, 3] = qv                                 # sequence 0, query head 7
    ref, _ = _oracle(w)
    log(f"[case] q element {qv} x log2(e) = {qv * 1.4427:.0f} (finite expected: {finite})")
    out, _, err = run(w)
    assert err == 0
    if finite:
        parity(out, ref, what="q at the f16 limit")
    else:
        assert not np.isfinite(out[0, 0, 7]).all()
        parity(out[1:], ref[1:], what="q past the limit, other sequence")
    out_v, _, err = run(w, engine="valu")
    assert err == 0
    parity(out_v, ref, what=f"q {qv}, fp32 vector path")
