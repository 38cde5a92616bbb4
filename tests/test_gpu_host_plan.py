"""The host-planned route of pa_decode / pa_prefill (pa_decode_ext.seq_lens_host):
the split-K plan computed on the host from a host copy of seq_lens and carried
with the launch.  It must give bitwise the same outputs as the device-planned
call (same chunks, same summation order) and pass the oracle parity bar."""

import numpy as np
import pytest

from oracle import attention
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import log, parity, run
from test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu


def _oracle(w):
    return attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"],
                                  w["block_table"], w["seq_lens"], w["scale"])


def _same(a, b, what):
    assert np.array_equal(np.isnan(a), np.isnan(b)), what
    assert np.array_equal(np.nan_to_num(a, nan=0.0), np.nan_to_num(b, nan=0.0)), f"{what}: not bitwise equal"


CASES = [
    # (K, V, T, lens, page size, table)
    ("q4_0", "q4_0", 1, [131072 // 16, 8192 // 16] + [512] * 6, 16, "round_robin"),
    ("q4_0", "q4_0", 1, [0, 2, 63, 64, 65, 700, 1500, 3001], 48, "shuffled"),
    ("q8_0", "q4_0", 3, [5000, 17, 1, 0, 9000], 256, "shuffled"),
    ("bf16", "bf16", 2, [333, 2048, 17], 64, "shuffled"),
    ("f16", "q8_0", 8, [4000, 300, 8], 32, "shuffled"),
    ("q4_0", "q4_0", 5, [2000] * 3, 16, "round_robin"),
    # more work items than resident workgroups: the host plan hands out the
    # full-length chunks first, then the short last chunks longest first
    ("q4_0", "q8_0", 1, [int(x) for x in np.random.default_rng(31).integers(1, 4000, 200)] + [0, 1024, 2048, 3072],
     32, "shuffled"),
    ("bf16", "bf16", 2, [int(x) for x in np.random.default_rng(32).integers(500, 3000, 150)] + [4096] * 3 + [2304, 3456], 64,
     "shuffled"),
]


@pytest.mark.parametrize("engine", ["mfma", "valu"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"K{c[0]}-V{c[1]}-T{c[2]}-P{c[4]}")
def test_host_plan_bitwise_and_parity(case, engine):
    kk, vk, T, lens, P, table = case
    w = synth.make_workload(f"hp_{kk}_{vk}_{T}", lens, T, kk, vk, P, table=table, seed=401 + T)
    log(f"[case] host plan {kk}/{vk} T={T} P={P} lens={lens[:4]}.. {engine}")
    od, ld, ed = run(w, lse=True, engine=engine)
    oh, lh, eh = run(w, lse=True, engine=engine, host_plan=True)
    assert ed == 0 and eh == 0
    _same(od, oh, "out")
    _same(ld, lh, "lse")
    parity(oh, _oracle(w)[0], what=f"host plan {kk}/{vk} T={T}")


def test_host_plan_single_chunk_batch_skips_merge():
    # every sequence fits one chunk: the split kernel writes every row, no merge launch
    w = synth.make_workload("hp_single", [5, 50, 100, 0, 128], 1, "q4_0", "q4_0", 16, table="shuffled", seed=411)
    log("[case] host plan, one chunk per sequence")
    oh, lh, eh = run(w, lse=True, host_plan=True)
    od, ld, ed = run(w, lse=True)
    assert eh == 0 and ed == 0
    _same(od, oh, "out")
    ref, rlse = _oracle(w)
    parity(oh, ref, what="host plan single chunk")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lh))
    assert np.max(np.abs(lh[fin] - rlse[fin])) < 1e-3


@pytest.mark.parametrize("n_seq", [63, 65, 256, 257])
def test_host_plan_batch_limits(n_seq):
    # past 64 sequences the device plan is block-wide; 256 is the host plan's
    # limit, 257 falls back to the device plan
    rng = np.random.default_rng(421 + n_seq)
    lens = [int(x) for x in rng.integers(1, 600, size=n_seq)]
    lens[3] = 20000
    w = synth.make_workload(f"hp_n{n_seq}", lens, 1, "q8_0", "q4_0", 64, table="shuffled", seed=431)
    log(f"[case] host plan, {n_seq} sequences")
    od, _, ed = run(w)
    oh, _, eh = run(w, host_plan=True)
    assert ed == 0 and eh == 0
    _same(od, oh, "out")
    parity(oh, _oracle(w)[0], what=f"host plan n_seq={n_seq}")


def test_host_plan_corrupt_length():
    w = synth.make_workload("hp_corrupt", [700, 900, 60], 1, "q4_0", "q4_0", 16, seed=441)
    cap = w["block_table"].shape[1] * 16
    w["seq_lens"] = np.array([700, cap + 16, 60], dtype=np.int32)
    log("[case] host plan, a length beyond the table row")
    oh, _, eh = run(w, host_plan=True)
    od, _, ed = run(w)
    assert eh == 2 and ed == 2
    _same(od, oh, "out")
    assert np.isnan(oh[1]).all() and np.isfinite(oh[0]).all() and np.isfinite(oh[2]).all()


def test_host_plan_contiguous():
    w = synth.make_workload("hp_contig", [3000, 100, 1200], 2, "q4_0", "q4_0", 16, table="shuffled", seed=451)
    cap = w["block_table"].shape[1] * 16
    kc = synth.contiguous_from_table(w["k_pool"], w["block_table"], w["seq_lens"], cap)
    vc = synth.contiguous_from_table(w["v_pool"], w["block_table"], w["seq_lens"], cap)
    log("[case] host plan, contiguous storage")
    od, _, _ = run(w, contiguous=True, kc=kc, vc=vc)
    oh, _, _ = run(w, contiguous=True, kc=kc, vc=vc, host_plan=True)
    op, _, _ = run(w, host_plan=True)
    _same(od, oh, "contiguous")
    _same(op, oh, "paged vs contiguous")


@pytest.mark.parametrize("engine", ["mfma", "valu"])
def test_host_plan_prefill(engine):
    w = synth.make_workload("hp_prefill", [17, 40, 2500], 17, "q8_0", "q4_0", 64, seed=461)
    log(f"[case] host plan, prefill T=17 {engine}")
    od, ld, ed = run_prefill(w, lse=True, engine=engine)
    oh, lh, eh = run_prefill(w, lse=True, engine=engine, host_plan=True)
    assert ed == 0 and eh == 0
    _same(od, oh, "prefill out")
    _same(ld, lh, "prefill lse")
    parity(oh, _oracle(w)[0], what="host plan prefill")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_device_plan_equals_host_plan(seed):
    # the device-planned split kernel leaves its chunk length and each
    # sequence's first chunk in the workspace header (words 1 and 2 + s, up to
    # 1022 sequences); they must equal pa_split_plan's for this device's CU
    # count and the resident split workgroups per CU the library reports for
    # a one-token Q4_0 call
    import torch
    from paged_kv_attention_walk_amd import binding as pb
    rng = np.random.default_rng(470 + seed)
    n = int(rng.integers(2, 40))
    lens = [int(x) for x in rng.integers(0, 6000, size=n)]
    lens[0] = 20000
    w = synth.make_workload(f"hp_dev_{seed}", lens, 1, "q4_0", "q4_0", 16, table="shuffled", seed=481 + seed)
    log(f"[case] device plan header vs pa_split_plan, {n} sequences, seed {seed}")
    from gpu_util import workspace
    ws = workspace(n, 1)
    _, _, err = run(w, ws=ws)
    assert err == 0
    hdr = ws[:2 + n].cpu().numpy()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = pb.split_workgroups_per_cu("q4_0", 1)
    assert wgs >= 1
    chunk, items, first = pb.split_plan(w["seq_lens"], w["block_table"].shape[1] * 16, n_cu, wgs)
    assert hdr[1] == chunk, (hdr[1], chunk)
    assert list(hdr[2:2 + n]) == list(first[:n])


def test_occupancy_query_follows_the_launch_groups():
    # on the matrix-core path a call of 6..8 tokens runs as two groups of at
    # most four: the occupancy it plans with is the group kernel's; and the
    # kernels of up to five tokens with quantized V fit two workgroups per
    # compute unit (Q4_0 K with Q8_0 V only at one token)
    for kv in ("q8_0", "q4_0", "bf16", "f16", pb.kv_type("q8_0", "q4_0")):
        w = {t: pb.split_workgroups_per_cu(kv, t) for t in range(1, 9)}
        log(f"[occupancy] {kv}: {w}")
        assert w[6] == w[3] and w[7] == w[4] and w[8] == w[4], w
    for kv in ("q8_0", "q4_0", pb.kv_type("q8_0", "q4_0"), pb.kv_type("f16", "q4_0")):
        assert all(pb.split_workgroups_per_cu(kv, t) == 2 for t in range(1, 6)), kv
    assert pb.split_workgroups_per_cu("bf16", 1) == 2
