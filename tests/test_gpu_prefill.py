"""GPU parity of pa_prefill (paged chunked prefill: more query tokens than a
decode step, taken in token groups) against the float64 oracle, through the
C ABI."""

import numpy as np
import pytest
import torch

from oracle import attention
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity

pytestmark = pytest.mark.gpu

ENGINES = {"mfma": 0, "valu": pb.DECODE_VECTOR_REFERENCE}


def run_prefill(w, *, engine="mfma", contiguous=False, kc=None, vc=None, dbt=None, lse=False, scale=None,
                host_plan=False):
    n_seq, T, P = len(w["seq_lens"]), w["n_qtok"], w["page_size"]
    kv = pb.kv_type(w["k_kind"], w["v_kind"])
    dq = dev(w["q"])
    dlens = dev(w["seq_lens"].astype(np.int32))
    if contiguous:
        dk, dv, bt = dev(kc), dev(vc), None
        bt_stride, nb = kc.shape[2] // P, 0
    else:
        dk, dv = dev(w["k_pool"]), dev(w["v_pool"])
        bt = dev(w["block_table"].astype(np.int32)) if dbt is None else dbt
        bt_stride, nb = w["block_table"].shape[1], w["k_pool"].shape[0]
    out = torch.empty((n_seq, T, 24, 256), dtype=torch.float32, device="cuda")
    lse_t = torch.empty((n_seq, T, 24), dtype=torch.float32, device="cuda") if lse else None
    n = pb.prefill_workspace_size(n_seq, T, torch.cuda.current_device())
    ws = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda")
    ext = pb.make_ext(bt_stride, nb, w["scale"] if scale is None else scale, lse_t, ws, ws.numel() * 4,
                      flags=ENGINES[engine], seq_lens_host=w["seq_lens"] if host_plan else None)
    st = pb.prefill_status(dq, dk, dv, bt, dlens, n_seq, T, kv, P, out, ext=ext)
    assert st == pb.OK, st
    err = pb.device_error(ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse_t.cpu().numpy() if lse else None), err


def _oracle(w, bt=None):
    return attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"],
                                  w["block_table"] if bt is None else bt, w["seq_lens"], w["scale"])


CASES = [
    # (kinds, T, lens, page size)
    (("q4_0", "q4_0"), 9, [0, 5, 9, 700, 3001], 16),          # empty, L < T, L == T (a fresh prompt)
    (("q8_0", "q4_0"), 17, [17, 40, 2500], 64),
    (("bf16", "bf16"), 64, [64, 1000, 130], 48),
    (("f16", "q8_0"), 100, [100, 2100], 256),
    (("q4_0", "bf16"), 23, [1, 23, 1500, 777], 32),
    (("q8_0", "q8_0"), 10, [10, 3000, 6], 16),             # groups of four and a rest of two
]


@pytest.mark.parametrize("engine", list(ENGINES))
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"K{c[0][0]}-V{c[0][1]}-T{c[1]}")
def test_prefill_parity(case, engine):
    (k, v), T, lens, P = case
    w = synth.make_workload(f"prefill_{k}_{v}_{T}", lens, T, k, v, P, table="shuffled", seed=300 + T)
    log(f"[case] prefill K={k} V={v} T={T} P={P} lens={lens} {engine}")
    out, lse, err = run_prefill(w, engine=engine, lse=True)
    ref, rlse = _oracle(w)
    assert err == 0
    parity(out, ref, what=f"prefill K={k} V={v} T={T}")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-3


def test_prefill_unscaled_logits():
    # logits of order 16: the max subtraction and the chunk merge both matter
    w = synth.make_workload("prefill_unscaled", [300, 4096], 40, "q8_0", "q8_0", 64, seed=311, scale=1.0)
    log("[case] prefill unscaled q8_0 T=40")
    out, _, err = run_prefill(w)
    assert err == 0
    parity(out, _oracle(w)[0], what="prefill unscaled")


@pytest.mark.parametrize("P", [16, 256])
def test_prefill_paged_equals_contiguous_bitwise(P):
    lens = [4 * P + 3, 33, 9 * P - 1]
    w = synth.make_workload(f"prefill_pc_{P}", lens, 33, "q4_0", "q8_0", P, table="shuffled", seed=320 + P)
    log(f"[case] prefill paged == contiguous P={P}")
    cap = w["block_table"].shape[1] * P
    kc = synth.contiguous_from_table(w["k_pool"], w["block_table"], lens, cap)
    vc = synth.contiguous_from_table(w["v_pool"], w["block_table"], lens, cap)
    a, al, _ = run_prefill(w, lse=True)
    b, bl, _ = run_prefill(w, contiguous=True, kc=kc, vc=vc, lse=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(al.view(np.uint32), bl.view(np.uint32))
    c, _, _ = run_prefill(w)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))          # repeatable
    parity(a, _oracle(w)[0], what=f"prefill pc P={P}")


def test_prefill_corrupt_table():
    w = synth.make_workload("prefill_corrupt", [500, 900, 60], 12, "q4_0", "q4_0", 16, seed=331)
    log("[case] prefill corrupt table entry")
    bt = w["block_table"].copy()
    bt[1, 7] = w["n_blocks"] + 3
    out, _, err = run_prefill(w, dbt=dev(bt))
    assert err & pb.DEVERR_TABLE
    ref, _ = _oracle(w, bt=bt)
    assert np.all(np.isnan(out[1]))
    parity(out[[0, 2]], ref[[0, 2]], what="prefill intact sequences")


def test_prefill_rows_equal_decode_of_prefixes():
    # token t of a T-token prefill attends exactly what a one-token decode at
    # length L - T + t + 1 attends (parity with the oracle on both sides)
    L, T = 1200, 20
    w = synth.make_workload("prefill_prefix", [L], T, "q8_0", "q4_0", 16, table="shuffled", seed=341)
    log("[case] prefill rows vs one-token decodes")
    out, _, _ = run_prefill(w)
    ref, _ = _oracle(w)
    parity(out, ref, what="prefill vs oracle")
    for t in (0, 7, 8, 19):
        lt = L - T + t + 1
        one = attention.paged_decode(w["q"][:, t:t + 1], w["k_pool"], w["v_pool"], "q8_0", "q4_0",
                                     w["block_table"], np.array([lt], np.int32), w["scale"])[0]
        parity(out[:, t:t + 1], one, what=f"prefill token {t} vs one-token oracle")
