"""pa_decode_scratch: the decode step with its workspace in the library's
static device buffer (no allocation, no workspace argument).  Through the C
ABI, its output must equal pa_decode's (same kernels, same plan: bitwise) on
two calls in a row, the second smaller, and both must meet the oracle bar;
the buffer's error word is cleared per call; sizes past the buffer are
refused before anything runs."""

import numpy as np
import pytest
import torch

from oracle import attention
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity, run

pytestmark = pytest.mark.gpu


def _scratch_call(w, *, dk=None, dv=None, dbt=None, dlens=None, host_plan=False):
    n_seq, T, P = len(w["seq_lens"]), w["n_qtok"], w["page_size"]
    kv = pb.kv_type(w["k_kind"], w["v_kind"])
    dq = dev(w["q"])
    dk = dev(w["k_pool"]) if dk is None else dk
    dv = dev(w["v_pool"]) if dv is None else dv
    dbt = dev(w["block_table"].astype(np.int32)) if dbt is None else dbt
    dlens = dev(w["seq_lens"].astype(np.int32)) if dlens is None else dlens
    out = torch.full((n_seq, T, 24, 256), 7.0, dtype=torch.float32, device="cuda")
    ext = pb.make_ext(w["block_table"].shape[1], w["k_pool"].shape[0], w["scale"],
                      seq_lens_host=w["seq_lens"] if host_plan else None)
    st = pb.decode_scratch_status(dq, dk, dv, dbt, dlens, n_seq, T, kv, P, out, None, ext)
    assert st == pb.OK, st
    err = pb.scratch_device_error()
    torch.cuda.synchronize()
    return out.cpu().numpy(), err


@pytest.mark.parametrize("host_plan", [False, True])
def test_scratch_decode_equals_pa_decode_two_calls(host_plan):
    torch.cuda.set_device(0)
    big = synth.make_workload("scratch_big", [9000, 17, 0, 4100, 640, 33, 2500, 1], 2, "q4_0", "q4_0", 16,
                              table="shuffled", seed=801)
    small = synth.make_workload("scratch_small", [300, 1, 77], 1, "q8_0", "q4_0", 48, table="shuffled", seed=802)
    for name, w in (("big", big), ("small", small)):
        log(f"[case] pa_decode_scratch {name} host_plan={host_plan} lens={list(w['seq_lens'])}")
        got, err = _scratch_call(w, host_plan=host_plan)
        assert err == 0
        want, _, err2 = run(w, host_plan=host_plan)
        assert err2 == 0
        assert np.array_equal(got.view(np.int32), want.view(np.int32)), f"{name}: differs from pa_decode"
        ref, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"],
                                        w["block_table"], w["seq_lens"], w["scale"])
        parity(got, ref, what=f"pa_decode_scratch {name}")


def test_scratch_error_word_is_per_call_and_large_sizes_are_refused():
    torch.cuda.set_device(0)
    w = synth.make_workload("scratch_err", [200, 90], 1, "q8_0", "q8_0", 16, table="shuffled", seed=803)
    bad = w["seq_lens"].copy()
    bad[1] = w["block_table"].shape[1] * 16 + 5                # longer than the table row: error bit 2
    log("[case] pa_decode_scratch corrupt length, then a clean call")
    out, err = _scratch_call(w, dlens=dev(bad.astype(np.int32)))
    assert err == pb.DEVERR_LENGTH
    assert np.isnan(out[1]).all() and not np.isnan(out[0]).any()
    _, err = _scratch_call(w)
    assert err == 0                                            # cleared by the next call
    # a call whose workspace would exceed the static buffer is refused before
    # anything is enqueued (the output keeps its bytes)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_seq = 4096
    need = pb.workspace_size(n_seq, 8, 0)
    assert need > pb.SCRATCH_BYTES, (need, n_cu)
    out = torch.full((4, 8, 24, 256), 3.0, device="cuda")
    ext = pb.make_ext(8, 64, 1 / 16)
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    st = pb.decode_scratch_status(out, z, z, z, z, n_seq, 8, pb.kv_type("q4_0"), 16, out, None, ext)
    assert st == pb.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out == 3.0).all()
