"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (pa_decode with an explicit workspace, the same plan), on the
whole output: uniform 8 x 4096 Q4_0; the ragged 131072 + 7 x 8192 Q4_0 step,
the single-sequence Q8_0 verify contexts and the 128-stream BF16 serving
steps (16 steps of pa_append_kv then decode; one device append then decode),
whose oracle output is assembled one
(sequence, KV head) block at a time to bound host memory.  Each block is also
held to the bar against its own RMS (stricter for long sequences, whose
outputs are small).  Also batches of more than 64 / 256 / 1022 sequences,
which take the block-wide plan, the device plan and the merge's own plan."""

import numpy as np
import pytest
import torch

from oracle import attention, encode, pool_model, quant
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity, run

pytestmark = pytest.mark.gpu


def _oracle_head(w, s, h, patch=None):
    """Oracle output [T][6][256] of sequence s, KV head h (its 6 query heads).
    ``patch``: a list of (position, K row bytes, V row bytes), each replacing
    one stored row."""
    L = int(w["seq_lens"][s])
    kb = pool_model.gather_rows(w["k_pool"][:, h:h + 1], w["block_table"][s], L)
    vb = pool_model.gather_rows(w["v_pool"][:, h:h + 1], w["block_table"][s], L)
    for pos, krow, vrow in (patch or []):
        kb[0, pos] = krow
        vb[0, pos] = vrow
    k = quant.decode(kb, w["k_kind"])
    v = quant.decode(vb, w["v_kind"])
    out, _ = attention.decode_sequence(w["q"][s][:, 6 * h:6 * h + 6], k, v, L, w["scale"])
    return out


def _bench_route(w, **kw):
    """The decode as the benchmark launches it (split-K plan computed on the
    host from a host copy of seq_lens), checked bitwise against the
    device-planned call of the same inputs."""
    out, lse, err = run(w, host_plan=True, **kw)
    out_d, lse_d, err_d = run(w, **kw)
    assert err == err_d
    assert np.array_equal(out.view(np.int32), out_d.view(np.int32)), "host- and device-planned outputs differ"
    if lse is not None:
        assert np.array_equal(lse.view(np.int32), lse_d.view(np.int32))
    return out, lse, err


def test_uniform_8x4096_q4_0_whole():
    w = synth.config2()
    log("[case] uniform 8 x 4096 Q4_0, whole output")
    out, _, err = _bench_route(w)
    assert err == 0
    ref, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q4_0", "q4_0", w["block_table"],
                                    w["seq_lens"], w["scale"])
    parity(out, ref, what="uniform 8x4096")


def _whole(out, w, what, patches=None):
    """The whole output against the oracle assembled block by block, then
    every (sequence, KV head) block against its own RMS."""
    n_seq = len(w["seq_lens"])
    ref = np.empty(out.shape, np.float64)
    for s in range(n_seq):
        for h in range(4):
            patch = patches(s, h) if patches else None
            ref[s][:, 6 * h:6 * h + 6] = _oracle_head(w, s, h, patch=patch)
    parity(out, ref, what=f"{what}, whole output")
    for s in range(n_seq):
        for h in range(4):
            blk = ref[s][:, 6 * h:6 * h + 6]
            if np.sqrt(np.mean(blk ** 2)) > 0:
                parity(out[s][:, 6 * h:6 * h + 6][None], blk[None], what=f"{what} seq {s} head {h}")


@pytest.mark.parametrize("engine", ["mfma", "valu"])
def test_ragged_128k_7x8k_q4_0_whole(engine):
    w = synth.config3()
    log(f"[case] ragged 131072 + 7 x 8192 Q4_0, whole output, {engine}")
    out, _, err = _bench_route(w, engine=engine)
    assert err == 0
    _whole(out, w, "ragged")


@pytest.mark.parametrize("ctx,T", [(32768, 1), (32768, 4), (131072, 1), (131072, 2), (131072, 3), (131072, 4), (131072, 5), (131072, 8), (32768, 6),
                                   (262144, 1), (262144, 3)])
def test_mtp_q8_0_whole(ctx, T):
    w = synth.config4(ctx=ctx, n_qtok=T)
    log(f"[case] Q8_0 single sequence ctx={ctx} T={T}, whole output")
    out, _, err = _bench_route(w)
    assert err == 0
    _whole(out, w, f"mtp ctx={ctx} T={T}")


def test_serving_128_streams_16_steps_whole():
    # the benchmark's serving cycle: 16 consecutive steps, each appending one
    # BF16 row per stream at its next position with pa_append_kv (one packed
    # upload and a scatter kernel), then decoding at the new lengths, so that
    # pages fill up and new pages start inside the window.  Each step's rows
    # differ.  Steps 0 and 15 are checked on the whole output, the others on
    # eight sequences.
    w = synth.config5_rolling()
    n_seq, P, roll = len(w["seq_lens"]), w["page_size"], w["steps"]
    base = w["seq_lens"].astype(np.int64)
    kp, vp = dev(w["k_pool"]), dev(w["v_pool"])
    nb = w["k_pool"].shape[0]
    pool = pb.Pool(nb, P, "bf16", k_pool=kp, v_pool=vp, max_seqs=1, max_blocks_per_seq=w["block_table"].shape[1])
    pool.alloc(nb)
    rows = []                               # per step: (positions, K rows, V rows)
    few = np.random.default_rng(15).choice(n_seq, size=8, replace=False)
    for k in range(roll):
        pos = base + k
        blocks = w["block_table"][np.arange(n_seq), pos // P].astype(np.int32)
        slots = (pos % P).astype(np.int32)
        krows = synth.encode(synth.normal((n_seq, 4, 256), seed=700 + k), "bf16")
        vrows = synth.encode(synth.normal((n_seq, 4, 256), seed=800 + k), "bf16")
        rows.append((pos, krows, vrows))
        log(f"[case] 128-stream BF16 serving, step {k}: pa_append_kv at L0+{k}, decode at L0+{k + 1}")
        assert pool.append_kv(blocks, slots, krows, vrows) == pb.OK
        wk = synth.Workload(w)
        wk["seq_lens"] = (base + k + 1).astype(np.int32)
        out, _, err = _bench_route(wk, dk=kp, dv=vp) if k in (0, roll - 1) else run(wk, dk=kp, dv=vp, host_plan=True)
        assert err == 0
        assert pool.device_error() == 0

        def patches(s, h, k=k):
            return [(int(rows[j][0][s]), rows[j][1][s][h], rows[j][2][s][h]) for j in range(k + 1)]
        if k in (0, roll - 1):
            _whole(out, wk, f"serving step {k}", patches=patches)
        else:
            for s in few:
                ref = np.stack([_oracle_head(wk, s, h, patch=patches(s, h)) for h in range(4)], axis=1)
                parity(out[s][None], ref.reshape(1, 1, 24, 256),
                       what=f"serving step {k} seq {s}")
    pool.destroy()


def test_serving_128_streams_device_append_then_decode_whole():
    # the other append route: float32 rows already on the device, encoded to
    # BF16 by pa_append_kv_device on the way into the pages
    w = synth.config5()
    n_seq, P = len(w["seq_lens"]), w["page_size"]
    log("[case] 128-stream BF16 serving step (device append + decode), whole output")
    last = w["seq_lens"].astype(np.int64) - 1
    blocks = w["block_table"][np.arange(n_seq), last // P].astype(np.int32)
    slots = (last % P).astype(np.int32)
    xk = synth.normal((n_seq, 4, 256), seed=505)
    xv = synth.normal((n_seq, 4, 256), seed=506)
    kp, vp = dev(w["k_pool"]), dev(w["v_pool"])
    pool = pb.Pool(w["k_pool"].shape[0], P, "bf16", k_pool=kp, v_pool=vp, max_seqs=1,
                   max_blocks_per_seq=w["block_table"].shape[1])
    pool.append_kv_device(dev(blocks), dev(slots), dev(xk), dev(xv), "f32")
    torch.cuda.synchronize()
    assert pool.device_error() == 0
    out, _, err = _bench_route(w, dk=kp, dv=vp)
    assert err == 0
    # the oracle's rows: the generated pages, with the appended row encoded by the oracle encoder
    _whole(out, w, "serving",
           patches=lambda s, h: [(int(last[s]), encode.encode(xk[s][h], "bf16"), encode.encode(xv[s][h], "bf16"))])
    pool.destroy()


@pytest.mark.parametrize("engine", ["mfma", "valu"])
@pytest.mark.parametrize("n_seq", [62, 63, 64, 65, 130, 1100])
def test_many_sequences_with_long_ones(n_seq, engine):
    # mostly short sequences and a few long ones, so the long ones split into
    # several chunks: the plan runs block-wide past 64 sequences, the host plan
    # stops at 256, and the merge plans for itself past the 1022 sequences its
    # header holds
    rng = np.random.default_rng(n_seq)
    lens = [int(x) for x in rng.integers(0, 200, size=n_seq)]
    for i in rng.choice(n_seq, size=4, replace=False):
        lens[int(i)] = int(rng.integers(15000, 25000))
    lens[0] = 0
    w = synth.make_workload(f"many_{n_seq}", lens, 2, "q4_0", "q8_0", 16, table="shuffled", seed=900 + n_seq)
    log(f"[case] {n_seq} sequences (4 long), {engine}")
    out, lse, err = _bench_route(w, lse=True, engine=engine)
    assert err == 0
    ref, rlse = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q4_0", "q8_0", w["block_table"],
                                       w["seq_lens"], w["scale"])
    parity(out, ref, what=f"{n_seq} sequences")
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rlse[fin])) < 1e-3


def test_600_sequences_three_tokens():
    # the plan's scan walks ten blocks of 64 sequences
    rng = np.random.default_rng(600)
    lens = [int(x) for x in rng.integers(0, 96, size=600)]
    for i in rng.choice(600, size=3, replace=False):
        lens[int(i)] = int(rng.integers(20000, 30000))
    w = synth.make_workload("many_600", lens, 3, "q8_0", "q4_0", 32, table="shuffled", seed=1600)
    log("[case] 600 sequences (3 long), T=3")
    out, _, err = run(w)
    assert err == 0
    ref, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q4_0", w["block_table"],
                                    w["seq_lens"], w["scale"])
    parity(out, ref, what="600 sequences")


def test_prefill_70_sequences():
    # prefill of 70 sequences, two of them long enough to split: every token
    # group of the split ones is merged, from the plan the split kernel leaves
    # in the workspace header
    rng = np.random.default_rng(70)
    lens = [int(x) for x in rng.integers(12, 160, size=70)]
    lens[5], lens[40] = 9000, 12000
    T = 12
    w = synth.make_workload("prefill_70", lens, T, "q4_0", "q4_0", 16, table="shuffled", seed=1700)
    log("[case] prefill, 70 sequences, T=12")
    n_seq = len(lens)
    n = pb.prefill_workspace_size(n_seq, T, torch.cuda.current_device())
    ws = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda")
    out = torch.empty((n_seq, T, 24, 256), dtype=torch.float32, device="cuda")
    ext = pb.make_ext(w["block_table"].shape[1], w["k_pool"].shape[0], w["scale"], None, ws, ws.numel() * 4)
    st = pb.prefill_status(dev(w["q"]), dev(w["k_pool"]), dev(w["v_pool"]), dev(w["block_table"]),
                           dev(w["seq_lens"]), n_seq, T, pb.kv_type("q4_0"), 16, out, ext=ext)
    assert st == pb.OK
    assert pb.device_error(ws) == 0
    ref, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q4_0", "q4_0", w["block_table"],
                                    w["seq_lens"], w["scale"])
    parity(out.cpu().numpy(), ref, what="prefill 70 sequences")


def test_prefill_1100_sequences():
    # prefill past the 1022 sequences the workspace header holds: the merge
    # computes the plan for itself, for every token group of the long ones
    rng = np.random.default_rng(1100)
    lens = [int(x) for x in rng.integers(10, 40, size=1100)]
    for i in rng.choice(1100, size=3, replace=False):
        lens[int(i)] = int(rng.integers(9000, 14000))
    T = 10
    w = synth.make_workload("prefill_1100", lens, T, "q8_0", "q4_0", 16, table="shuffled", seed=1701)
    log("[case] prefill, 1100 sequences (3 long), T=10")
    n_seq = len(lens)
    n = pb.prefill_workspace_size(n_seq, T, torch.cuda.current_device())
    ws = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda")
    out = torch.empty((n_seq, T, 24, 256), dtype=torch.float32, device="cuda")
    ext = pb.make_ext(w["block_table"].shape[1], w["k_pool"].shape[0], w["scale"], None, ws, ws.numel() * 4)
    st = pb.prefill_status(dev(w["q"]), dev(w["k_pool"]), dev(w["v_pool"]), dev(w["block_table"]),
                           dev(w["seq_lens"]), n_seq, T, pb.kv_type("q8_0", "q4_0"), 16, out, ext=ext)
    assert st == pb.OK
    assert pb.device_error(ws) == 0
    ref, _ = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], "q8_0", "q4_0", w["block_table"],
                                    w["seq_lens"], w["scale"])
    parity(out.cpu().numpy(), ref, what="prefill 1100 sequences")
