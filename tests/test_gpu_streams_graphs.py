"""pa_decode under the ways a serving loop drives it: two streams at once,
each with its own workspace, and a captured HIP graph replayed with new
queries.  Every result must be bitwise the eager single-stream result of the
same inputs (the kernels and the plan do not depend on how they were
launched), and the device error word must stay clear."""

import numpy as np
import pytest
import torch

from oracle import attention
from paged_kv_attention_walk_amd import binding as pb
from paged_kv_attention_walk_amd import synth
from gpu_util import dev, log, parity, workspace

pytestmark = pytest.mark.gpu


class _Call:
    """Device-resident inputs of one decode workload and its launch."""

    def __init__(self, w, host_plan):
        self.w = w
        self.n, self.T, self.P = len(w["seq_lens"]), w["n_qtok"], w["page_size"]
        self.kv = pb.kv_type(w["k_kind"], w["v_kind"])
        self.dq = dev(w["q"])
        self.dk, self.dv = dev(w["k_pool"]), dev(w["v_pool"])
        self.dbt = dev(w["block_table"].astype(np.int32))
        self.dlens = dev(w["seq_lens"].astype(np.int32))
        self.ws = workspace(self.n, self.T)
        self.ext = pb.make_ext(w["block_table"].shape[1], w["k_pool"].shape[0], w["scale"], None, self.ws,
                               self.ws.numel() * 4, seq_lens_host=w["seq_lens"] if host_plan else None)

    def out(self):
        return torch.full((self.n, self.T, 24, 256), 7.0, dtype=torch.float32, device="cuda")

    def launch(self, out, stream=None):
        pb.decode(self.dq, self.dk, self.dv, self.dbt, self.dlens, self.T, self.kv, self.P, out, ext=self.ext,
                  stream=stream)

    def error(self):
        return pb.device_error(self.ws)


def _workloads():
    a = synth.make_workload("sg_a", [4096, 700, 1, 0, 2500], 1, "q4_0", "q4_0", 16, table="shuffled", seed=1201)
    b = synth.make_workload("sg_b", [3000, 9000, 64], 3, "q8_0", "q8_0", 256, table="shuffled", seed=1202)
    return a, b


@pytest.mark.parametrize("host_plan", [False, True], ids=["device_plan", "host_plan"])
def test_two_streams_at_once_bitwise(host_plan):
    wa, wb = _workloads()
    ca, cb = _Call(wa, host_plan), _Call(wb, host_plan)
    ref_a, ref_b = ca.out(), cb.out()
    ca.launch(ref_a)
    cb.launch(ref_b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()      # default priority
    outs = []
    for _ in range(6):                                      # no host wait between the launches
        oa, ob = ca.out(), cb.out()
        torch.cuda.synchronize()
        ca.launch(oa, stream=s1)
        cb.launch(ob, stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for i, (oa, ob) in enumerate(outs):
        assert torch.equal(oa, ref_a), f"stream 1, launch {i}"
        assert torch.equal(ob, ref_b), f"stream 2, launch {i}"
    assert ca.error() == 0 and cb.error() == 0
    log(f"[streams] 6 x 2 concurrent launches equal the eager ones ({'host' if host_plan else 'device'} plan)")


@pytest.mark.parametrize("host_plan", [False, True], ids=["device_plan", "host_plan"])
def test_graph_replay_with_new_queries_bitwise(host_plan):
    wa, _ = _workloads()
    c = _Call(wa, host_plan)
    out_g = c.out()
    # capture on a side stream (torch's graph capture), after a warm-up
    # launch so that every lazily initialised piece of the library exists
    warm = c.out()
    c.launch(warm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.launch(out_g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1203)
    for i in range(4):
        q = rng.standard_normal(wa["q"].shape).astype(np.float32) * (1.0 + i)
        c.dq.copy_(torch.from_numpy(q).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = c.out()
        c.launch(eager)                                     # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i} differs from the eager call"
    assert c.error() == 0
    ref = attention.paged_decode(q, wa["k_pool"], wa["v_pool"], wa["k_kind"], wa["v_kind"], wa["block_table"],
                                 wa["seq_lens"], wa["scale"])[0]
    parity(out_g.cpu().numpy(), ref, what="graph replay")


def test_graph_replay_of_the_no_alloc_entry_point():
    wa, _ = _workloads()
    c = _Call(wa, True)
    ext = pb.make_ext(wa["block_table"].shape[1], wa["k_pool"].shape[0], wa["scale"], seq_lens_host=wa["seq_lens"])

    def launch(out):
        st = pb.decode_scratch_status(c.dq, c.dk, c.dv, c.dbt, c.dlens, c.n, c.T, c.kv, c.P, out, None, ext)
        assert st == pb.OK, st

    warm = c.out()
    launch(warm)
    torch.cuda.synchronize()
    out_g = c.out()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(out_g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1204)
    for i in range(3):
        c.dq.copy_(torch.from_numpy(rng.standard_normal(wa["q"].shape).astype(np.float32)).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = c.out()
        c.launch(eager)                                     # pa_decode with a workspace: same kernels and plan
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {i} of pa_decode_scratch differs from pa_decode"


def test_graph_replay_device_plan_follows_new_lengths():
    # the device plan reads seq_lens when the kernels run, so one capture
    # serves decode steps whose lengths grow (the grid depends on n_seq only)
    lens_max = np.array([4099, 703, 4, 3, 2503], np.int32)
    w = synth.make_workload("sg_grow", lens_max, 1, "q4_0", "q8_0", 16, table="shuffled", seed=1205)
    c = _Call(w, False)
    lens0 = lens_max - 3
    c.dlens.copy_(torch.from_numpy(lens0).cuda())
    warm = c.out()
    c.launch(warm)
    torch.cuda.synchronize()
    out_g = c.out()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.launch(out_g)
    torch.cuda.synchronize()
    for k in range(4):
        lens = lens0 + k
        c.dlens.copy_(torch.from_numpy(lens).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = c.out()
        c.launch(eager)
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"step {k}: replay differs from the eager call"
        ref = attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"], w["block_table"],
                                     lens, w["scale"])[0]
        parity(out_g.cpu().numpy(), ref, what=f"graph replay, lengths + {k}")
    assert c.error() == 0
