"""Benchmark of one paged decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ragged|uniform|mtp|f16|serving|...]

A step is one pa_decode call -- plan, block-table walk, K/V stream, dequant,
QK^T, online softmax, PV, chunk epilogue, LSE merge -- over the ragged
131072 + 7 x 8192 Q4_0 workload (16-token pages, interleaved table), with
inputs resident in HBM.  The headline is cold: consecutive steps rotate over
replicas of the pools whose total exceeds twice the 256 MB last-level cache,
so K/V bytes come from HBM.  Prints one JSON line.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention-step ms, effective K/V GB/s (% HBM peak), paged÷contiguous ratio"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # dense fp16 / bf16 matrix peak
SPLIT_KERNEL = "split_mfma_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before each timed run (after --settle)")
    ap.add_argument("--workload", default="ragged",
                    choices=["ragged", "ragged_q8k_q4v", "uniform", "mtp", "f16", "serving", "prefill"],
                    help="ragged: 131072 + 7 x 8192 Q4_0 (the headline); ragged_q8k_q4v: same with Q8_0 K and Q4_0 V; "
                         "uniform: --nseq x 4096 Q4_0; mtp: one --ctx-position Q8_0 sequence (default 131072), --qtok "
                         "query tokens; f16: one 1024-position F16 sequence; serving: 128 BF16 streams of "
                         "512..8192 positions in 64-position pages over 16 consecutive steps, each step an append "
                         "of one K/V row per stream (see --append) followed by the decode; prefill: one "
                         "--ctx-position sequence (default 16384), Q8_0 K and Q4_0 V, whose last --qtok positions "
                         "are the new tokens (pa_prefill)")
    ap.add_argument("--qtok", type=int, default=4, help="query tokens for --workload mtp / prefill")
    ap.add_argument("--kv", default="q8_0", choices=["q8_0", "q4_0", "bf16", "f16"],
                    help="K and V encoding of --workload mtp (default q8_0)")
    ap.add_argument("--append", default="host", choices=["device", "host"],
                    help="serving: the per-step append of one row per stream; host: pa_append_kv (rows already "
                         "BF16-encoded in host memory, one packed upload through pinned staging and a scatter "
                         "kernel); device: pa_append_kv_device (float32 rows already on the GPU, encoded into the "
                         "pool's BF16 on the way in)")
    ap.add_argument("--ctx", type=int, default=None, help="context for --workload mtp (default 131072) and prefill "
                                                          "(default 16384)")
    ap.add_argument("--nseq", type=int, default=8, help="sequences of 4096 positions for --workload uniform")
    ap.add_argument("--replicas", type=int, default=0, help="pool replicas for cold timing (0: auto)")
    ap.add_argument("--plan", default="host", choices=["host", "device"],
                    help="host: the call also passes a host copy of seq_lens (pa_decode_ext.seq_lens_host), so the "
                         "split-K plan is computed on the host and travels with the launch; device: the kernels "
                         "compute it from the device seq_lens.  The other route is timed too and reported")
    ap.add_argument("--no-contiguous", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of back-to-back untimed steps before every timed run (on top of --warmup): "
                         "the clocks reach their steady state only after some milliseconds of continuous work")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="only sweep pa_read_bandwidth_probe_ex over its configurations (the measured read ceiling)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only time a plain 2 GiB device-to-device copy (read-bandwidth ceiling; also the "
                         "known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_ceiling(steps=20, nbytes=2 << 30):
    """Bandwidth of torch's device copy over `nbytes` (read nbytes + write nbytes)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes, "ms_per_copy": round(ms, 4),
            "read_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1), "read_plus_write_gbps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def read_ceiling(steps=20, nbytes=2 << 30):
    """HBM read rate of pa_read_bandwidth_probe (16-byte loads, every byte of
    `nbytes` read once) on this machine: the practical ceiling of the K/V stream,
    reported beside the 8 TB/s nominal peak (bench.py --ceiling-sweep times
    the probe's other configurations)."""
    import torch
    from paged_kv_attention_walk_amd import binding as pb
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(32 * n_cu, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pb.read_bandwidth_probe(a, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        pb.read_bandwidth_probe(a, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del a, sink
    return {"kernel": "pa_read_bandwidth_probe over 2 GiB (16-byte loads, 8 workgroups per CU, one load in flight "
                      "per lane: the fastest configuration of the sweep in profiles/read_ceiling_sweep.md)",
            "bytes_read": nbytes, "ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def ceiling_sweep(steps=10):
    """pa_read_bandwidth_probe_ex over workgroups per CU x loads in flight x
    access (grid-stride or per-workgroup slice) x load kind (registers or
    direct to LDS) on a 4 GiB buffer, then the best configurations on 2 and
    8 GiB.  Returns {"runs": [...], "best": {...}}."""
    import torch
    from paged_kv_attention_walk_amd import binding as pb
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(4 * 32 * n_cu, dtype=torch.int32, device="cuda")
    bufs = {gib: torch.ones((gib << 30) // 4, dtype=torch.int32, device="cuda") for gib in (2, 4, 8)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(buf, wgs, u, flags):
        for _ in range(2):
            pb.read_bandwidth_probe_ex(buf, sink, wgs, u, flags)
        e0.record()
        for _ in range(steps):
            pb.read_bandwidth_probe_ex(buf, sink, wgs, u, flags)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return round(buf.numel() * 4 / (ms * 1e-3) / 1e9, 1)

    runs = []
    for flags in (0, pb.PROBE_SLICE, pb.PROBE_LDS, pb.PROBE_SLICE | pb.PROBE_LDS):
        for wgs in (1, 2, 4, 8, 16, 32):
            for u in (1, 2, 4, 8, 16):
                runs.append({"gib": 4, "wgs_per_cu": wgs, "loads_in_flight": u,
                             "slice": bool(flags & pb.PROBE_SLICE), "lds": bool(flags & pb.PROBE_LDS),
                             "gbps": rate(bufs[4], wgs, u, flags)})
    top = sorted(runs, key=lambda r: -r["gbps"])[:4]
    for r in top:
        flags = (pb.PROBE_SLICE if r["slice"] else 0) | (pb.PROBE_LDS if r["lds"] else 0)
        for gib in (2, 8):
            runs.append(dict(r, gib=gib, gbps=rate(bufs[gib], r["wgs_per_cu"], r["loads_in_flight"], flags)))
    del bufs
    return {"runs": runs, "best": max(runs, key=lambda r: r["gbps"])}


def kernel_source_hash():
    """Hash of the code (comments and blank space removed) of the sources that
    decide what the split and merge kernels do and how they are launched."""
    import re
    h = hashlib.sha256()
    for f in ("pa_mfma.hip", "pa_kernels.hip", "pa_device.h", "pa_internal.h", "pa_host.cpp"):
        text = open(os.path.join(ROOT, "paged_kv_attention_walk_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload_name):
    """HBM traffic per launch measured with rocprofv3 counters, if the kernel
    source is unchanged since the counters were taken (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def synth_row_bytes(kind):
    return {"f16": 512, "bf16": 512, "q8_0": 272, "q4_0": 144}[kind]


def host_info():
    """CPU model, logical CPUs and ROCm version of the machine the bench runs on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    rocm = None
    for f in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            rocm = open(f).read().strip()
            break
        except OSError:
            continue
    import torch
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "rocm": rocm, "torch": torch.__version__,
            "torch_hip": getattr(torch.version, "hip", None)}


def cpu_baseline(w, seconds):
    """The float64 oracle, as it stands, on the whole workload (every
    sequence, all 24 query heads), repeated until `seconds` have passed (at
    least once).  Reported in K/V GB/s like the GPU value."""
    from threadpoolctl import threadpool_info
    from oracle import attention
    t0 = time.perf_counter()
    n = 0
    while True:
        attention.paged_decode(w["q"], w["k_pool"], w["v_pool"], w["k_kind"], w["v_kind"], w["block_table"],
                               w["seq_lens"], w["scale"])
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(w.kv_bytes * n / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole workload ({len(w['seq_lens'])} sequences, {int(sum(w['seq_lens']))} positions, "
                      f"24 query heads, {w['n_qtok']} token(s)), {n} pass(es) in {dt:.1f} s on the host; "
                      f"{os.cpu_count()} logical CPUs",
            "seconds_per_step": round(dt / n, 3)}


def load_profile(workload_name):
    """Split-kernel duration from the committed rocprofv3 kernel trace of the
    default bench command, if the kernel sources are unchanged since it was
    taken (else None): a cross-check of the live event timing."""
    p = os.path.join(ROOT, "profiles", f"trace_{workload_name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from paged_kv_attention_walk_amd import binding as pb
    from paged_kv_attention_walk_amd import synth

    torch.cuda.set_device(0)
    if args.ceiling:
        print(json.dumps({"copy_ceiling": copy_ceiling()}), flush=True)
        return
    if args.ceiling_sweep:
        print(json.dumps({"read_ceiling_sweep": ceiling_sweep()}), flush=True)
        return
    ceiling = read_ceiling()
    t_gen = time.perf_counter()
    if args.workload == "ragged":
        w = synth.config3()
    elif args.workload == "ragged_q8k_q4v":
        w = synth.ragged_mixed()
    elif args.workload == "uniform":
        w = synth.config2(n_seq=args.nseq)
    elif args.workload == "mtp":
        w = synth.config4(ctx=args.ctx or 131072, n_qtok=args.qtok, kind=args.kv)
    elif args.workload == "serving":
        w = synth.config5_rolling()
    elif args.workload == "prefill":
        w = synth.prefill_workload(ctx=args.ctx or 16384, n_qtok=args.qtok)
    else:
        w = synth.config1()
    print(f"[bench] workload {w['name']} generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    n_seq, T, P = len(w["seq_lens"]), w["n_qtok"], w["page_size"]
    kv = pb.kv_type(w["k_kind"], w["v_kind"])
    # serving: `roll` consecutive decode steps; step k appends one row per
    # stream at position L0 + k and decodes at L0 + k + 1 (pages fill up and
    # new ones start); the timed steps cycle through them
    roll = int(w.get("steps", 1))
    if roll > 1:
        base = w["seq_lens"].astype(np.int64)
        lens_steps = [(base + k + 1).astype(np.int32) for k in range(roll)]
    else:
        lens_steps = [w["seq_lens"]]
    row_kv = synth_row_bytes(w["k_kind"]) + synth_row_bytes(w["v_kind"])
    kv_bytes = float(np.mean([int(np.sum(x)) for x in lens_steps])) * 4 * row_kv
    pool_bytes = w["k_pool"].nbytes + w["v_pool"].nbytes
    reps = args.replicas or max(1, min(16, int(np.ceil(2 * 2 * 256e6 / pool_bytes))))
    dq = torch.from_numpy(w["q"]).cuda()
    dlens_steps = [torch.from_numpy(x).cuda() for x in lens_steps]
    k0 = torch.from_numpy(w["k_pool"]).cuda()
    v0 = torch.from_numpy(w["v_pool"]).cuda()
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(reps - 1)]
    bts = [torch.from_numpy(w["block_table"]).cuda() for _ in range(reps)]
    out = torch.empty((n_seq, T, 24, 256), device="cuda")
    prefill = args.workload == "prefill"
    nbytes = pb.prefill_workspace_size(n_seq, T, 0) if prefill else pb.workspace_size(n_seq, T, 0)
    ws = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device="cuda")
    bt_stride = w["block_table"].shape[1]
    nblocks = w["k_pool"].shape[0]

    def settle(calls, seconds):
        """Back-to-back steps for `seconds` of wall time before a timed run:
        the GPU's clocks reach their steady state only after some milliseconds
        of continuous work, whatever the untimed warm-up count."""
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(64):
                calls[i % len(calls)](None)
                i += 1
            torch.cuda.synchronize()
        return i

    def timed(calls, steps, warmup):
        """calls: list of callables taking an event pair or None.  After the
        settle phase and `warmup` untimed steps, times `steps` steps with no
        events (wall clock between two synchronisations, ms/step), then the
        same steps again with the split kernel's timing events attached to its
        dispatch (the kernel's execution time).  Returns (ms/step,
        split-kernel ms mean, median)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:          # create the events on this stream
            a.record()
            b.record()
        settle(calls, args.settle)
        for i in range(warmup):
            calls[i % len(calls)](None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            calls[i % len(calls)](None)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) * 1e3 / steps
        for i in range(steps):
            calls[i % len(calls)]((evs[i][0].cuda_event, evs[i][1].cuda_event))
        torch.cuda.synchronize()
        ks = [a.elapsed_time(b) for a, b in evs]
        return dt, float(np.mean(ks)), float(np.median(ks))

    lib = pb.lib()
    stream = torch.cuda.current_stream().cuda_stream

    # serving: every step first appends one new K/V row per stream at the
    # position the step adds, then decodes.  Default: pa_append_kv, the rows
    # already BF16-encoded in host memory, one packed upload through pinned
    # staging and a scatter kernel; --append device: pa_append_kv_device,
    # float32 rows already on the GPU encoded into the pool on the way in
    serving = args.workload == "serving"
    append = None
    if serving:
        nk, nv = synth.normal((n_seq, 4, 256), seed=505), synth.normal((n_seq, 4, 256), seed=506)
        h_k = np.ascontiguousarray(synth.encode(nk, w["k_kind"]))
        h_v = np.ascontiguousarray(synth.encode(nv, w["v_kind"]))
        xk, xv = torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda()
        dst = []                          # per step: (host block, host slot, device block, device slot)
        for k in range(roll):
            pos = lens_steps[k].astype(np.int64) - 1
            hb = w["block_table"][np.arange(n_seq), pos // P].astype(np.int32)
            hs = (pos % P).astype(np.int32)
            dst.append((hb, hs, torch.from_numpy(hb).cuda(), torch.from_numpy(hs).cuda()))
        append_pools = [pb.Pool(nblocks, P, kv, k_pool=kp, v_pool=vp, max_seqs=1, max_blocks_per_seq=bt_stride)
                        for kp, vp in pools]
        for ap_pool in append_pools:      # every page of the pool is in use (allocated through pa_alloc_blocks)
            ap_pool.alloc(nblocks)
        append = {"rows": n_seq, "steps_rolled": roll,
                  "src": "f32 on the device" if args.append == "device" else "bf16 rows in host memory",
                  "entry": "pa_append_kv_device" if args.append == "device" else "pa_append_kv",
                  "keep": (xk, xv, dst)}

    def make_call(kp, vp, bt, nb, pool=None, plan=args.plan, k=0):
        """Step k of the length cycle with every pointer and the ext struct
        prepared up front, so that the timed loop is one ctypes call per step
        (two with an append)."""
        ext = pb.make_ext(bt_stride, nb, w["scale"], None, ws, ws.numel() * 4,
                          seq_lens_host=lens_steps[k] if plan == "host" else None)
        ext_ref = ctypes.byref(ext)
        a = (dq.data_ptr(), kp.data_ptr(), vp.data_ptr(), bt.data_ptr() if bt is not None else None,
             dlens_steps[k].data_ptr(), n_seq, T, kv, P, out.data_ptr(), stream)
        ap = None
        if pool is not None:
            hb, hs, db, ds = dst[k]
            if args.append == "device":
                ap = (pool._h, n_seq, db.data_ptr(), ds.data_ptr(), xk.data_ptr(), xv.data_ptr(), pb.F32,
                      ws.data_ptr(), stream)
            else:
                ap = (pool._h, n_seq, hb.ctypes.data, hs.ctypes.data, h_k.ctypes.data, h_v.ctypes.data, stream)
        append_fn = lib.pa_append_kv_device if args.append == "device" else lib.pa_append_kv

        entry = lib.pa_prefill if prefill else lib.pa_decode

        def f(events):
            if ap is not None:
                st = append_fn(*ap)
                if st != pb.OK:
                    raise pb.PaError(st, "pa_append_kv_device" if args.append == "device" else "pa_append_kv")
            ext.split_events[0], ext.split_events[1] = (events if events else (None, None))
            st = entry(*a, ext_ref)
            if st != pb.OK:
                raise pb.PaError(st, "pa_prefill" if prefill else "pa_decode")
        f.keep = (ext, kp, vp, bt, pool)
        return f

    def cycle(make, rs):
        """Calls over replicas rs and the length steps: consecutive calls
        rotate the replicas, each replica walks the steps in order."""
        return [make(rs[i % len(rs)], (i // len(rs)) % roll) for i in range(len(rs) * roll)]

    def paged_calls(rs, with_append=True, plan=args.plan):
        return cycle(lambda r, k: make_call(pools[r][0], pools[r][1], bts[r], nblocks,
                                            append_pools[r] if (serving and with_append) else None, plan, k), rs)

    other = "device" if args.plan == "host" else "host"
    o_ms, o_k, _ = timed(paged_calls(list(range(reps)), plan=other), args.steps, args.warmup)
    res_other = out.clone()
    cold_ms, cold_k, cold_k_med = timed(paged_calls(list(range(reps))), args.steps, args.warmup)
    other_plan = {"plan": other, "ms_per_step": round(o_ms, 4), "split_kernel_ms": round(o_k, 4),
                  "bitwise_equal": bool(torch.equal(out.view(torch.int32), res_other.view(torch.int32)))}
    hot_ms, hot_k, _ = timed(paged_calls([0]), args.steps, args.warmup)
    decode_only_ms = None
    if serving:
        decode_only_ms, _, _ = timed(paged_calls(list(range(reps)), False), args.steps, args.warmup)
        append["ms_per_step_decode_only"] = round(decode_only_ms, 4)
        append["append_ms_est"] = round(cold_ms - decode_only_ms, 4)
    err = pb.device_error(ws)
    if err:
        raise RuntimeError(f"device error word {err}")
    res_paged = out.clone()

    contig = None
    if not args.no_contiguous:
        max_len = bt_stride * P
        # with appends, the pools now hold the appended rows (replica 0 has
        # walked every step of the cycle): copy those, up to the last step's
        # lengths
        hk = k0.cpu().numpy() if serving else w["k_pool"]
        hv = v0.cpu().numpy() if serving else w["v_pool"]
        kc = synth.contiguous_from_table(hk, w["block_table"], lens_steps[-1], max_len)
        vc = synth.contiguous_from_table(hv, w["block_table"], lens_steps[-1], max_len)
        del hk, hv
        # as many replicas as the paged pools: the step reads the same live
        # rows either way, so the same rotation keeps both cold
        creps = reps
        kc0 = torch.from_numpy(kc).cuda()
        vc0 = torch.from_numpy(vc).cuda()
        del kc, vc
        cpools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(creps - 1)]

        def contig_calls(rs):
            return cycle(lambda r, k: make_call(cpools[r][0], cpools[r][1], None, 0, None, args.plan, k), rs)
        c_ms, c_k, _ = timed(contig_calls(list(range(creps))), args.steps, args.warmup)
        # the last step of both runs used the same lengths when the step count is a multiple of the cycle
        same = bool(torch.equal(out.view(torch.int32), res_paged.view(torch.int32)))
        ch_ms, ch_k, _ = timed(contig_calls([0]), args.steps, args.warmup)
        contig = {"ms_per_step": round(c_ms, 4), "split_kernel_ms": round(c_k, 4), "replicas": creps,
                  "bitwise_equal_to_paged": same,
                  "hot": {"ms_per_step": round(ch_ms, 4), "split_kernel_ms": round(ch_k, 4)}}
        del cpools, kc0, vc0

    gbps = kv_bytes / (cold_ms * 1e-3) / 1e9
    achieved = kv_bytes / (cold_k * 1e-3) / 1e9
    # algorithmic flops: QK^T and PV, 2 x 2 x 256 per (query row, visible
    # key), the mean over the steps of the cycle like kv_bytes
    vis = np.mean([sum(max(0, min(int(L), int(L) - T + t + 1)) for L in ls for t in range(T)) for ls in lens_steps])
    flops = 4.0 * 256 * 24 * vis
    roofline = {"kernel": SPLIT_KERNEL, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(w["name"]),
                "split_kernel_ms_mean": round(cold_k, 5), "split_kernel_ms_median": round(cold_k_med, 5),
                "timing": "timing events attached to the split kernel's dispatch (its execution), mean over the "
                          "cold steps"}
    roofline["frac_of_read_ceiling"] = round(achieved / ceiling["gbps"], 4)
    prof = load_profile(w["name"])
    if prof is not None:      # the committed rocprofv3 trace of this command, same kernel sources
        pk = prof["split_kernel_avg_ns"] * 1e-6
        roofline["profile"] = {"file": f"profiles/trace_{w['name']}.json", "split_kernel_ms": round(pk, 5),
                               "frac": round(kv_bytes / (pk * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    tflops = flops / (cold_k * 1e-3) / 1e12
    if flops / kv_bytes > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):   # past the ridge point
        roofline.update({"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                         "kv_gbps": round(achieved, 2), "algorithmic_flops": flops})
    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle,
        "ms_per_step": round(cold_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w["name"] + (f"_{roll}steps" if roll > 1 else ""), "n_seq": n_seq,
                   "seq_lens": ("131072+7x8192" if args.workload.startswith("ragged") else
                                f"U{{512..8192}}+1..{roll} (each step appends one row per stream; {roll} steps)"
                                if serving else ",".join(str(int(x)) for x in w["seq_lens"])),
                   "entry": "pa_prefill" if prefill else "pa_decode",
                   "n_qtok": T, "kv": w["k_kind"] if w["k_kind"] == w["v_kind"] else f"K {w['k_kind']} V {w['v_kind']}",
                   "page_size": P, "q_heads": 24, "kv_heads": 4, "head_dim": 256, "kv_bytes": int(kv_bytes)},
        "attention_step_ms": round(cold_ms, 4),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        # the contiguous step has no append: compare it with the decode alone
        "paged_over_contiguous": (round(contig["ms_per_step"] / (decode_only_ms or cold_ms), 4) if contig else None),
        "paged_over_contiguous_hot": (round(contig["hot"]["ms_per_step"] / hot_ms, 4) if contig and not serving else None),
        "contiguous": contig,
        "append": append and {k: v for k, v in append.items() if k != "keep"},
        "hot": {"ms_per_step": round(hot_ms, 4), "split_kernel_ms": round(hot_k, 4),
                "gbps": round(kv_bytes / (hot_ms * 1e-3) / 1e9, 2)},
        "replicas": reps,
        "plan": args.plan,
        "other_plan": other_plan,
        "roofline": roofline,
        "read_ceiling": ceiling,
        "split_tflops": round(tflops, 2),
        "cpu_baseline": None,
        "host": host_info(),
    }
    if not args.no_cpu_baseline:
        w0 = synth.Workload(w)            # the first step's lengths (the same as w's without an append cycle)
        w0["seq_lens"] = lens_steps[0]
        line["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
