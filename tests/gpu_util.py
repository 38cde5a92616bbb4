"""Helpers for GPU tests: device upload, a decode call through the C ABI with
an explicit workspace, and the parity measure (max |gpu - oracle| over the
call's output against the oracle output's RMS, also per sequence)."""

import sys

import numpy as np
import torch

from paged_kv_attention_walk_amd import binding as pb

TOL = 2e-3   # max abs error <= TOL * RMS(oracle output), fp32 accumulation


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def workspace(n_seq, n_qtok):
    n = pb.workspace_size(n_seq, n_qtok, torch.cuda.current_device())
    ws = torch.zeros(n // 4 + 64, dtype=torch.int32, device="cuda")
    # 256-byte alignment of the base is what the ABI asks; torch gives >= 512.
    assert ws.data_ptr() % 256 == 0
    return ws


ENGINES = {"mfma": 0, "valu": pb.DECODE_VECTOR_REFERENCE}


def run(w, *, contiguous=False, kc=None, vc=None, scale=None, lse=False, ws=None, dq=None, dk=None, dv=None,
        dbt=None, dlens=None, out=None, events=None, stream=None, engine="mfma", host_plan=False):
    """Decode workload ``w`` (synth.Workload) through pa_decode with an ext.
    With ``host_plan`` the ext carries a host copy of seq_lens (the plan is
    computed on the host).  Returns (out np.float32, lse np.float32 or None,
    error word)."""
    n_seq = len(w["seq_lens"])
    T = w["n_qtok"]
    P = w["page_size"]
    kv = pb.kv_type(w["k_kind"], w["v_kind"])
    dq = dev(w["q"]) if dq is None else dq
    dlens = dev(w["seq_lens"].astype(np.int32)) if dlens is None else dlens
    if contiguous:
        dk = dev(kc) if dk is None else dk
        dv = dev(vc) if dv is None else dv
        bt = None
        bt_stride = kc.shape[2] // P
        nblocks = 0
    else:
        dk = dev(w["k_pool"]) if dk is None else dk
        dv = dev(w["v_pool"]) if dv is None else dv
        bt = dev(w["block_table"].astype(np.int32)) if dbt is None else dbt
        bt_stride = w["block_table"].shape[1]
        nblocks = w["k_pool"].shape[0]
    out = torch.empty((n_seq, T, 24, 256), dtype=torch.float32, device="cuda") if out is None else out
    lse_t = torch.empty((n_seq, T, 24), dtype=torch.float32, device="cuda") if lse else None
    ws = workspace(n_seq, T) if ws is None else ws
    ext = pb.make_ext(bt_stride, nblocks, w["scale"] if scale is None else scale, lse_t, ws, ws.numel() * 4,
                      split_events=events, flags=ENGINES[engine],
                      seq_lens_host=w["seq_lens"] if host_plan else None)
    pb.decode(dq, dk, dv, bt, dlens, T, kv, P, out, ext=ext, stream=stream)
    err = pb.device_error(ws, stream=stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse_t.cpu().numpy() if lse else None), err


def parity(got, ref, tol=TOL, what=""):
    """Max abs error vs tol * RMS(ref), overall and per sequence.  Returns the
    overall ratio err/RMS.  NaN positions must agree."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_r = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_r), f"{what}: NaN pattern differs"
    fin = ~nan_r
    if not fin.any():
        return 0.0
    rms = np.sqrt(np.mean(ref[fin] ** 2))
    err = np.abs(got[fin] - ref[fin]).max()
    worst = []
    for s in range(ref.shape[0]):
        f = fin[s]
        if not f.any():
            continue
        rs = np.sqrt(np.mean(ref[s][f] ** 2))
        es = np.abs(got[s][f] - ref[s][f]).max()
        worst.append((es / rs if rs > 0 else es, s))
    worst.sort(reverse=True)
    log(f"[parity] {what}: max|err|={err:.3e} rms={rms:.3e} ratio={err / rms if rms > 0 else err:.3e} "
        f"worst seq ratio={worst[0][0]:.3e} (seq {worst[0][1]})" if worst else "")
    if rms == 0:
        assert err == 0, what
        return 0.0
    assert err <= tol * rms, f"{what}: max|err| {err:.3e} > {tol} * rms {rms:.3e}"
    return err / rms
