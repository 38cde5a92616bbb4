"""Plain float64 decode attention over paged K/V (oracle; test infrastructure
only).

Method (lucebox#555, Summary; llama.cpp-PR2, split-K decode commit): decode
attention with head size D = 256 and grouped queries (Hq = 24 query heads over
Hkv = 4 KV heads), one to four new query tokens per sequence, K/V read through
a block table.  Split-K over context chunks with a stable log-sum-exp merge is
exact (llama.cpp-PR2, log-sum-exp output commit: attending parts separately
and merging the normalised results reproduces the whole), so the oracle is
one softmax per query row over all its visible keys.

Readings where the pages leave a step open:

* query head h reads KV head h // (Hq/Hkv): consecutive query heads share a
  KV head;
* the T new tokens' K/V rows are already stored; with ``L`` stored rows, new
  token t sits at position L - T + t and sees keys 0 .. L - T + t (causal
  mask among the new tokens);
* softmax scale defaults to 1/sqrt(D) = 1/16;
* log-sum-exp is natural-log, max + ln(sum of exp(logit - max)), over the
  scaled, masked logits (llama.cpp-PR2, log-sum-exp output commit);
* a row with no visible key (empty sequence, or L < T) outputs exactly 0 and
  has lse = -inf (lucebox#555, Validation, covers empty sequences;
  llama.cpp-PR2, pd_combine fix: an all-masked row is 0, not 0/0);
* a sequence whose table points outside the pool (or whose length exceeds the
  table row) outputs NaN for all its rows; lucebox#555, Validation, tests
  corrupt block-table bounds guards but does not say what they return.
"""

import numpy as np

from . import quant, pool_model

HEAD_DIM = 256
N_Q_HEADS = 24
N_KV_HEADS = 4


def attend_one(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, n_visible,
               scale: float):
    """Softmax attention of ``q_rows`` [R][D] over the first ``n_visible[r]``
    rows of ``k``/``v`` [L][D] (float64).  Returns (out [R][D], lse [R])."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    R = q_rows.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    if k.shape[0] == 0:
        return out, lse
    logits = scale * (q_rows @ k.T)                             # [R][L]
    for r in range(R):
        n = int(n_visible[r])
        if n <= 0:
            continue                                            # no key: 0, -inf
        s = logits[r, :n]
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        out[r] = (e @ v[:n]) / l
        lse[r] = m + np.log(l)
    return out, lse


def decode_sequence(q_seq: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray,
                    seq_len: int, scale: float):
    """One sequence.  ``q_seq`` [T][Hq][D] fp32/fp64; ``k_rows``/``v_rows``
    decoded float64 [Hkv][L][D].  Returns (out [T][Hq][D], lse [T][Hq])."""
    T, Hq, D = q_seq.shape
    Hkv = k_rows.shape[0]
    group = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for kv in range(Hkv):
        heads = range(kv * group, (kv + 1) * group)
        rows, vis = [], []
        for t in range(T):
            last = seq_len - T + t                                  # position of token t
            n = min(last + 1, seq_len) if last >= 0 else 0
            for h in heads:
                rows.append(q_seq[t, h].astype(np.float64))
                vis.append(n)
        o, l = attend_one(np.stack(rows), k_rows[kv], v_rows[kv], vis, scale)
        i = 0
        for t in range(T):
            for h in heads:
                out[t, h] = o[i]
                lse[t, h] = l[i]
                i += 1
    return out, lse


def paged_decode(q, k_pool, v_pool, k_kind, v_kind, block_table, seq_lens,
                 scale=None):
    """The whole decode step through block tables.

    q: [n_seq][T][Hq][D] float32.  k_pool / v_pool: uint8
    [n_blocks][Hkv][page_size][row_bytes] of encodings k_kind / v_kind.
    block_table: int [n_seq][bt_stride].  seq_lens: int [n_seq] (stored rows,
    including the T new tokens).  Returns (out [n_seq][T][Hq][D] float64,
    lse [n_seq][T][Hq] float64)."""
    q = np.asarray(q)
    n_seq, T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((n_seq, T, Hq, D), dtype=np.float64)
    lse = np.full((n_seq, T, Hq), -np.inf, dtype=np.float64)
    for s in range(n_seq):
        L = int(seq_lens[s])
        try:
            if L < 0:
                raise IndexError("negative length")
            kb = pool_model.gather_rows(k_pool, block_table[s], L)
            vb = pool_model.gather_rows(v_pool, block_table[s], L)
        except IndexError:
            out[s] = np.nan
            lse[s] = np.nan
            continue
        k = quant.decode(kb, k_kind, D)
        v = quant.decode(vb, v_kind, D)
        out[s], lse[s] = decode_sequence(q[s], k, v, L, scale)
    return out, lse


def contiguous_decode(q, k_cont, v_cont, k_kind, v_kind, seq_lens, scale=None):
    """The same step over contiguous storage [n_seq][Hkv][max_len][row_bytes]."""
    q = np.asarray(q)
    n_seq, T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    max_len = k_cont.shape[2]
    out = np.zeros((n_seq, T, Hq, D), dtype=np.float64)
    lse = np.full((n_seq, T, Hq), -np.inf, dtype=np.float64)
    for s in range(n_seq):
        L = int(seq_lens[s])
        if L < 0 or L > max_len:
            out[s] = np.nan
            lse[s] = np.nan
            continue
        k = quant.decode(k_cont[s, :, :L, :], k_kind, D)
        v = quant.decode(v_cont[s, :, :L, :], v_kind, D)
        out[s], lse[s] = decode_sequence(q[s], k, v, L, scale)
    return out, lse


def merge(parts_out, parts_lse):
    """Stable merge of chunk partials (lucebox#555, Summary: stable
    split-softmax merge; llama.cpp-PR2, pd_combine fix).

    parts_out: [C][..., D] normalised chunk outputs; parts_lse: [C][...] their
    log-sum-exps.  M = max_c lse_c; if M = -inf the result is 0 with lse
    -inf; otherwise w_c = exp(lse_c - M), out = sum w_c o_c / sum w_c and
    lse = M + ln(sum w_c).  Returns (out, lse)."""
    o = np.asarray(parts_out, dtype=np.float64)
    l = np.asarray(parts_lse, dtype=np.float64)
    M = l.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - Ms[None]), 0.0)     # [C][...]
    wsum = w.sum(axis=0)
    num = (w[..., None] * o).sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(finite[..., None], num / np.where(finite, wsum, 1.0)[..., None], 0.0)
        lse = np.where(finite, Ms + np.log(np.where(finite, wsum, 1.0)), -np.inf)
    return out, lse


def chunked_decode_sequence(q_seq, k_rows, v_rows, seq_len, scale, bounds):
    """Split-K evaluation of one sequence: attend each key range
    [bounds[i], bounds[i+1]) separately (each range's masked logits, its own
    max and sum), then merge with ``merge``.  Used to check that split + merge
    equals the single pass."""
    T, Hq, D = q_seq.shape
    Hkv = k_rows.shape[0]
    group = Hq // Hkv
    parts_o, parts_l = [], []
    for c in range(len(bounds) - 1):
        k0, k1 = int(bounds[c]), int(bounds[c + 1])
        o = np.zeros((T, Hq, D))
        l = np.full((T, Hq), -np.inf)
        for t in range(T):
            last = seq_len - T + t
            hi = min(k1, last + 1, seq_len)
            n = hi - k0
            for h in range(Hq):
                kv = h // group
                if n <= 0:
                    continue
                oo, ll = attend_one(q_seq[t, h][None].astype(np.float64),
                                    k_rows[kv, k0:hi], v_rows[kv, k0:hi], [n], scale)
                o[t, h], l[t, h] = oo[0], ll[0]
        parts_o.append(o)
        parts_l.append(l)
    return merge(parts_o, parts_l)
