"""Seeded synthetic inputs for paged K/V decode: values, encoded rows, pools,
block tables and the five workload shapes.

This module is the only code that the tests, the benchmark and the oracle
checks have in common.  It makes inputs and holds none of the decode path's
arithmetic: no decoding of rows, no attention, no merge.  Encoding float data
into rows (the quantisers below) only manufactures stored bytes; every check
decodes those bytes on its own side.

Workloads follow the source pages' synthetic benchmarks: D = 256 with 24 query
heads over 4 KV heads (lucebox#555, Benchmark results); Q4_0 K/V in 16-token
pages with an interleaved table, uniform 8 x 4096 and ragged 131072 + 7 x 8192
(same section); Q8_0 K/V for 1-4 query tokens in 256-token pages at 32K to
262K (llama.cpp-PR2, split-K decode and page-table commits); many ragged
streams of up to 8192 positions in 64-token pages with a one-row append per
step (colibri#372, Summary).
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 256
N_Q_HEADS = 24
N_KV_HEADS = 4
QBLOCK = 32

KINDS = ("f16", "bf16", "q8_0", "q4_0")
ROW_BYTES = {"f16": 512, "bf16": 512, "q8_0": 272, "q4_0": 144}


# --------------------------------------------------------------------------
# random values
# --------------------------------------------------------------------------

def normal(shape, seed, scale=1.0, dtype=np.float32) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x.astype(dtype, copy=False)


# --------------------------------------------------------------------------
# encoders (test-data manufacture)
# --------------------------------------------------------------------------

def _round_half_away(x: np.ndarray) -> np.ndarray:
    # in float64, where |x| + 0.5 is exact for float32 x (in float32 it can
    # round up to the next integer just below a half)
    x = np.asarray(x, dtype=np.float64)
    return np.sign(x) * np.floor(np.abs(x) + 0.5)


def encode_f16(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return np.ascontiguousarray(x.astype(np.float16)).view(np.uint8).reshape(x.shape[:-1] + (2 * x.shape[-1],))


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 with round-to-nearest-even (finite inputs)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16).view(np.uint8).reshape(x.shape[:-1] + (2 * x.shape[-1],))


def encode_q8_0(x: np.ndarray) -> np.ndarray:
    """Blocks of 32: fp16 scale d = max|x|/127, int8 codes round(x/d)."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(-1, D // QBLOCK, QBLOCK)
    d = (np.abs(blk).max(axis=-1) / 127.0).astype(np.float16)
    df = d.astype(np.float32)
    inv = np.where(df > 0, 1.0 / np.where(df > 0, df, 1.0), 0.0).astype(np.float32)
    codes = np.clip(_round_half_away(blk * inv[..., None]), -127, 127).astype(np.int8)
    out = np.empty(blk.shape[:2] + (2 + QBLOCK,), dtype=np.uint8)
    out[..., 0:2] = d[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:] = codes.view(np.uint8)
    return out.reshape(lead + (D // QBLOCK * 34,))


def encode_q4_0(x: np.ndarray) -> np.ndarray:
    """Blocks of 32: fp16 scale d = max|x|/8 (the workload's definition),
    codes clamp(round(x/d) + 8, 0, 15) -- a block's positive extreme would give
    16 and is clipped to 15 -- packed with element j in the low nibble and
    element j+16 in the high nibble of byte j."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(-1, D // QBLOCK, QBLOCK)
    d = (np.abs(blk).max(axis=-1) / 8.0).astype(np.float16)
    df = d.astype(np.float32)
    inv = np.where(df > 0, 1.0 / np.where(df > 0, df, 1.0), 0.0).astype(np.float32)
    c = np.clip(_round_half_away(blk * inv[..., None]) + 8, 0, 15).astype(np.uint8)
    packed = c[..., :16] | (c[..., 16:] << 4)
    out = np.empty(blk.shape[:2] + (18,), dtype=np.uint8)
    out[..., 0:2] = d[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:] = packed
    return out.reshape(lead + (D // QBLOCK * 18,))


ENCODERS = {"f16": encode_f16, "bf16": encode_bf16, "q8_0": encode_q8_0, "q4_0": encode_q4_0}


def encode(x: np.ndarray, kind: str) -> np.ndarray:
    return ENCODERS[kind](x)


def random_rows(shape_lead, kind, seed, scale=1.0, chunk=1 << 22) -> np.ndarray:
    """Encoded rows of N(0, scale^2) values, shape ``shape_lead + (row_bytes,)``.
    Generated in chunks of rows so that large pools fit in host memory."""
    n = int(np.prod(shape_lead)) if len(shape_lead) else 1
    rb = ROW_BYTES[kind]
    out = np.empty((n, rb), dtype=np.uint8)
    rng = np.random.default_rng(seed)
    step = max(1, chunk // HEAD_DIM)
    for i in range(0, n, step):
        m = min(step, n - i)
        x = rng.standard_normal(size=(m, HEAD_DIM), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[i:i + m] = encode(x, kind)
    return out.reshape(tuple(shape_lead) + (rb,))


# --------------------------------------------------------------------------
# block tables
# --------------------------------------------------------------------------

def blocks_needed(seq_len: int, page_size: int) -> int:
    return -(-int(seq_len) // page_size)


def round_robin_table(seq_lens, page_size, bt_stride=None):
    """Interleaved table: in round b, each sequence that still needs a b-th page
    takes the next pool index, in sequence order (the order concurrent decode
    produces).  Returns (table [n_seq][bt_stride] int32, n_blocks).  Unused
    entries are -1."""
    need = [blocks_needed(L, page_size) for L in seq_lens]
    stride = max(need + [1]) if bt_stride is None else bt_stride
    table = np.full((len(seq_lens), stride), -1, dtype=np.int32)
    nxt = 0
    for b in range(max(need + [0])):
        for s, n in enumerate(need):
            if b < n:
                table[s, b] = nxt
                nxt += 1
    return table, nxt


def shuffled_table(seq_lens, page_size, seed, bt_stride=None, n_blocks=None):
    """Every sequence's pages at seeded random, distinct pool indices.  With
    ``n_blocks`` larger than needed the unused pool pages are spread among
    them.  Returns (table, n_blocks)."""
    need = [blocks_needed(L, page_size) for L in seq_lens]
    total = sum(need)
    nb = total if n_blocks is None else int(n_blocks)
    if nb < total:
        raise ValueError("pool too small")
    stride = max(need + [1]) if bt_stride is None else bt_stride
    perm = np.random.default_rng(seed).permutation(nb)[:total].astype(np.int32)
    table = np.full((len(seq_lens), stride), -1, dtype=np.int32)
    i = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[i:i + n]
        i += n
    return table, nb


def contiguous_from_table(pool: np.ndarray, table, seq_lens, max_len: int) -> np.ndarray:
    """Per-sequence contiguous copy ``[n_seq][Hkv][max_len][row_bytes]`` of the
    rows a paged pool ``[n_blocks][Hkv][P][row_bytes]`` holds (zero padding)."""
    n_blocks, hkv, P, rb = pool.shape
    out = np.zeros((len(seq_lens), hkv, max_len, rb), dtype=np.uint8)
    for s, L in enumerate(seq_lens):
        L = int(L)
        for lp in range(blocks_needed(L, P)):
            n = min(P, L - lp * P)
            out[s, :, lp * P: lp * P + n, :] = pool[int(table[s, lp]), :, :n, :]
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

class Workload(dict):
    """q [n_seq][T][24][256] float32, k_pool / v_pool uint8
    [n_blocks][4][P][row_bytes], block_table int32, seq_lens int32, plus
    k_kind, v_kind, page_size, scale, name."""

    @property
    def kv_bytes(self) -> int:
        """Algorithmic K/V bytes: each live row read once per KV head."""
        L = int(np.sum(self["seq_lens"]))
        return L * N_KV_HEADS * (ROW_BYTES[self["k_kind"]] + ROW_BYTES[self["v_kind"]])


def make_workload(name, seq_lens, n_qtok, k_kind, v_kind, page_size, *,
                  table="shuffled", seed=0, perm_seed=None, value_scale=1.0,
                  q_scale=1.0, scale=1.0 / 16.0, n_blocks=None, bt_stride=None):
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if table == "round_robin":
        bt, nb = round_robin_table(seq_lens, page_size, bt_stride)
    elif table == "shuffled":
        bt, nb = shuffled_table(seq_lens, page_size, 100 + seed if perm_seed is None else perm_seed,
                                bt_stride, n_blocks)
    else:
        raise ValueError(table)
    if n_blocks is not None and table == "round_robin":
        nb = max(nb, int(n_blocks))
    nb = max(nb, 1)
    q = normal((len(seq_lens), n_qtok, N_Q_HEADS, HEAD_DIM), seed * 7919 + 1, q_scale)
    k_pool = random_rows((nb, N_KV_HEADS, page_size), k_kind, seed * 7919 + 2, value_scale)
    v_pool = random_rows((nb, N_KV_HEADS, page_size), v_kind, seed * 7919 + 3, value_scale)
    return Workload(name=name, q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                    seq_lens=seq_lens, n_qtok=n_qtok, k_kind=k_kind, v_kind=v_kind,
                    page_size=page_size, scale=scale, n_blocks=nb)


def config1(seed=1):
    """One sequence of 1024 F16 positions, one query token, 16-token pages at a
    seeded permutation of a 64-page pool; q, K, V ~ N(0,1)/16; scale 1/16."""
    return make_workload("f16_1x1024_p16_shuffled", [1024], 1, "f16", "f16", 16,
                         table="shuffled", seed=seed, value_scale=1 / 16, q_scale=1 / 16)


def config2(seed=2, n_seq=8):
    """Uniform batch of 4096-position Q4_0 sequences, 16-token interleaved pages."""
    return make_workload(f"q4_0_{n_seq}x4096_p16_interleaved", [4096] * n_seq, 1, "q4_0", "q4_0", 16,
                         table="round_robin", seed=seed)


RAGGED_LENS = [131072] + [8192] * 7


def config3(seed=3, table="round_robin"):
    """Ragged 131072 + 7 x 8192 Q4_0, 16-token pages, interleaved table over a
    pool of exactly 11,776 pages (188,416 live positions)."""
    return make_workload("q4_0_ragged_128k_7x8k_p16_" + ("interleaved" if table == "round_robin" else "shuffled"),
                         RAGGED_LENS, 1, "q4_0", "q4_0", 16, table=table, seed=seed)


def ragged_mixed(seed=3, k_kind="q8_0", v_kind="q4_0"):
    """The ragged 131072 + 7 x 8192 step with K and V pools of different
    encodings (Q8_0 K with Q4_0 V by default), same table and pages."""
    return make_workload(f"{k_kind}k_{v_kind}v_ragged_128k_7x8k_p16_interleaved", RAGGED_LENS, 1, k_kind, v_kind, 16,
                         table="round_robin", seed=seed)


def config4(ctx=32768, n_qtok=1, seed=4, kind="q8_0"):
    """One sequence, 1-4 query tokens with a causal mask among them, Q8_0 K/V
    (or `kind` for both), 256-token shuffled pages."""
    return make_workload(f"{kind}_1x{ctx}_t{n_qtok}_p256_shuffled", [ctx], n_qtok, kind, kind, 256,
                         table="shuffled", seed=seed)


def prefill_workload(ctx=16384, n_qtok=65, seed=6):
    """One sequence of `ctx` stored positions whose last `n_qtok` are the new
    query tokens, Q8_0 K and Q4_0 V in 256-token shuffled pages."""
    return make_workload(f"q8_0k_q4_0v_1x{ctx}_t{n_qtok}_p256_shuffled", [ctx], n_qtok, "q8_0", "q4_0", 256,
                         table="shuffled", seed=seed)


def config5_lengths(seed=5, n_seq=128):
    """Lengths before the step: uniform integers in [512, 8192]."""
    return np.random.default_rng(seed).integers(512, 8192, size=n_seq, endpoint=True).astype(np.int32)


def config5(seed=5, n_seq=128):
    """128 streams, lengths U{512..8192} before the step plus one appended row,
    BF16 K/V in 64-token pages shuffled through one pool."""
    lens = config5_lengths(seed, n_seq) + 1
    return make_workload("bf16_128streams_512-8192_p64_shuffled", lens, 1, "bf16", "bf16", 64,
                         table="shuffled", seed=seed)


def config5_rolling(seed=5, n_seq=128, steps=16):
    """The many-stream serving step over `steps` consecutive decode steps:
    stream s holds L0_s ~ U{512..8192} rows before the first step; step k
    appends one row at position L0_s + k and decodes at length L0_s + k + 1,
    so pages fill up and new pages start within the window.  The table and
    pool cover L0_s + steps positions (the rows past L0_s are written by the
    appends); seq_lens holds L0_s, the lengths before the first step."""
    base = config5_lengths(seed, n_seq)
    w = make_workload("bf16_128streams_512-8192_p64_shuffled", base + steps, 1, "bf16", "bf16", 64,
                      table="shuffled", seed=seed)
    w["seq_lens"] = base.copy()
    w["steps"] = steps
    return w
