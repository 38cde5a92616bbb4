"""Checks that pin the oracle to things other than itself.

Each ``check_*`` takes the oracle function(s) under test as arguments and
raises AssertionError on a mismatch, so that the same check runs against the
real oracle (must pass) and against a copy with a planted mistake (must fail,
see test_oracle_controls.py).
"""

import math

import numpy as np
import torch

from paged_kv_attention_walk_amd import synth

D = 256
HQ = 24
HKV = 4


# ---------------------------------------------------------------- decoding

def hand_q4_0_row():
    """A Q4_0 row built byte by byte: block b has scale 2**(b-3) and code byte
    j = j | (15 - j) << 4, so element j is j - 8 and element j + 16 is 7 - j."""
    row = bytearray()
    expect = []
    for b in range(8):
        d = 2.0 ** (b - 3)
        row += np.float16(d).tobytes()
        row += bytes((j | ((15 - j) << 4)) for j in range(16))
        expect += [(j - 8) * d for j in range(16)] + [(7 - j) * d for j in range(16)]
    return np.frombuffer(bytes(row), dtype=np.uint8), np.array(expect)


def hand_q8_0_row():
    """A Q8_0 row: every block has scale 2**-7 (fp16 bits 0x2000) and codes
    walking through -127..127; value = code / 128 exactly."""
    row = bytearray()
    expect = []
    codes = list(range(-127, 128))
    k = 0
    for b in range(8):
        row += bytes([0x00, 0x20])                    # 2**-7, little-endian
        for i in range(32):
            c = codes[k % len(codes)]
            k += 7
            row += int(c & 0xFF).to_bytes(1, "little")
            expect.append(c / 128.0)
    return np.frombuffer(bytes(row), dtype=np.uint8), np.array(expect)


def check_closed_forms(decode):
    """decode(rows, kind) -> float64 values."""
    r, e = hand_q4_0_row()
    got = decode(r[None], "q4_0")[0]
    assert np.array_equal(got, e), "Q4_0 hand-built row"
    r, e = hand_q8_0_row()
    got = decode(r[None], "q8_0")[0]
    assert np.array_equal(got, e), "Q8_0 hand-built row"
    # F16 bit patterns: 1, -2, 65504, smallest subnormal 2**-24, -0.
    bits = np.zeros(256, dtype=np.uint16)
    bits[:5] = [0x3C00, 0xC000, 0x7BFF, 0x0001, 0x8000]
    got = decode(bits.view(np.uint8)[None], "f16")[0]
    assert list(got[:5]) == [1.0, -2.0, 65504.0, 2.0 ** -24, 0.0] and np.signbit(got[4])
    assert np.all(got[5:] == 0)
    # BF16 bit patterns: 1, -5, 2**-133 (smallest subnormal), 3.0e38-ish.
    bits = np.zeros(256, dtype=np.uint16)
    bits[:4] = [0x3F80, 0xC0A0, 0x0001, 0x7F7F]
    got = decode(bits.view(np.uint8)[None], "bf16")[0]
    assert got[0] == 1.0 and got[1] == -5.0 and got[2] == 2.0 ** -133
    assert got[3] == float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), dtype=np.float32)[0])


def check_scale_position(decode, fixture):
    """Q4_0 block v's scale sits at byte 18*v of the row (fixture).  Codes are
    all 9 (value +1 * scale) so block v decodes to its scale; scales are
    distinct powers of two."""
    row = np.full(144, 0x99, dtype=np.uint8)           # both nibbles 9
    for v, off in enumerate(fixture["scale_byte_in_row"]):
        assert off == fixture["piece_bytes"] * v + 2 * v
        row[off:off + 2] = np.frombuffer(np.float16(2.0 ** v).tobytes(), dtype=np.uint8)
    got = decode(row[None], "q4_0")[0]
    for v in range(8):
        assert np.all(got[32 * v:32 * v + 32] == 2.0 ** v), f"block {v}"


# ---------------------------------------------------------------- attention

def sdpa_reference(q, k, v, seq_len, scale):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the CPU.
    q [T][HQ][D]; k, v [HKV][L][D] float64.  Query head h reads KV head
    h // 6 (expanded with repeat_interleave); token t sees keys <= L-T+t.
    Rows with no visible key are returned as NaN (excluded by callers)."""
    T = q.shape[0]
    L = k.shape[1]
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()      # [HQ][T][D]
    kt = torch.from_numpy(k).double().repeat_interleave(HQ // HKV, dim=0)           # [HQ][L][D]
    vt = torch.from_numpy(v).double().repeat_interleave(HQ // HKV, dim=0)
    pos = torch.arange(L)[None, :]
    last = (seq_len - T + torch.arange(T))[:, None]
    mask = pos <= last                                                              # [T][L]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt[None], kt[None], vt[None], attn_mask=mask[None, None], scale=scale)[0]
    out = out.numpy().transpose(1, 0, 2)                                            # [T][HQ][D]
    empty = ~mask.any(dim=1).numpy()
    out = out.copy()
    out[empty] = np.nan
    return out


def brute_force(q, k, v, seq_len, scale):
    """Pure-Python loops (tiny inputs only): returns out [T][HQ][D], lse [T][HQ]."""
    T = q.shape[0]
    out = np.zeros((T, HQ, D))
    lse = np.full((T, HQ), -math.inf)
    for t in range(T):
        visible = [j for j in range(seq_len) if j <= seq_len - T + t]
        for h in range(HQ):
            kv = h // (HQ // HKV)
            if not visible:
                continue
            logits = []
            for j in visible:
                acc = 0.0
                for d in range(D):
                    acc += float(q[t, h, d]) * float(k[kv, j, d])
                logits.append(acc * scale)
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            tot = math.fsum(w)
            for d in range(D):
                out[t, h, d] = math.fsum(w[i] * float(v[kv, j, d]) for i, j in enumerate(visible)) / tot
            lse[t, h] = m + math.log(tot)
    return out, lse


def check_against_sdpa(decode_sequence, cases):
    """cases: iterable of (q [T][HQ][D], k, v [HKV][L][D], L, scale)."""
    for (q, k, v, L, scale) in cases:
        got, _ = decode_sequence(q, k, v, L, scale)
        ref = sdpa_reference(q, k, v, L, scale)
        ok = ~np.isnan(ref)
        assert np.all(got[~ok] == 0), "rows with no visible key must be 0"
        denom = max(1e-300, np.abs(ref[ok]).max()) if ok.any() else 1.0
        err = np.abs(got[ok] - ref[ok]).max() / denom if ok.any() else 0.0
        assert err <= 1e-12, f"SDPA mismatch {err:.3e} (L={L}, T={q.shape[0]})"


def check_against_brute_force(decode_sequence, cases):
    for (q, k, v, L, scale) in cases:
        got, glse = decode_sequence(q, k, v, L, scale)
        ref, rlse = brute_force(q, k, v, L, scale)
        denom = max(1e-300, np.abs(ref).max())
        assert np.abs(got - ref).max() <= 1e-12 * denom, f"brute force out (L={L})"
        fin = np.isfinite(rlse)
        assert np.array_equal(fin, np.isfinite(glse)), "lse finiteness"
        assert np.all(np.abs(glse[fin] - rlse[fin]) <= 1e-12 * (1 + np.abs(rlse[fin]))), "brute force lse"


def random_sequence_case(rng, L, T, kind_k, kind_v, scale=1 / 16, q_scale=1.0, value_scale=1.0):
    """Decoded-float test data for one sequence, made by encoding random values
    and decoding with ``decode`` later by the caller.  Returns encoded rows."""
    q = rng.standard_normal((T, HQ, D)).astype(np.float32) * np.float32(q_scale)
    kx = rng.standard_normal((HKV, L, D)).astype(np.float32) * np.float32(value_scale)
    vx = rng.standard_normal((HKV, L, D)).astype(np.float32) * np.float32(value_scale)
    return q, synth.encode(kx, kind_k), synth.encode(vx, kind_v)


# ---------------------------------------------------------------- paging

def check_paged_equals_contiguous(paged_decode, contiguous_decode, pages=(16, 48, 128, 256, 512),
                                  seed=0, kinds=("q4_0", "q8_0", "f16", "bf16")):
    """Two or more sequences' pages shuffled through one pool: the paged result
    must equal the contiguous result exactly (same float64 arithmetic on the
    same logical rows)."""
    rng = np.random.default_rng(seed)
    for P in pages:
        for kind in kinds:
            lens = [int(x) for x in rng.integers(1, 3 * P, size=3)] + [0]
            T = int(rng.integers(1, 9))
            w = synth.make_workload("t", lens, T, kind, kind, P, table="shuffled",
                                    seed=int(rng.integers(1 << 30)), n_blocks=sum(
                                        synth.blocks_needed(L, P) for L in lens) + 3)
            max_len = max(lens)
            kc = synth.contiguous_from_table(w["k_pool"], w["block_table"], lens, max_len)
            vc = synth.contiguous_from_table(w["v_pool"], w["block_table"], lens, max_len)
            a, al = paged_decode(w["q"], w["k_pool"], w["v_pool"], kind, kind, w["block_table"], lens, 1 / 16)
            b, bl = contiguous_decode(w["q"], kc, vc, kind, kind, lens, 1 / 16)
            assert np.array_equal(a, b) and np.array_equal(al, bl), f"paged != contiguous (P={P}, {kind})"


# ---------------------------------------------------------------- encoding
#
# Each check takes ``enc(x, kind)``: float32 [..., 256] -> encoded rows.

def _row_of_blocks(blocks):
    """A 256-value float32 row from up to 8 blocks of 32 (the rest zero)."""
    row = np.zeros(256, np.float32)
    for b, v in enumerate(blocks):
        row[32 * b:32 * b + 32] = v
    return row


def q4_fields(row_bytes):
    """(scale, 32 codes) of each block of a Q4_0 row, read byte by byte: the
    fp16 scale first, then byte j = code j | code j+16 << 4."""
    out = []
    for b in range(8):
        blk = row_bytes[18 * b:18 * b + 18]
        d = float(np.frombuffer(bytes(blk[0:2]), "<f2")[0])
        out.append((d, [int(blk[2 + j]) & 15 for j in range(16)] + [int(blk[2 + j]) >> 4 for j in range(16)]))
    return out


def q8_fields(row_bytes):
    """(scale, 32 codes) of each block of a Q8_0 row."""
    out = []
    for b in range(8):
        blk = row_bytes[34 * b:34 * b + 34]
        d = float(np.frombuffer(bytes(blk[0:2]), "<f2")[0])
        out.append((d, [int(c) for c in np.frombuffer(bytes(blk[2:]), np.int8)]))
    return out


def _one_block(enc, kind, blk):
    fields = q4_fields if kind == "q4_0" else q8_fields
    return fields(enc(_row_of_blocks([blk])[None], kind)[0])[0]


def check_encode_closed_forms(enc):
    """Blocks built from codes: Q4_0 values (c-8) 2^e with a code 0 present
    (max|x| = 8 2^e, so d = 2^e exactly), Q8_0 values c 2^e with |c| = 127
    present; the encoder must return exactly those scales and codes."""
    for e in (-14, -5, 0, 3, 12):
        rng = np.random.default_rng(e + 100)
        blocks = []
        for _ in range(8):
            c = rng.integers(0, 16, size=32)
            c[rng.integers(0, 32)] = 0
            blocks.append(c)
        row = _row_of_blocks([(c - 8).astype(np.float32) * np.float32(2.0 ** e) for c in blocks])
        for (d, codes), c in zip(q4_fields(enc(row[None], "q4_0")[0]), blocks):
            assert d == 2.0 ** e and codes == [int(v) for v in c]
    for e in (-17, -7, 0, 4, 8):
        rng = np.random.default_rng(e + 200)
        blocks = []
        for _ in range(8):
            c = rng.integers(-127, 128, size=32)
            c[rng.integers(0, 32)] = rng.choice([-127, 127])
            blocks.append(c)
        row = _row_of_blocks([c.astype(np.float32) * np.float32(2.0 ** e) for c in blocks])
        for (d, codes), c in zip(q8_fields(enc(row[None], "q8_0")[0]), blocks):
            assert d == 2.0 ** e and codes == [int(v) for v in c]


def check_encode_clip_and_zero(enc):
    """Q4_0: a block whose max|x| is a positive value maps it to 16 steps,
    stored as 15; blocks of zeros store scale 0 and codes 8 (Q4_0) / 0."""
    blk = np.linspace(-3, 8, 32).astype(np.float32)
    d, codes = _one_block(enc, "q4_0", blk)
    assert d == 1.0 and codes[31] == 15 and codes[0] == 5
    z = np.zeros((1, 256), np.float32)
    q4, q8 = enc(z, "q4_0")[0], enc(z, "q8_0")[0]
    for b in range(8):
        assert q4[18 * b] == 0 and q4[18 * b + 1] == 0 and np.all(q4[18 * b + 2:18 * b + 18] == 0x88)
        assert np.all(q8[34 * b:34 * b + 34] == 0)


def check_encode_rounding(enc):
    """Codes: halves away from zero; a float32 just below a half rounds down
    (0.5 - 2^-25, whose float32 sum with 0.5 is 1); the step is the stored
    fp16 scale; the product x r is a float32 operation."""
    vals = np.array([2.5, -2.5, 0.5, -0.5, 1.4999999, -1.4999999, 126.5], np.float32)
    blk = np.zeros(32, np.float32)
    blk[:len(vals)], blk[31] = vals, 127.0
    d, codes = _one_block(enc, "q8_0", blk)
    assert d == 1.0 and codes[:len(vals)] == [3, -3, 1, -1, 1, -1, 127]
    blk = np.zeros(32, np.float32)
    blk[:4], blk[31] = [0.5, -0.5, 3.5, -7.5], -8.0
    d, codes = _one_block(enc, "q4_0", blk)
    assert d == 1.0 and codes[:4] == [9, 7, 12, 0] and codes[31] == 0
    v = np.float32(0.5) - np.float32(2.0 ** -25)
    assert v < 0.5 and np.float32(v + np.float32(0.5)) == 1.0
    blk = np.zeros(32, np.float32)
    blk[0], blk[1], blk[2], blk[31] = v, -v, 0.5, 127.0
    d, codes = _one_block(enc, "q8_0", blk)
    assert d == 1.0 and codes[:3] == [0, 0, 1]
    # max 127.0127: d = 1.0001, stored as fp16 1.0; 2.50015 is 2.50015 stored
    # steps (code 3) but 2.4999 unrounded ones
    blk = np.zeros(32, np.float32)
    blk[0], blk[31] = 2.50015, 127.0127
    d, codes = _one_block(enc, "q8_0", blk)
    assert d == 1.0 and codes[0] == 3 and codes[31] == 127
    # d = 3 (max 381), r = float32(1/3): x = 7.5 - 2^-21 has x / 3 < 2.5 but
    # float32(x r) == 2.5, so the code is 3
    x = np.float32(7.5) - np.float32(2.0 ** -21)
    assert float(x) / 3.0 < 2.5 and np.float32(x * (np.float32(1) / np.float32(3))) == np.float32(2.5)
    blk = np.zeros(32, np.float32)
    blk[0], blk[31] = x, 381.0
    d, codes = _one_block(enc, "q8_0", blk)
    assert d == 3.0 and codes[0] == 3


def check_encode_scale_rounding(enc):
    """max|x| / 127 is stored as the nearest fp16 (ties to even), subnormal
    scales included; below half the smallest subnormal the scale is 0."""
    for amax, d_want in [(127.0 * (1 + 2.0 ** -11), 1.0),
                         (127.0 * (1 + 3 * 2.0 ** -11), 1 + 2.0 ** -9),
                         (127.0 * 2.0 ** -24, 2.0 ** -24),
                         (127.0 * 2.0 ** -26, 0.0)]:
        blk = np.zeros(32, np.float32)
        blk[5] = -amax
        d, codes = _one_block(enc, "q8_0", blk)
        assert d == d_want, (amax, d)
        assert codes[5] == (max(-127, -round(amax / d_want)) if d_want else 0)


def check_encode_two_byte_rounding(enc):
    """F16 and BF16: nearest value, ties to even, overflow to infinity,
    subnormals kept."""
    vals = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65519.0, 65520.0, -2.0 ** -25, 2.0 ** -24], np.float32)
    with np.errstate(over="ignore"):
        f16 = enc(np.resize(vals, 256)[None], "f16")[0].view("<u2")[:len(vals)]
    assert list(f16) == [0x3C00, 0x3C02, 0x7BFF, 0x7C00, 0x8000, 0x0001]
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -7), 3.0e38, 1.0e-40], np.float32)
    bf = enc(np.resize(vals, 256)[None], "bf16")[0].view("<u2")[:len(vals)]
    assert list(bf) == [0x3F80, 0x3F82, 0xBF81, 0x7F62, 0x0001]
    x = (np.random.default_rng(1).standard_normal(256).astype(np.float32).view(np.uint32)
         & np.uint32(0xFFFF0000)).view(np.float32)
    assert np.array_equal(enc(x[None], "bf16")[0].view("<u2"), (x.view(np.uint32) >> 16).astype(np.uint16))
    assert np.all(enc(-np.zeros((1, 256), np.float32), "f16")[0][1::2] == 0x80)
    assert np.all(enc(-np.zeros((1, 256), np.float32), "bf16")[0][1::2] == 0x80)


ENCODE_CHECKS = (check_encode_closed_forms, check_encode_clip_and_zero, check_encode_rounding,
                 check_encode_scale_rounding, check_encode_two_byte_rounding)


# ------------------------------------------------------------ append scatter

def check_scatter(scatter, gather, P=16, rb=144, seed=0):
    """scatter(pool, blocks, slots, rows) against the logical positions that
    the (separately pinned) gather reads back.  Three sequences own every page
    of the pool through a shuffled table, so gathering all of them reads every
    byte.  Rows are appended at logical positions (s, pos): destination
    (table[s][pos // P], pos % P).  After the scatter, gathered row pos of
    sequence s is the appended row for each KV head; two rows aimed at one
    position leave the later; every other gathered row keeps its bytes."""
    rng = np.random.default_rng(seed)
    n_pages = [3, 5, 2]
    nb = sum(n_pages)
    perm = rng.permutation(nb)
    tables, k = [], 0
    for n in n_pages:
        tables.append(perm[k:k + n])
        k += n
    pool = rng.integers(0, 256, size=(nb, HKV, P, rb), dtype=np.uint8)
    before = [gather(pool, tables[s], n_pages[s] * P) for s in range(3)]
    # logical destinations: page boundaries, slot 0 and P - 1, and one repeat
    dests = [(0, 0), (0, P - 1), (0, P), (1, 2 * P + 7), (1, 5 * P - 1), (2, P + 3), (1, 2 * P + 7)]
    rows = rng.integers(0, 256, size=(len(dests), HKV, rb), dtype=np.uint8)
    blocks = np.array([tables[s][pos // P] for s, pos in dests], np.int32)
    slots = np.array([pos % P for s, pos in dests], np.int32)
    pool_copy = pool.copy()
    after = scatter(pool, blocks, slots, rows)
    assert np.array_equal(pool, pool_copy), "the input pool is left unmodified"
    expect = [b.copy() for b in before]
    for i, (s, pos) in enumerate(dests):
        expect[s][:, pos, :] = rows[i]                    # in order: the later row of a repeat wins
    for s in range(3):
        got = gather(after, tables[s], n_pages[s] * P)
        for h in range(HKV):
            for pos in range(n_pages[s] * P):
                assert np.array_equal(got[h, pos], expect[s][h, pos]), f"sequence {s}, KV head {h}, position {pos}"
    # out-of-range destinations raise and write nothing
    for b, sl in ((nb, 0), (-1, 0), (0, P), (0, -1)):
        try:
            scatter(pool, np.array([0, b], np.int32), np.array([1, sl], np.int32), rows[:2])
        except IndexError:
            pass
        else:
            raise AssertionError(f"destination (block {b}, slot {sl}) accepted")
