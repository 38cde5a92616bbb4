"""Negative controls: plausible mistakes planted in copies of oracle functions
must turn the pins red (CPU).  The real oracle is never modified; each test
builds a broken variant and runs the same check the real oracle passes.

The pages use the same kind of control: TensorFold#1156 (Verification) keeps a
swapped table over correctly placed pages and a planted row red; llama.cpp
PR 2 (LDS-read commit) reports that a broken K shift or V scale fails its
cases."""

import json
import os

import numpy as np
import pytest

from oracle import attention, encode, pool_model, quant
from oracle_checks import (check_against_brute_force, check_against_sdpa, check_closed_forms,
                           check_paged_equals_contiguous, check_scale_position, random_sequence_case)


def _decode_swapped_nibbles(rows, kind, head_dim=256):
    if kind != "q4_0":
        return quant.decode(rows, kind, head_dim)
    r = np.asarray(rows)
    blk = r.reshape(r.shape[:-1] + (8, 18))
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    cb = blk[..., 2:]
    codes = np.concatenate([(cb >> 4), (cb & 15)], axis=-1).astype(np.float64)   # planted
    return ((codes - 8) * d[..., None]).reshape(r.shape[:-1] + (256,))


def _decode_interleaved_nibbles(rows, kind, head_dim=256):
    if kind != "q4_0":
        return quant.decode(rows, kind, head_dim)
    r = np.asarray(rows)
    blk = r.reshape(r.shape[:-1] + (8, 18))
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    cb = blk[..., 2:]
    codes = np.stack([(cb & 15), (cb >> 4)], axis=-1).reshape(cb.shape[:-1] + (32,)).astype(np.float64)  # planted
    return ((codes - 8) * d[..., None]).reshape(r.shape[:-1] + (256,))


def _decode_scale_at_end(rows, kind, head_dim=256):
    if kind != "q4_0":
        return quant.decode(rows, kind, head_dim)
    r = np.asarray(rows)
    blk = r.reshape(r.shape[:-1] + (8, 18))
    d = blk[..., 16:18].copy().view(np.float16)[..., 0].astype(np.float64)       # planted
    cb = blk[..., 0:16]
    codes = np.concatenate([(cb & 15), (cb >> 4)], axis=-1).astype(np.float64)
    return ((codes - 8) * d[..., None]).reshape(r.shape[:-1] + (256,))


def _decode_q8_unsigned(rows, kind, head_dim=256):
    if kind != "q8_0":
        return quant.decode(rows, kind, head_dim)
    r = np.asarray(rows)
    blk = r.reshape(r.shape[:-1] + (8, 34))
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    return (blk[..., 2:].astype(np.float64) * d[..., None]).reshape(r.shape[:-1] + (256,))  # planted


@pytest.mark.parametrize("bad", [_decode_swapped_nibbles, _decode_interleaved_nibbles,
                                 _decode_scale_at_end, _decode_q8_unsigned])
def test_decode_mistakes_fail_closed_forms(bad):
    with pytest.raises(AssertionError):
        check_closed_forms(bad)


def test_scale_mistake_fails_position_pin(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "q4_0_scale_position_llamacpp_pr2.json")))
    with pytest.raises(AssertionError):
        check_scale_position(_decode_scale_at_end, fx)


def _cases(seed, lens=(3, 17, 40)):
    rng = np.random.default_rng(seed)
    out = []
    for i, L in enumerate(lens):
        T = 1 + (i + 2) % 4
        q, kb, vb = random_sequence_case(rng, L, T, "q8_0", "q4_0", q_scale=4.0)
        out.append((q, quant.decode(kb, "q8_0"), quant.decode(vb, "q4_0"), L, 1 / 16))
    return out


def _mutant(kind):
    def decode_sequence(q_seq, k_rows, v_rows, seq_len, scale):
        T, Hq, D = q_seq.shape
        out = np.zeros((T, Hq, D))
        lse = np.full((T, Hq), -np.inf)
        for t in range(T):
            last = seq_len - T + t + (1 if kind == "causal_off_by_one" else 0)
            n = min(last + 1, seq_len) if last >= 0 else 0
            for h in range(Hq):
                kv = h % 4 if kind == "gqa_modulo" else h // 6
                if n <= 0:
                    continue
                s = scale * (k_rows[kv, :n] @ q_seq[t, h].astype(np.float64))
                if kind == "no_scale":
                    s = s / scale
                m = s.max()
                e = np.exp(s - m)
                if kind == "drop_last_key":
                    e = e[:-1] if n > 1 else e
                vv = v_rows[kv, :len(e)]
                if kind == "transposed_v":
                    vv = v_rows[kv, :len(e)][:, ::-1]
                out[t, h] = e @ vv / e.sum()
                lse[t, h] = m + (np.log2(e.sum()) if kind == "log2_lse" else np.log(e.sum()))
        return out, lse
    return decode_sequence


@pytest.mark.parametrize("kind", ["causal_off_by_one", "gqa_modulo", "no_scale", "drop_last_key", "transposed_v"])
def test_attention_mistakes_fail_sdpa(kind):
    assert _mutant("none")  # the unmutated copy passes (sanity)
    check_against_sdpa(_mutant("none"), _cases(1))
    with pytest.raises(AssertionError):
        check_against_sdpa(_mutant(kind), _cases(1))


def test_lse_mistake_fails_brute_force():
    cases = _cases(2, lens=(5, 9))
    check_against_brute_force(_mutant("none"), cases)
    with pytest.raises(AssertionError):
        check_against_brute_force(_mutant("log2_lse"), cases)


def _paged_swapped_table(q, k_pool, v_pool, kk, vk, bt, lens, scale=None):
    bt = np.array(bt, copy=True)
    if bt.shape[1] >= 2:
        bt[:, [0, 1]] = bt[:, [1, 0]]              # planted: swapped table entries
    return attention.paged_decode(q, k_pool, v_pool, kk, vk, bt, lens, scale)


def _paged_planted_row(q, k_pool, v_pool, kk, vk, bt, lens, scale=None):
    k_pool = k_pool.copy()
    b = int(bt[0][0])
    k_pool[b, 0, 0, 2:] ^= 0x5A                     # planted: one row changed (not a scale byte)
    return attention.paged_decode(q, k_pool, v_pool, kk, vk, bt, lens, scale)


@pytest.mark.parametrize("bad", [_paged_swapped_table, _paged_planted_row])
def test_paging_mistakes_fail_paged_equals_contiguous(bad):
    with pytest.raises(AssertionError):
        check_paged_equals_contiguous(bad, attention.contiguous_decode, pages=(16,), kinds=("q8_0",))


def test_gather_mistake_is_caught():
    orig = pool_model.gather_rows

    def bad_gather(pool, table_row, seq_len):
        out = orig(pool, table_row, seq_len)
        P = pool.shape[2]
        if seq_len > P:
            out[:, P:] = out[:, P - 1:-1].copy()         # planted: off-by-one across a page boundary
        return out
    try:
        pool_model.gather_rows = bad_gather
        with pytest.raises(AssertionError):
            check_paged_equals_contiguous(attention.paged_decode, attention.contiguous_decode,
                                          pages=(16,), kinds=("f16",))
    finally:
        pool_model.gather_rows = orig


# ------------------------------------------------------------ row encoding

def _planted_encoder(mistake):
    """A copy of the block encoders with one planted mistake."""
    def enc(x, kind):
        if kind in ("f16", "bf16"):
            x = np.asarray(x, np.float32)
            if mistake == "bf16_truncate" and kind == "bf16":
                b = (x.view(np.uint32) >> 16).astype("<u2")
                return b.view(np.uint8).reshape(x.shape[:-1] + (512,))
            return encode.encode(x, kind)
        qmax = 127.0 if kind == "q8_0" else (7.0 if mistake == "q4_over_7" else 8.0)
        x = np.asarray(x, np.float32)
        blk = x.reshape(x.shape[:-1] + (8, 32))
        amax = np.abs(blk).max(-1)
        d16 = (amax / np.float32(qmax)).astype(np.float16)
        dd = amax / np.float32(qmax) if mistake == "unrounded_scale" else d16.astype(np.float32)
        r = np.where(dd != 0, np.float32(1) / np.where(dd != 0, dd, 1), 0).astype(np.float32)
        if mistake == "f64_division":
            v = blk.astype(np.float64) / np.where(dd != 0, dd, np.inf)[..., None].astype(np.float64)
        else:
            v = (blk * r[..., None]).astype(np.float32)
        if mistake == "half_even":
            c = np.rint(v)
        elif mistake == "f32_floor":
            c = np.sign(v) * np.floor(np.abs(v).astype(np.float32) + np.float32(0.5))
        else:
            c = encode.round_half_away(v)
        out = np.empty(blk.shape[:-1] + ((34,) if kind == "q8_0" else (18,)), np.uint8)
        out[..., 0:2] = d16.astype("<f2")[..., None].view(np.uint8)
        if kind == "q8_0":
            out[..., 2:] = np.clip(c, -127, 127).astype(np.int8).view(np.uint8)
        else:
            c = c + 8
            c = (c.astype(np.int64) & 15) if mistake == "q4_no_clip" else np.clip(c, 0, 15).astype(np.int64)
            c = c.astype(np.uint8)
            lo, hi = (c[..., 16:], c[..., :16]) if mistake == "q4_nibbles_swapped" else (c[..., :16], c[..., 16:])
            out[..., 2:] = lo | (hi << 4)
        return out.reshape(x.shape[:-1] + (out.shape[-2] * out.shape[-1],))
    return enc


@pytest.mark.parametrize("mistake", ["bf16_truncate", "q4_over_7", "unrounded_scale", "f64_division",
                                     "half_even", "f32_floor", "q4_no_clip", "q4_nibbles_swapped"])
def test_encode_mistakes_fail_pins(mistake):
    from oracle_checks import ENCODE_CHECKS
    bad = _planted_encoder(mistake)
    failed = []
    for check in ENCODE_CHECKS:
        try:
            check(bad)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"planted mistake {mistake!r} passed every encoder pin"


def test_planted_encoder_without_mistake_passes():
    # the harness of the controls is sound: with no mistake every pin passes
    from oracle_checks import ENCODE_CHECKS
    for check in ENCODE_CHECKS:
        check(_planted_encoder(None))
