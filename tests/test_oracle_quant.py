"""Pins of the oracle's row decoding (CPU)."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import quant
from paged_kv_attention_walk_amd import synth
from oracle_checks import check_closed_forms, check_scale_position


def test_row_bytes():
    assert quant.row_bytes("f16") == 512
    assert quant.row_bytes("bf16") == 512
    assert quant.row_bytes("q8_0") == 8 * 34
    assert quant.row_bytes("q4_0") == 8 * 18
    with pytest.raises(ValueError):
        quant.row_bytes("q5_1")


def test_closed_forms():
    check_closed_forms(quant.decode)


def test_scale_position(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "q4_0_scale_position_llamacpp_pr2.json")))
    assert fx["row_bytes"] == quant.row_bytes("q4_0")
    check_scale_position(quant.decode, fx)


def test_q8_0_fragment_offsets():
    # 8-quant fragments of a 34-byte block start at an even row offset whose
    # value mod 8 depends on the block alone (llama.cpp PR 2, LDS-read commit).
    for b in range(8):
        offs = {(34 * b + 2 + 8 * f) % 8 for f in range(4)}
        assert len(offs) == 1 and offs.pop() % 2 == 0


def test_zero_block_and_extremes():
    # all-zero block: scale 0 gives zeros whatever the codes
    row = np.zeros(144, dtype=np.uint8)
    row[2:18] = 0xFF
    assert np.all(quant.decode(row[None], "q4_0")[0][:32] == 0)
    # Q4_0 codes 0 and 15 with d = 65504 (largest half): -8*d and 7*d exactly
    row = np.zeros(144, dtype=np.uint8)
    row[0:2] = np.frombuffer(np.float16(65504).tobytes(), np.uint8)
    row[2:18] = 0xF0                                  # low nibble 0, high 15
    got = quant.decode(row[None], "q4_0")[0]
    assert np.all(got[:16] == -8 * 65504.0) and np.all(got[16:32] == 7 * 65504.0)
    # Q8_0 code -128 is a legal byte: decodes to -128 * d
    row = np.zeros(272, dtype=np.uint8)
    row[0:2] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    row[2] = 0x80
    assert quant.decode(row[None], "q8_0")[0][0] == -64.0


@pytest.mark.parametrize("kind", oracle.TYPES)
def test_round_trip_error_bound(kind):
    # Encoding random values then decoding stays within the encoding's own
    # step: |x - decode(encode(x))| <= step/2 (+ the fp16 scale's rounding).
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    y = quant.decode(synth.encode(x, kind), kind)
    blk = np.abs(x.reshape(64, 8, 32)).max(-1)
    if kind == "f16":
        assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -11 + 2.0 ** -25)
    elif kind == "bf16":
        assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8 + 1e-38)
    elif kind == "q8_0":
        step = blk / 127
        err = np.abs(y - x).reshape(64, 8, 32).max(-1)
        assert np.all(err <= 0.5 * step * (1 + 2 ** -10) + 1e-7)
    else:
        step = blk / 8
        err = np.abs(y - x).reshape(64, 8, 32).max(-1)
        # the positive extreme may clip from 8*d to 7*d: error up to one step
        # plus 7 times the fp16 scale's rounding
        assert np.all(err <= step * (1 + 8 * 2 ** -11) + 1e-7)


def test_decode_rejects_bad_shapes():
    with pytest.raises(ValueError):
        quant.decode(np.zeros((1, 100), np.uint8), "q4_0")
    with pytest.raises(TypeError):
        quant.decode(np.zeros((1, 144), np.int16), "q4_0")
