"""Pins of the oracle's row encoder (the quantiser of a device-side append).

Each test fixes the encoder by something other than its own code: hand-built
blocks whose codes follow from the workload definitions in closed form,
rounding cases decided by IEEE arithmetic, the round trip through the
separately pinned decoder, and invariances of the scale rule."""

import numpy as np
import pytest
import torch

from oracle import encode, quant
from paged_kv_attention_walk_amd import synth
from oracle_checks import ENCODE_CHECKS

KINDS = ("f16", "bf16", "q8_0", "q4_0")


@pytest.mark.parametrize("check", ENCODE_CHECKS, ids=lambda f: f.__name__)
def test_encoder_pins(check):
    check(encode.encode)


@pytest.mark.parametrize("kind", KINDS)
def test_round_trip_error_bound(kind):
    # decode(encode(x)) is within half a quantisation step of x, except the
    # Q4_0 positive extremes, within one step (decoder pinned separately)
    x = np.random.default_rng(7).standard_normal((64, 256)).astype(np.float32) * 3
    y = quant.decode(encode.encode(x, kind), kind)
    err = np.abs(y - x.astype(np.float64))
    if kind == "f16":
        assert np.all(err <= np.abs(x) * 2.0 ** -11 * (1 + 1e-9) + 2.0 ** -25)   # + half a subnormal step
    elif kind == "bf16":
        assert np.all(err <= np.abs(x) * 2.0 ** -8 * (1 + 1e-9))
    else:
        qmax = 127.0 if kind == "q8_0" else 8.0
        blk = x.reshape(64, 8, 32).astype(np.float64)
        amax = np.abs(blk).max(-1, keepdims=True)
        d = amax / qmax
        e = err.reshape(64, 8, 32)
        # half a step of the stored scale, which is within 2^-11 of d
        bound = 0.5 * d * (1 + 2.0 ** -10) + 1e-12
        if kind == "q4_0":
            ext = blk > 7.5 * d * (1 - 2.0 ** -10)     # round to code 16, clipped to 15
            assert np.all(e[~ext] <= np.broadcast_to(bound, e.shape)[~ext])
            # x - 7 d16 <= 8 d - 7 d (1 - 2^-11)
            assert np.all(e[ext] <= np.broadcast_to(d * (1 + 8 * 2.0 ** -11), e.shape)[ext])
        else:
            assert np.all(e <= bound)


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_power_of_two_scaling(kind):
    # multiplying a row by 2^k multiplies every stored scale by 2^k and keeps
    # every code (no fp16 overflow or subnormal scales in this range)
    x = np.random.default_rng(9).standard_normal((16, 256)).astype(np.float32)
    base = encode.encode(x, kind)
    bb = 34 if kind == "q8_0" else 18
    for k in (-6, -1, 3, 7):
        y = encode.encode(x * np.float32(2.0 ** k), kind)
        rb = base.reshape(16, 8, bb)
        ry = y.reshape(16, 8, bb)
        assert np.array_equal(rb[..., 2:], ry[..., 2:])
        ds = rb[..., 0:2].copy().view("<f2").astype(np.float64)
        dy = ry[..., 0:2].copy().view("<f2").astype(np.float64)
        assert np.array_equal(dy, ds * 2.0 ** k)


def test_widening_is_exact():
    h = np.random.default_rng(2).integers(0, 0x7C00, size=1000).astype(np.uint16)
    assert np.array_equal(encode.widen_f16(h).astype(np.float16).view(np.uint16), h)
    b = np.random.default_rng(3).integers(0, 0x7F80, size=1000).astype(np.uint16)
    w = encode.widen_bf16(b)
    assert np.array_equal(torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), b)


@pytest.mark.parametrize("kind", KINDS)
def test_agrees_with_test_data_generator(kind):
    # the seeded pools of the decode tests are written by the generator's own
    # encoders under the same rule; on random data the two give the same bytes
    x = np.random.default_rng(11).standard_normal((200, 256)).astype(np.float32)
    assert np.array_equal(encode.encode(x, kind), synth.encode(x, kind))
