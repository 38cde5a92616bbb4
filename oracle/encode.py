"""Encoding of float rows into the four K/V encodings (oracle; test
infrastructure only).

This is what a device-side append computes before it scatters a new row into
its page: K/V rows produced in float32 (or bf16 / f16, widened exactly to
float32) are written in the pool's encoding.  The formats themselves are
those ``quant`` decodes.  The pages fix, for the two block formats, the scale
of a block of 32 values (the workload definitions of Q4_0: fp16 scale
d = max|x|/8, codes 0..15, value (q-8)*d; and of Q8_0: fp16 scale
d = max|x|/127, int8 codes, value q*d), and colibri#372 (Summary) the append
step that uploads only the new rows and scatters them.  They say nothing more
about how codes are chosen.  Readings taken here, each the plainest one the
formats support:

* d is computed in float32 (max|x| / 8 or / 127, one correctly rounded
  division) and stored as the nearest fp16 value, ties to even;
* codes are chosen against the stored scale: c = round(x * r) with
  r = 1 / float(d16) (float32), the product rounded to float32, and round
  taking halves away from zero.  Floating point decides an integer here, so
  the decision is made in float32, the precision of the device encoder;
* Q4_0 stores c + 8 clipped to [0, 15]: a block's positive extreme gives 16
  and is stored as 15 (it decodes to 7d); Q8_0 clips to [-127, 127];
* a block of zeros has d = 0, r = 0 and codes 8 (Q4_0) / 0 (Q8_0);
* F16 and BF16 rows are the values rounded to nearest, ties to even.

Inputs must be finite; a block whose scale overflows fp16 (max|x| above
8 x 65504 for Q4_0) stores d = inf and codes 8 / 0.
"""

import numpy as np
import torch

QBLOCK = 32


def widen_f16(bits: np.ndarray) -> np.ndarray:
    """float32 values of little-endian binary16 bit patterns (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns: the pattern is the top half of
    the binary32 one (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_half_away(v: np.ndarray) -> np.ndarray:
    """Nearest integer, halves away from zero, of float32 values.  Evaluated in
    float64, where v + 0.5 is exact for every float32 v of the code range."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    return np.where(v >= 0, np.floor(v + 0.5), -np.floor(0.5 - v))


def block_scale(blocks: np.ndarray, qmax: float):
    """fp16 scale d = max|x| / qmax of each block of 32 float32 values, and the
    float32 reciprocal r of the stored scale (0 where d is 0)."""
    blocks = np.asarray(blocks, dtype=np.float32)
    amax = np.max(np.abs(blocks), axis=-1)                        # exact
    d16 = (amax / np.float32(qmax)).astype(np.float32).astype(np.float16)
    d32 = d16.astype(np.float32)
    r = np.zeros_like(d32)
    nz = d32 != 0
    r[nz] = np.float32(1.0) / d32[nz]
    return d16, r


def _codes(blocks: np.ndarray, r: np.ndarray) -> np.ndarray:
    prod = (np.asarray(blocks, dtype=np.float32) * r[..., None]).astype(np.float32)
    return round_half_away(prod)


def encode_q8_0(x: np.ndarray) -> np.ndarray:
    """[..., 256] float32 -> [..., 272] bytes: per block the fp16 scale, then
    32 int8 codes clip(round(x r), -127, 127)."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(lead + (D // QBLOCK, QBLOCK))
    d16, r = block_scale(blk, 127.0)
    c = np.clip(_codes(blk, r), -127, 127).astype(np.int8)
    out = np.empty(blk.shape[:-1] + (2 + QBLOCK,), dtype=np.uint8)
    out[..., 0:2] = d16.astype("<f2")[..., None].view(np.uint8)
    out[..., 2:] = c.view(np.uint8)
    return out.reshape(lead + (D // QBLOCK * (2 + QBLOCK),))


def encode_q4_0(x: np.ndarray) -> np.ndarray:
    """[..., 256] float32 -> [..., 144] bytes: per block the fp16 scale, then
    16 bytes; byte j holds code j in its low nibble and code j + 16 in its
    high nibble, codes clip(round(x r) + 8, 0, 15)."""
    x = np.asarray(x, dtype=np.float32)
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.reshape(lead + (D // QBLOCK, QBLOCK))
    d16, r = block_scale(blk, 8.0)
    c = np.clip(_codes(blk, r) + 8, 0, 15).astype(np.uint8)
    out = np.empty(blk.shape[:-1] + (2 + QBLOCK // 2,), dtype=np.uint8)
    out[..., 0:2] = d16.astype("<f2")[..., None].view(np.uint8)
    out[..., 2:] = c[..., :16] | (c[..., 16:] << 4)
    return out.reshape(lead + (D // QBLOCK * (2 + QBLOCK // 2),))


def encode_f16(x: np.ndarray) -> np.ndarray:
    """Nearest binary16 values (ties to even), little-endian bytes."""
    x = np.asarray(x, dtype=np.float32)
    return np.ascontiguousarray(x.astype("<f2")).view(np.uint8).reshape(x.shape[:-1] + (2 * x.shape[-1],))


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 values (ties to even, by torch's conversion),
    little-endian bytes."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return np.ascontiguousarray(b.astype("<u2")).view(np.uint8).reshape(x.shape[:-1] + (2 * x.shape[-1],))


ENCODERS = {"f16": encode_f16, "bf16": encode_bf16, "q8_0": encode_q8_0, "q4_0": encode_q4_0}


def encode(x: np.ndarray, kind: str) -> np.ndarray:
    """Encode ``[..., 256]`` float32 values as rows of encoding ``kind``."""
    try:
        fn = ENCODERS[kind]
    except KeyError:
        raise ValueError(f"unknown K/V encoding {kind!r}") from None
    return fn(x)
