"""Decoding of stored K/V rows to float64 (oracle; test infrastructure only).

A K or V row is one head's 256-wide vector for one position.  The pages name
four encodings:

* F16 and BF16 rows: 256 two-byte values (lucebox#555, Summary, lists F16;
  TensorFold#1156, Summary, keeps bf16 K/V of 4 heads x 256 per layer).
* Q8_0: blocks of 32 values, each block a 2-byte fp16 scale followed by 32
  signed 8-bit codes, 34 bytes in all (llama.cpp-PR2, LDS-read commit, which
  calls them 34-byte blocks); value = code * scale (the Q8_0 workload
  definition: int8 codes, value q*d).
* Q4_0: blocks of 32 values, a 2-byte fp16 scale followed by 16 bytes holding
  32 four-bit codes, 18 bytes in all.  The size follows from lucebox#555, K/V
  capacity: 1,048,576 padded slots take 1152 MiB for one layer, i.e. 1152
  bytes per position = 4 KV heads x (K + V) x 144 bytes = 8 blocks x 18.
  That the scale comes first is fixed by llama.cpp-PR2, LDS-read commit: the
  scale of block v of a row sits at byte 2*v of the row's 16-byte piece v,
  i.e. at byte 18*v.  value = (code - 8) * scale (the Q4_0 workload
  definition: codes 0..15, value (q-8)*d).

Reading where the pages are silent: which nibble of a Q4_0 byte holds which
element.  The pages fix only sizes and the value formula.  This oracle takes
the common GGML convention: byte j of a block's code bytes holds element j in
its low nibble and element j + 16 in its high nibble.  Scales are
little-endian IEEE half precision.
"""

import numpy as np

HEAD_DIM = 256
QBLOCK = 32                      # values per quantisation block
Q8_0_BLOCK_BYTES = 2 + QBLOCK    # 34
Q4_0_BLOCK_BYTES = 2 + QBLOCK // 2  # 18


def row_bytes(kind: str, head_dim: int = HEAD_DIM) -> int:
    """Bytes of one encoded row of ``head_dim`` values."""
    if kind in ("f16", "bf16"):
        return 2 * head_dim
    if kind == "q8_0":
        return head_dim // QBLOCK * Q8_0_BLOCK_BYTES
    if kind == "q4_0":
        return head_dim // QBLOCK * Q4_0_BLOCK_BYTES
    raise ValueError(f"unknown K/V encoding {kind!r}")


def _as_u8(rows: np.ndarray, kind: str, head_dim: int) -> np.ndarray:
    rows = np.ascontiguousarray(rows)
    if rows.dtype != np.uint8:
        raise TypeError("encoded rows must be uint8 arrays")
    rb = row_bytes(kind, head_dim)
    if rows.shape[-1] != rb:
        raise ValueError(f"{kind} rows of {head_dim} values have {rb} bytes, got {rows.shape[-1]}")
    return rows


def _half_le(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """IEEE binary16 from two little-endian bytes, as float64."""
    bits = lo.astype(np.uint16) | (hi.astype(np.uint16) << np.uint16(8))
    return bits.view(np.float16).astype(np.float64)


def decode_f16(rows: np.ndarray, head_dim: int = HEAD_DIM) -> np.ndarray:
    """F16 rows (lucebox#555, Summary): little-endian binary16 values."""
    r = _as_u8(rows, "f16", head_dim)
    return _half_le(r[..., 0::2], r[..., 1::2])


def decode_bf16(rows: np.ndarray, head_dim: int = HEAD_DIM) -> np.ndarray:
    """BF16 rows (TensorFold#1156, Summary): the top 16 bits of a binary32."""
    r = _as_u8(rows, "bf16", head_dim)
    bits = r[..., 0::2].astype(np.uint32) | (r[..., 1::2].astype(np.uint32) << np.uint32(8))
    return (bits << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_q8_0(rows: np.ndarray, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Q8_0 rows: per 34-byte block, fp16 scale d then 32 int8 codes c; x = c*d
    (llama.cpp-PR2, LDS-read commit, for the block size; the Q8_0 workload
    definition for the value)."""
    r = _as_u8(rows, "q8_0", head_dim)
    nb = head_dim // QBLOCK
    blk = r.reshape(r.shape[:-1] + (nb, Q8_0_BLOCK_BYTES))
    d = _half_le(blk[..., 0], blk[..., 1])                     # [..., nb]
    codes = blk[..., 2:].view(np.int8).astype(np.float64)       # [..., nb, 32]
    return (codes * d[..., None]).reshape(r.shape[:-1] + (head_dim,))


def decode_q4_0(rows: np.ndarray, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Q4_0 rows: per 18-byte block, fp16 scale d then 16 code bytes; byte j
    gives element j (low nibble) and element j+16 (high nibble); x = (c-8)*d
    (lucebox#555, K/V capacity, for the size; llama.cpp-PR2, LDS-read commit,
    for the scale position; the Q4_0 workload definition for the value)."""
    r = _as_u8(rows, "q4_0", head_dim)
    nb = head_dim // QBLOCK
    blk = r.reshape(r.shape[:-1] + (nb, Q4_0_BLOCK_BYTES))
    d = _half_le(blk[..., 0], blk[..., 1])
    code_bytes = blk[..., 2:]                                   # [..., nb, 16]
    lo = (code_bytes & 0x0F).astype(np.int64)
    hi = (code_bytes >> 4).astype(np.int64)
    codes = np.concatenate([lo, hi], axis=-1)                   # element j, then j+16
    return ((codes - 8).astype(np.float64) * d[..., None]).reshape(r.shape[:-1] + (head_dim,))


DECODERS = {
    "f16": decode_f16,
    "bf16": decode_bf16,
    "q8_0": decode_q8_0,
    "q4_0": decode_q4_0,
}


def decode(rows: np.ndarray, kind: str, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Decode ``[..., row_bytes]`` uint8 rows of encoding ``kind`` to float64."""
    try:
        fn = DECODERS[kind]
    except KeyError:
        raise ValueError(f"unknown K/V encoding {kind!r}") from None
    return fn(rows, head_dim)
