"""ctypes binding of libpa_walk.so (C ABI in include/pa.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  Device buffers are passed as torch tensors (only their data
pointers and the current HIP stream are used) or as raw integer addresses;
host buffers as numpy arrays.  Loading fails loudly when the library has not
been built (``python -m paged_kv_attention_walk_amd.build``); there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa_walk.so")
ABI_VERSION = "0.3.0"      # the library version whose structs this binding mirrors

F16, BF16, Q8_0, Q4_0 = 1, 2, 3, 4
F32 = 5                                   # a source type of pa_append_kv_device only
SRC_CODES = {"f32": F32, "bf16": BF16, "f16": F16}
TYPE_CODES = {"f16": F16, "bf16": BF16, "q8_0": Q8_0, "q4_0": Q4_0}
ROW_BYTES = {F16: 512, BF16: 512, Q8_0: 272, Q4_0: 144}
HEAD_DIM, N_Q_HEADS, N_KV_HEADS, MAX_QTOK = 256, 24, 4, 8

OK, ERR_INVALID, ERR_NOMEM, ERR_STALE, ERR_UNSUPPORTED, ERR_HIP, ERR_NOT_FOUND = 0, -1, -2, -3, -4, -5, -6
DEVERR_TABLE, DEVERR_LENGTH, DEVERR_APPEND = 1, 2, 4
DECODE_VECTOR_REFERENCE = 1
SCRATCH_BYTES = 64 << 20      # PA_SCRATCH_BYTES
POOL_HOST_ONLY = 1

EXPORTS = ("pa_status_string", "pa_version", "pa_row_bytes", "pa_pool_create", "pa_pool_destroy",
           "pa_pool_get_info", "pa_alloc_blocks", "pa_free_blocks", "pa_append_kv", "pa_append_kv_device",
           "pa_decode",
           "pa_decode_workspace_size", "pa_get_device_error", "pa_debug_gather", "pa_prefill",
           "pa_prefill_workspace_size", "pa_split_plan", "pa_read_bandwidth_probe", "pa_split_workgroups_per_cu",
           "pa_read_bandwidth_probe_ex", "pa_decode_scratch")


def kv_type(k, v=0) -> int:
    k = TYPE_CODES.get(k, k)
    v = TYPE_CODES.get(v, v)
    return int(k) | (int(v) << 8)


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().pa_status_string(status).decode()} ({status})")


class PoolDesc(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("page_size", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_type", ctypes.c_int32), ("device", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_append_rows", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p)]


class PoolInfo(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("k_row_bytes", ctypes.c_size_t),
                ("v_row_bytes", ctypes.c_size_t), ("k_page_bytes", ctypes.c_size_t),
                ("v_page_bytes", ctypes.c_size_t), ("n_blocks", ctypes.c_int32), ("n_free", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("kv_type", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("device", ctypes.c_int32)]


class DecodeExt(ctypes.Structure):
    _fields_ = [("bt_stride", ctypes.c_int32), ("n_pool_blocks", ctypes.c_int32), ("scale", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("lse_out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("split_events", ctypes.c_void_p * 2),
                ("seq_lens_host", ctypes.c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_walk_amd.build` "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, VP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        sig = {
            "pa_status_string": (ctypes.c_char_p, [I32]),
            "pa_version": (ctypes.c_char_p, []),
            "pa_row_bytes": (SZ, [I32]),
            "pa_pool_create": (I32, [ctypes.POINTER(PoolDesc), ctypes.POINTER(P)]),
            "pa_pool_destroy": (I32, [P]),
            "pa_pool_get_info": (I32, [P, ctypes.POINTER(PoolInfo)]),
            "pa_alloc_blocks": (I32, [P, I32, VP, VP]),
            "pa_free_blocks": (I32, [P, I32, VP]),
            "pa_append_kv": (I32, [P, I32, VP, VP, VP, VP, VP]),
            "pa_append_kv_device": (I32, [P, I32, VP, VP, VP, VP, I32, VP, VP]),
            "pa_decode": (I32, [VP, VP, VP, VP, VP, I32, I32, I32, I32, VP, VP, ctypes.POINTER(DecodeExt)]),
            "pa_decode_workspace_size": (I32, [I32, I32, I32, ctypes.POINTER(SZ)]),
            "pa_decode_scratch": (I32, [VP, VP, VP, VP, VP, I32, I32, I32, I32, VP, VP, ctypes.POINTER(DecodeExt)]),
            "pa_prefill": (I32, [VP, VP, VP, VP, VP, I32, I32, I32, I32, VP, VP, ctypes.POINTER(DecodeExt)]),
            "pa_prefill_workspace_size": (I32, [I32, I32, I32, ctypes.POINTER(SZ)]),
            "pa_get_device_error": (I32, [P, VP, VP, I32, ctypes.POINTER(I32)]),
            "pa_debug_gather": (I32, [VP, I32, VP, I32, I32, I32, I32, I32, VP, VP, VP]),
            "pa_split_plan": (I32, [VP, I32, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32), VP]),
            "pa_read_bandwidth_probe": (I32, [VP, SZ, VP, SZ, VP]),
            "pa_read_bandwidth_probe_ex": (I32, [VP, SZ, VP, SZ, I32, I32, ctypes.c_uint32, VP]),
            "pa_split_workgroups_per_cu": (I32, [I32, I32, ctypes.c_uint32, ctypes.POINTER(I32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        got = lib.pa_version().decode()
        if got != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} is version {got}, this binding mirrors {ABI_VERSION}: rebuild it with "
                               "`python -m paged_kv_attention_walk_amd.build`")
        _LIB = lib
    return _LIB


def lib():
    """The loaded library (ctypes.CDLL)."""
    return _lib()


def version() -> str:
    return _lib().pa_version().decode()


def _check(status: int, what: str):
    if status != OK:
        raise PaError(status, what)


def _ptr(x):
    """Address of a torch tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be C-contiguous")
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("device tensors must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_size(n_seq: int, n_qtok: int, device: int = 0) -> int:
    n = ctypes.c_size_t()
    _check(_lib().pa_decode_workspace_size(n_seq, n_qtok, device, ctypes.byref(n)), "pa_decode_workspace_size")
    return n.value


class Pool:
    """A pa_pool.  ``k_pool``/``v_pool`` may be caller-owned device tensors
    (kept referenced here) or None for library-owned memory."""

    def __init__(self, n_blocks, page_size, kv, *, device=0, max_seqs=0, max_blocks_per_seq=0,
                 max_append_rows=0, host_only=False, k_pool=None, v_pool=None):
        self._keep = (k_pool, v_pool)
        d = PoolDesc(n_blocks=n_blocks, page_size=page_size, n_kv_heads=N_KV_HEADS, head_dim=HEAD_DIM,
                     kv_type=kv if isinstance(kv, int) else kv_type(kv), device=device, max_seqs=max_seqs,
                     max_blocks_per_seq=max_blocks_per_seq, max_append_rows=max_append_rows,
                     flags=POOL_HOST_ONLY if host_only else 0, k_pool=_ptr(k_pool), v_pool=_ptr(v_pool))
        h = ctypes.c_void_p()
        self._h = None
        _check(_lib().pa_pool_create(ctypes.byref(d), ctypes.byref(h)), "pa_pool_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def info(self) -> PoolInfo:
        i = PoolInfo()
        _check(_lib().pa_pool_get_info(self._h, ctypes.byref(i)), "pa_pool_get_info")
        return i

    def alloc(self, n: int):
        """Returns (handles uint64[n], indices int32[n]); raises PaError."""
        hs = np.zeros(max(n, 1), dtype=np.uint64)
        ix = np.zeros(max(n, 1), dtype=np.int32)
        _check(_lib().pa_alloc_blocks(self._h, n, hs.ctypes.data, ix.ctypes.data), "pa_alloc_blocks")
        return hs[:n], ix[:n]

    def alloc_status(self, n: int, handles=True, indices=True):
        hs = np.zeros(max(n, 1), dtype=np.uint64)
        ix = np.zeros(max(n, 1), dtype=np.int32)
        st = _lib().pa_alloc_blocks(self._h, n, hs.ctypes.data if handles else None,
                                    ix.ctypes.data if indices else None)
        return st, hs[:max(n, 0)], ix[:max(n, 0)]

    def free(self, handles):
        hs = np.ascontiguousarray(np.asarray(handles, dtype=np.uint64))
        _check(_lib().pa_free_blocks(self._h, len(hs), hs.ctypes.data if len(hs) else None), "pa_free_blocks")

    def free_status(self, handles) -> int:
        hs = np.ascontiguousarray(np.asarray(handles, dtype=np.uint64))
        return _lib().pa_free_blocks(self._h, len(hs), hs.ctypes.data if len(hs) else None)

    def append_kv(self, blocks, slots, k_rows, v_rows, stream=None) -> int:
        b = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32))
        s = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
        k = np.ascontiguousarray(k_rows, dtype=np.uint8)
        v = np.ascontiguousarray(v_rows, dtype=np.uint8)
        return _lib().pa_append_kv(self._h, len(b), _ptr(b), _ptr(s), _ptr(k), _ptr(v), _stream(stream))

    def append_kv_device_status(self, n_rows, blocks, slots, k_src, v_src, src_type, err_word=None,
                                stream=None) -> int:
        """pa_append_kv_device: device int32 ``blocks`` / ``slots`` and device
        rows [n_rows][4][256] of ``src_type`` ("f32", "bf16", "f16" or a code)."""
        st = SRC_CODES.get(src_type, src_type)
        return _lib().pa_append_kv_device(self._h, int(n_rows), _ptr(blocks), _ptr(slots), _ptr(k_src),
                                          _ptr(v_src), int(st), _ptr(err_word), _stream(stream))

    def append_kv_device(self, blocks, slots, k_src, v_src, src_type="f32", err_word=None, stream=None):
        n = int(blocks.shape[0])
        _check(self.append_kv_device_status(n, blocks, slots, k_src, v_src, src_type, err_word, stream),
               "pa_append_kv_device")

    def device_error(self, stream=None, clear=True) -> int:
        e = ctypes.c_int32()
        _check(_lib().pa_get_device_error(self._h, None, _stream(stream), int(clear), ctypes.byref(e)),
               "pa_get_device_error")
        return e.value

    def destroy(self):
        if self._h is not None:
            _lib().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def make_ext(bt_stride, n_pool_blocks=0, scale=0.0, lse_out=None, workspace=None, workspace_bytes=None,
             split_events=None, flags=0, seq_lens_host=None) -> DecodeExt:
    e = DecodeExt(bt_stride=int(bt_stride), n_pool_blocks=int(n_pool_blocks), scale=float(scale), flags=int(flags),
                  lse_out=_ptr(lse_out), workspace=_ptr(workspace),
                  workspace_bytes=int(workspace_bytes if workspace_bytes is not None else
                                      (workspace.numel() * workspace.element_size() if workspace is not None else 0)))
    if split_events is not None:
        e.split_events[0] = split_events[0]
        e.split_events[1] = split_events[1]
    if seq_lens_host is not None:
        # host int32 copy of seq_lens: the plan is computed on the host; the
        # array is kept alive with the struct
        lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
        e._seq_lens_host = lens
        e.seq_lens_host = lens.ctypes.data
    return e


def decode_status(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv, page_size, out,
                  stream=None, ext: DecodeExt | None = None) -> int:
    """pa_decode; returns the status code."""
    return _lib().pa_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                            int(n_seq), int(n_qtok), kv if isinstance(kv, int) else kv_type(kv), int(page_size),
                            _ptr(out), _stream(stream), ctypes.byref(ext) if ext is not None else None)


def prefill_status(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv, page_size, out,
                   stream=None, ext: DecodeExt | None = None) -> int:
    """pa_prefill; returns the status code."""
    return _lib().pa_prefill(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                             int(n_seq), int(n_qtok), kv if isinstance(kv, int) else kv_type(kv), int(page_size),
                             _ptr(out), _stream(stream), ctypes.byref(ext) if ext is not None else None)


def split_workgroups_per_cu(kv, n_qtok=1, flags=0) -> int:
    """pa_split_workgroups_per_cu on the current device."""
    w = ctypes.c_int32()
    _check(_lib().pa_split_workgroups_per_cu(kv if isinstance(kv, int) else kv_type(kv), int(n_qtok), int(flags),
                                             ctypes.byref(w)), "pa_split_workgroups_per_cu")
    return w.value


def split_plan(seq_lens, cap, n_cu=256, wgs_per_cu=2):
    """pa_split_plan: (chunk, n_items, first[n_seq + 1]) of a one-token decode
    call, computed on the host."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    n = int(lens.shape[0])
    chunk, items = ctypes.c_int32(), ctypes.c_int32()
    first = np.zeros(n + 1, dtype=np.int32)
    _check(_lib().pa_split_plan(lens.ctypes.data if n else None, n, int(cap), int(n_cu), int(wgs_per_cu),
                                ctypes.byref(chunk), ctypes.byref(items), first.ctypes.data), "pa_split_plan")
    return chunk.value, items.value, first


def read_bandwidth_probe(src, sink, stream=None):
    """pa_read_bandwidth_probe over the whole of device tensor `src` (its size
    a multiple of 16 bytes), folding into device int32/uint32 tensor `sink`."""
    _check(_lib().pa_read_bandwidth_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(),
                                          _stream(stream)), "pa_read_bandwidth_probe")


PROBE_SLICE, PROBE_LDS = 1, 2


def read_bandwidth_probe_ex(src, sink, wgs_per_cu, loads_in_flight, flags=0, stream=None):
    """pa_read_bandwidth_probe_ex: the probe with an explicit configuration."""
    _check(_lib().pa_read_bandwidth_probe_ex(_ptr(src), src.numel() * src.element_size(), _ptr(sink), sink.numel(),
                                             int(wgs_per_cu), int(loads_in_flight), int(flags), _stream(stream)),
           "pa_read_bandwidth_probe_ex")


def prefill_workspace_size(n_seq, n_qtok, device=0) -> int:
    n = ctypes.c_size_t()
    _check(_lib().pa_prefill_workspace_size(int(n_seq), int(n_qtok), int(device), ctypes.byref(n)),
           "pa_prefill_workspace_size")
    return n.value


def decode(q, k_pool, v_pool, block_table, seq_lens, n_qtok, kv, page_size, out, *, n_seq=None, stream=None,
           ext: DecodeExt | None = None):
    n = int(seq_lens.shape[0]) if n_seq is None else int(n_seq)
    _check(decode_status(q, k_pool, v_pool, block_table, seq_lens, n, n_qtok, kv, page_size, out, stream, ext),
           "pa_decode")
    return out


def decode_scratch_status(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv, page_size, out, stream,
                          ext: DecodeExt) -> int:
    """pa_decode_scratch (the workspace is the library's static device
    buffer; ext is required and carries no workspace); returns the status."""
    return _lib().pa_decode_scratch(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                                    int(n_seq), int(n_qtok), kv if isinstance(kv, int) else kv_type(kv),
                                    int(page_size), _ptr(out), _stream(stream),
                                    ctypes.byref(ext) if ext is not None else None)


def scratch_device_error(stream=None, clear=True) -> int:
    """The error word of pa_decode_scratch's buffer on the current device."""
    e = ctypes.c_int32()
    _check(_lib().pa_get_device_error(None, None, _stream(stream), int(clear), ctypes.byref(e)),
           "pa_get_device_error")
    return e.value


def device_error(workspace, stream=None, clear=True) -> int:
    e = ctypes.c_int32()
    _check(_lib().pa_get_device_error(None, _ptr(workspace), _stream(stream), int(clear), ctypes.byref(e)),
           "pa_get_device_error")
    return e.value


def debug_gather(pool, row_bytes, block_table, bt_stride, n_pool_blocks, seq, seq_len, page_size, dst,
                 err_word=None, stream=None):
    _check(_lib().pa_debug_gather(_ptr(pool), int(row_bytes), _ptr(block_table), int(bt_stride),
                                  int(n_pool_blocks), int(seq), int(seq_len), int(page_size), _ptr(dst),
                                  _ptr(err_word), _stream(stream)), "pa_debug_gather")
    return dst
