"""The C ABI library on the CPU: it loads, exports every declared symbol,
its allocator matches the allocator model bit for bit, and host-side argument
checks fail before anything reaches the device.  No compute call is made."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import alloc_model as am
from paged_kv_attention_walk_amd import binding as pb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "pa_decode" in names and "pa_append_kv" in names and "pa_append_kv_device" in names
    assert "pa_prefill" in names and len(names) >= 16
    lib = pb.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(pb.EXPORTS) == set(names)
    assert pb.version().count(".") == 2
    assert pb.version() == pb.ABI_VERSION


def test_row_bytes_and_status_strings():
    lib = pb.lib()
    assert [lib.pa_row_bytes(t) for t in (1, 2, 3, 4, 5)] == [512, 512, 272, 144, 0]
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert lib.pa_status_string(s)


def _host_pool(n, P=16, kv="q4_0"):
    return pb.Pool(n, P, kv, host_only=True)


def test_allocator_matches_model_random_histories():
    rng = np.random.default_rng(5)
    for n_blocks in (1, 63, 64, 65, 300):
        pool = _host_pool(n_blocks)
        model = am.AllocModel(n_blocks)
        live = []
        for step in range(1500):
            r = rng.random()
            if r < 0.45:
                n = int(rng.integers(0, 9))
                st, h, ix = pool.alloc_status(n)
                mst, mh, mix = model.alloc(n)
                assert {pb.OK: am.OK, pb.ERR_NOMEM: am.NOMEM}[st] == mst
                if st == pb.OK:
                    assert list(h) == mh and list(ix) == mix
                    live += mh
            elif r < 0.9 and live:
                k = int(rng.integers(1, min(5, len(live)) + 1))
                pick = [live[i] for i in rng.choice(len(live), size=k, replace=False)]
                if rng.random() < 0.15:
                    pick.append(pick[0])
                if rng.random() < 0.1:
                    pick.append(am.handle(7, int(rng.integers(0, n_blocks))))   # forged generation
                st = pool.free_status(pick)
                mst = model.free_handles(pick)
                assert {pb.OK: am.OK, pb.ERR_STALE: am.STALE, pb.ERR_INVALID: am.INVALID}[st] == mst
                if st == pb.OK:
                    for x in pick:
                        live.remove(x)
            else:
                # stale handle: an old generation of an index that is live or free
                if live:
                    g, i = am.split(live[0])
                    st = pool.free_status([am.handle(g + 1 if g < 0xFFFFFFFF else 1, i)])
                    assert st == pb.ERR_STALE
            assert pool.info().n_free == model.n_free
        pool.destroy()


def test_allocator_edge_cases():
    pool = _host_pool(4)
    assert pool.alloc_status(0)[0] == pb.OK
    assert pool.alloc_status(-1)[0] == pb.ERR_INVALID
    assert pool.alloc_status(2, handles=False, indices=False)[0] == pb.ERR_INVALID
    st, h, ix = pool.alloc_status(2, handles=False)
    assert st == pb.OK and list(ix) == [0, 1]
    assert pool.alloc_status(3)[0] == pb.ERR_NOMEM and pool.info().n_free == 2
    assert pool.free_status([am.handle(1, 4)]) == pb.ERR_INVALID      # index out of range
    assert pool.free_status([am.handle(1, 2)]) == pb.ERR_STALE        # not allocated
    assert pool.free_status([am.handle(1, 0), am.handle(1, 1)]) == pb.OK
    assert pool.free_status([am.handle(1, 0)]) == pb.ERR_STALE        # double free
    assert pool.info().n_free == 4
    pool.destroy()


def test_pool_create_rejects_bad_descriptors():
    for kwargs, status in [(dict(n_blocks=0, page_size=16, kv="f16"), pb.ERR_INVALID),
                           (dict(n_blocks=4, page_size=24, kv="f16"), pb.ERR_UNSUPPORTED),
                           (dict(n_blocks=4, page_size=1024, kv="f16"), pb.ERR_UNSUPPORTED),
                           (dict(n_blocks=4, page_size=16, kv=9), pb.ERR_INVALID)]:
        with pytest.raises(pb.PaError) as e:
            pb.Pool(kwargs["n_blocks"], kwargs["page_size"], kwargs["kv"], host_only=True)
        assert e.value.status == status
    p = pb.Pool(4, 48, "bf16", host_only=True)                         # 48: non-power-of-two page
    assert p.info().page_size == 48
    p.destroy()
    p = pb.Pool(4, 16, pb.kv_type("q8_0", "q4_0"), host_only=True)     # K and V of different types
    info = p.info()
    assert (info.k_row_bytes, info.v_row_bytes) == (272, 144)
    assert (info.k_page_bytes, info.v_page_bytes) == (4 * 16 * 272, 4 * 16 * 144)
    p.destroy()


def test_decode_host_checks_fail_before_device_work():
    # Fake, never-dereferenced addresses: every call must fail in host checks.
    a = 1 << 20
    kvq4 = pb.kv_type("q4_0")
    st = lambda **kw: pb.decode_status(**{**dict(q=a, k_pool=a, v_pool=a, block_table=a, seq_lens=a, n_seq=1,
                                                  n_qtok=1, kv=kvq4, page_size=16, out=a, stream=0), **kw})
    assert st(n_qtok=0) == pb.ERR_INVALID
    assert st(n_qtok=9) == pb.ERR_INVALID
    assert st(n_qtok=8) == pb.ERR_NOT_FOUND               # 8 tokens pass the checks
    assert st(n_seq=-1) == pb.ERR_INVALID
    assert st(kv=0x10000 | 4) == pb.ERR_INVALID
    assert st(kv=pb.kv_type("q4_0", "f16")) == pb.ERR_NOT_FOUND     # a mixed pair passes the type checks
    assert st(page_size=40) == pb.ERR_UNSUPPORTED
    assert st(q=a + 4) == pb.ERR_INVALID                  # misaligned
    assert st(k_pool=a + 8) == pb.ERR_INVALID
    assert st(out=None) == pb.ERR_INVALID
    assert st() == pb.ERR_NOT_FOUND                        # no ext and not a pool's K pointer
    assert st(n_seq=0) == pb.OK                            # nothing to do
    e = pb.make_ext(bt_stride=0)
    assert st(ext=e) == pb.ERR_INVALID
    e = pb.make_ext(bt_stride=4, n_pool_blocks=8)
    e.flags = 2                                             # unknown flag
    assert st(ext=e) == pb.ERR_INVALID


def test_append_host_checks():
    pool = _host_pool(8)
    z = np.zeros((1, 4, 144), np.uint8)
    assert pool.append_kv([0], [0], z, z, stream=0) == pb.ERR_INVALID       # host-only pool
    pool.destroy()


def test_append_device_host_checks():
    pool = _host_pool(8)
    a = 1 << 20
    st = lambda **kw: pool.append_kv_device_status(**{**dict(n_rows=3, blocks=a, slots=a, k_src=a, v_src=a,
                                                              src_type="f32", stream=0), **kw})
    assert st(src_type=9) == pb.ERR_INVALID
    assert st(src_type=pb.Q4_0) == pb.ERR_INVALID            # an encoding, not a source type
    assert st(n_rows=-1) == pb.ERR_INVALID
    assert st(n_rows=0) == pb.OK                             # nothing to do
    assert st(blocks=None) == pb.ERR_INVALID
    assert st() == pb.ERR_INVALID                            # host-only pool: no device memory
    for src in ("f32", "bf16", "f16"):
        assert st(src_type=src) == pb.ERR_INVALID
    pool.destroy()
    assert pb.lib().pa_append_kv_device(None, 1, a, a, a, a, pb.F32, None, None) == pb.ERR_INVALID


def test_prefill_host_checks_and_workspace():
    a = 1 << 20
    kvq = pb.kv_type("q4_0")
    st = lambda **kw: pb.prefill_status(**{**dict(q=a, k_pool=a, v_pool=a, block_table=a, seq_lens=a, n_seq=1,
                                                   n_qtok=100, kv=kvq, page_size=16, out=a, stream=0), **kw})
    assert st(n_qtok=0) == pb.ERR_INVALID
    assert st(n_qtok=65537) == pb.ERR_INVALID
    assert st() == pb.ERR_NOT_FOUND                       # passes the checks; no ext and no pool
    assert st(n_qtok=65536) == pb.ERR_NOT_FOUND
    assert st(q=a + 4) == pb.ERR_INVALID
    # a workspace of exactly pa_prefill_workspace_size() bytes is accepted, one
    # item (48 rows of 257 floats) less is not
    for n_seq in (1, 3, 64):
        for T in (1, 9, 17, 100, 4096):
            n = pb.prefill_workspace_size(n_seq, T, 0)
            ok = pb.make_ext(8, 64, 0.0, None, 1 << 30, n)
            assert pb.prefill_status(a, a, a, a, a, n_seq, T, kvq, 16, a, 0, ok) != pb.ERR_INVALID, (n_seq, T)
            small = pb.make_ext(8, 64, 0.0, None, 1 << 30, n - 48 * 257 * 4)
            assert pb.prefill_status(a, a, a, a, a, n_seq, T, kvq, 16, a, 0, small) == pb.ERR_INVALID, (n_seq, T)
    # a dispatch holds at most 2^32 - 1 work items (16777215 workgroups of
    # 256): 10 sequences of 65536 tokens fit the merge grid (15.7M query
    # rows), 11 do not (17.3M) and are refused before anything is enqueued
    for n_seq, want_unsupported in ((10, False), (11, True)):
        n = pb.prefill_workspace_size(n_seq, 65536, 0)
        ext = pb.make_ext(4096, 64, 0.0, None, 1 << 30, n)
        got = pb.prefill_status(a, a, a, a, a, n_seq, 65536, kvq, 16, a, 0, ext)
        assert (got == pb.ERR_UNSUPPORTED) == want_unsupported, (n_seq, got)
        assert got != pb.ERR_INVALID


def test_workspace_size_is_accepted_and_needed():
    # pa_decode must accept a workspace of exactly pa_decode_workspace_size()
    # bytes for every n_seq / n_qtok, and refuse one a work item (6 n_qtok
    # rows of 257 floats) smaller; a workspace sized for 8 tokens serves every
    # n_qtok.  On a
    # machine without a GPU a call that passes every host check fails at the
    # launch with PA_ERR_HIP, never with PA_ERR_INVALID.
    a = 1 << 20
    for n_seq in list(range(1, 70)) + [127, 128, 129, 500, 512, 1000]:
        for T in (1, 4, 5, 8):
            n = pb.workspace_size(n_seq, T, 0)
            ok = pb.make_ext(8, 64, 0.0, None, 1 << 30, n)
            st = pb.decode_status(a, a, a, a, a, n_seq, T, pb.kv_type("q8_0"), 16, a, 0, ok)
            assert st != pb.ERR_INVALID, (n_seq, T, n)
            small = pb.make_ext(8, 64, 0.0, None, 1 << 30, n - 6 * T * 257 * 4)
            st = pb.decode_status(a, a, a, a, a, n_seq, T, pb.kv_type("q8_0"), 16, a, 0, small)
            assert st == pb.ERR_INVALID, (n_seq, T, n)
        big = pb.make_ext(8, 64, 0.0, None, 1 << 30, pb.workspace_size(n_seq, 8, 0))
        for T in range(1, 9):
            st = pb.decode_status(a, a, a, a, a, n_seq, T, pb.kv_type("q4_0"), 16, a, 0, big)
            assert st != pb.ERR_INVALID, (n_seq, T)


def test_read_bandwidth_probe_host_checks():
    # argument errors come back before any HIP call (addresses are never touched)
    lib = pb.lib()
    a = 1 << 20                                          # a 16-byte aligned stand-in address
    assert lib.pa_read_bandwidth_probe(None, 1024, a, 1 << 20, None) == pb.ERR_INVALID      # null source
    assert lib.pa_read_bandwidth_probe(a, 1024, None, 1 << 20, None) == pb.ERR_INVALID      # null sink
    assert lib.pa_read_bandwidth_probe(a, 0, a, 1 << 20, None) == pb.ERR_INVALID            # nothing to read
    assert lib.pa_read_bandwidth_probe(a, 1000, a, 1 << 20, None) == pb.ERR_INVALID         # not a multiple of 16
    assert lib.pa_read_bandwidth_probe(a + 4, 1024, a, 1 << 20, None) == pb.ERR_INVALID     # misaligned source
    assert lib.pa_read_bandwidth_probe(a, 1024, a + 2, 1 << 20, None) == pb.ERR_INVALID     # misaligned sink
    assert lib.pa_read_bandwidth_probe(a, 1024, a, 4, None) == pb.ERR_INVALID               # sink too small
    ex = lib.pa_read_bandwidth_probe_ex
    for wgs, u, flags in ((0, 4, 0), (33, 4, 0), (8, 0, 0), (8, 3, 0), (8, 32, 0), (8, 4, 4)):
        assert ex(a, 1024, a, 1 << 20, wgs, u, flags, None) == pb.ERR_INVALID, (wgs, u, flags)
    assert ex(a, 1024, a, 4 * 16 * 256 - 1, 16, 4, 0, None) == pb.ERR_INVALID                  # short of 4 x wgs x 256 CUs
    assert ex(None, 1024, a, 1 << 20, 8, 4, 0, None) == pb.ERR_INVALID
    assert ex(a, 1000, a, 1 << 20, 8, 4, 0, None) == pb.ERR_INVALID


def test_split_workgroups_per_cu_rejects_bad_arguments():
    # argument checks come before any device call
    lib = pb.lib()
    w = ctypes.c_int32(-7)
    q4 = pb.kv_type("q4_0")
    assert lib.pa_split_workgroups_per_cu(q4, 1, 0, None) == pb.ERR_INVALID
    for kv, t, flags in ((q4, 0, 0), (q4, pb.MAX_QTOK + 1, 0), (0, 1, 0), (9, 1, 0), (q4 | (9 << 8), 1, 0),
                         (q4, 1, 2)):
        assert lib.pa_split_workgroups_per_cu(kv, t, flags, ctypes.byref(w)) == pb.ERR_INVALID
    assert w.value == -7


def test_decode_scratch_rejects_bad_arguments():
    # checks before any device call: ext is required and carries no workspace
    a = 1 << 20
    ext = pb.make_ext(8, 64, 0.0)
    assert pb.decode_scratch_status(a, a, a, a, a, 2, 1, pb.kv_type("q4_0"), 16, a, 0, None) == pb.ERR_INVALID
    with_ws = pb.make_ext(8, 64, 0.0, None, 1 << 30, 1 << 20)
    assert pb.decode_scratch_status(a, a, a, a, a, 2, 1, pb.kv_type("q4_0"), 16, a, 0, with_ws) == pb.ERR_INVALID
    for T in (0, pb.MAX_QTOK + 1):
        assert pb.decode_scratch_status(a, a, a, a, a, 2, T, pb.kv_type("q4_0"), 16, a, 0, ext) == pb.ERR_INVALID
    assert pb.decode_scratch_status(a, a, a, a, a, -1, 1, pb.kv_type("q4_0"), 16, a, 0, ext) == pb.ERR_INVALID


def test_header_constants_match_binding():
    # the binding's copies of pa.h's flag and size macros
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    defs = {m[0]: int(m[1]) << int(m[2] or 0)
            for m in re.findall(r"#define (PA_\w+) +\(?([0-9]+)u?(?: *<< *([0-9]+)\))?", text)}
    assert defs["PA_DECODE_VECTOR_REFERENCE"] == pb.DECODE_VECTOR_REFERENCE
    assert defs["PA_SCRATCH_BYTES"] == pb.SCRATCH_BYTES
    assert defs["PA_MAX_QTOK"] == pb.MAX_QTOK


def test_scratch_batch_limits_documented():
    # pa.h states the largest batches pa_decode_scratch takes on 256 compute
    # units; they follow from pa_decode_workspace_size (256 CUs is also the
    # size the library assumes without a device)
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    m = re.search(r"up to (\d+)\s+\*\s+sequences of one token, (\d+) of four, (\d+) of eight", text)
    assert m, "scratch limits sentence not found in pa.h"
    for n, T in zip(map(int, m.groups()), (1, 4, 8)):
        assert pb.workspace_size(n, T, 0) <= pb.SCRATCH_BYTES < pb.workspace_size(n + 1, T, 0), (n, T)
