"""Argument checks of the C ABI that return before any GPU work: they run on
a host without a GPU.  Null device pointers are never dereferenced because
every call here is rejected first."""
import ctypes

import pytest

from paged_kv_cache_363_amd import _lib

L = None
NULL = None


def lib():
    return _lib.lib()


def decode(**kw):
    a = dict(out=NULL, q=NULL, k=NULL, v=NULL, bt=NULL, cl=NULL, S=4, hq=8, hkv=2, d=128, bs=16,
             nb=10, mb=4, scale=0.1, qd=_lib.PKV_BF16, kvd=_lib.PKV_BF16, ks=1.0, vs=1.0, ps=0,
             ws=NULL, wsb=0, algo=0, stream=NULL)
    a.update(kw)
    return lib().pkv_paged_decode_attention_algo(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["S"], a["hq"], a["hkv"], a["d"],
        a["bs"], a["nb"], a["mb"], a["scale"], a["qd"], a["kvd"], a["ks"], a["vs"], a["ps"],
        a["ws"], a["wsb"], a["algo"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bs=32), _lib.PKV_ERR_UNSUPPORTED),
    (dict(d=96), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=6, hkv=4), _lib.PKV_ERR_INVALID_ARG),
    (dict(qd=_lib.PKV_F32, kvd=_lib.PKV_BF16), _lib.PKV_ERR_UNSUPPORTED),
    (dict(qd=_lib.PKV_BF16, kvd=_lib.PKV_F16), _lib.PKV_ERR_UNSUPPORTED),
    (dict(qd=_lib.PKV_FP8_E4M3, kvd=_lib.PKV_FP8_E4M3), _lib.PKV_ERR_UNSUPPORTED),
    (dict(qd=7), _lib.PKV_ERR_INVALID_ARG),
    (dict(ps=24), _lib.PKV_ERR_INVALID_ARG),
    (dict(algo=5), _lib.PKV_ERR_INVALID_ARG),
    (dict(qd=_lib.PKV_F32, kvd=_lib.PKV_F32, algo=_lib.PKV_ALGO_MFMA), _lib.PKV_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), _lib.PKV_ERR_INVALID_ARG),
    (dict(), _lib.PKV_ERR_INVALID_ARG),                       # NULL pointers
])
def test_decode_rejects(kw, status):
    assert decode(**kw) == status
    assert lib().pkv_last_error() != b""


def test_decode_workspace_error_before_launch():
    # 16-byte aligned fake pointers are never touched: the workspace check fails first
    fake = ctypes.c_void_p(1 << 20)
    st = decode(out=fake, q=fake, k=fake, v=fake, bt=fake, cl=fake, mb=256, ps=512, ws=NULL, wsb=0)
    assert st == _lib.PKV_ERR_WORKSPACE


def test_zero_sequences_is_a_no_op():
    assert decode(S=0) == _lib.PKV_OK


def test_workspace_and_partition_helpers():
    l = lib()
    assert l.pkv_decode_workspace_size(4, 4, 2, 64, 3, 0, 0) == 0      # single pass
    # 16-bit cache, partition 0: the balanced schedule (reported as 0)
    assert l.pkv_decode_partition_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0) == 0
    # f32 cache: fixed partitions of the library's choice
    ps = l.pkv_decode_partition_size(64, 32, 8, 128, 256, _lib.PKV_F32, 0)
    assert ps % 16 == 0 and ps >= 128
    assert l.pkv_decode_partition_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 256) == 256
    # more sequences than the balanced schedule takes: fixed partitions
    assert l.pkv_decode_partition_size(5000, 32, 8, 128, 256, _lib.PKV_BF16, 0) > 0
    assert l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0) > 0
    n = l.pkv_decode_workspace_size(16, 32, 8, 128, 2048, 2, 512)
    rows = 16 * 32 * 64
    assert n >= rows * (128 + 2) * 4
    assert l.pkv_decode_partition_size(1, 1, 1, 128, 4, 2, 24) == -1
    assert l.pkv_decode_algo_for(64, 8, 128, _lib.PKV_BF16, _lib.PKV_FP8_E4M3) == _lib.PKV_ALGO_MFMA
    # MHA (g = 1): the vector kernel; one WG per (sequence, kv-head) fills the GPU -> single pass
    assert l.pkv_decode_algo_for(32, 32, 128, _lib.PKV_F16, _lib.PKV_F16) == _lib.PKV_ALGO_VECTOR
    assert l.pkv_decode_algo_for(32, 16, 128, _lib.PKV_F16, _lib.PKV_F16) == _lib.PKV_ALGO_MFMA
    assert l.pkv_decode_partition_size(256, 32, 32, 128, 128, _lib.PKV_F16, 0) == 2048
    assert l.pkv_decode_workspace_size(256, 32, 32, 128, 128, _lib.PKV_F16, 2048) == 0
    assert l.pkv_decode_algo_for(4, 2, 64, _lib.PKV_F32, _lib.PKV_F32) == _lib.PKV_ALGO_VECTOR
    assert l.pkv_decode_algo_for(4, 2, 96, _lib.PKV_F32, _lib.PKV_F32) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(bs=8), _lib.PKV_ERR_UNSUPPORTED),
    (dict(d=12), _lib.PKV_ERR_UNSUPPORTED),
    (dict(nd=_lib.PKV_FP8_E4M3), _lib.PKV_ERR_UNSUPPORTED),
    (dict(nd=_lib.PKV_BF16, kvd=_lib.PKV_F16), _lib.PKV_ERR_UNSUPPORTED),
    (dict(kvd=_lib.PKV_FP8_E4M3, ks=0.0), _lib.PKV_ERR_INVALID_ARG),
    (dict(kvd=_lib.PKV_FP8_E4M3, vs=float("nan")), _lib.PKV_ERR_INVALID_ARG),
    (dict(T=-1), _lib.PKV_ERR_INVALID_ARG),
    (dict(), _lib.PKV_ERR_INVALID_ARG),                       # NULL pointers
])
def test_append_rejects(kw, status):
    a = dict(T=3, h=2, d=64, bs=16, nb=4, nd=_lib.PKV_BF16, kvd=_lib.PKV_BF16, ks=1.0, vs=1.0)
    a.update(kw)
    st = lib().pkv_paged_cache_append(NULL, NULL, NULL, NULL, NULL, a["T"], a["h"], a["d"],
                                      a["bs"], a["nb"], a["nd"], a["kvd"], a["ks"], a["vs"], NULL)
    assert st == status


def test_stream_workgroups_setting_changes_workspace():
    l = lib()
    base = l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0)
    assert l.pkv_set_stream_workgroups(1024) == _lib.PKV_OK
    try:
        assert l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0) > base
    finally:
        assert l.pkv_set_stream_workgroups(0) == _lib.PKV_OK
    assert l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0) == base
    assert l.pkv_set_stream_workgroups(-1) == _lib.PKV_ERR_INVALID_ARG


def test_copy_blocks_rejects():
    assert lib().pkv_copy_blocks(NULL, NULL, NULL, 1, 4, 24, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert lib().pkv_copy_blocks(NULL, NULL, NULL, 0, 4, 32, NULL) == _lib.PKV_OK


def multiquery(**kw):
    a = dict(out=NULL, q=NULL, k=NULL, v=NULL, bt=NULL, cl=NULL, qs=NULL, S=4, rows=16, maxq=4,
             hq=8, hkv=2, d=128, bs=16, nb=10, mb=4, scale=0.1, qd=_lib.PKV_BF16,
             kvd=_lib.PKV_BF16, ks=1.0, vs=1.0, ps=0, ws=NULL, wsb=0, stream=NULL)
    a.update(kw)
    return lib().pkv_paged_multiquery_attention(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qs"], a["S"], a["rows"], a["maxq"],
        a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["scale"], a["qd"], a["kvd"],
        a["ks"], a["vs"], a["ps"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bs=32), _lib.PKV_ERR_UNSUPPORTED),
    (dict(d=96), _lib.PKV_ERR_UNSUPPORTED),
    (dict(hq=6, hkv=4), _lib.PKV_ERR_INVALID_ARG),
    (dict(qd=_lib.PKV_F32, kvd=_lib.PKV_F32), _lib.PKV_ERR_UNSUPPORTED),   # MFMA only
    (dict(qd=_lib.PKV_BF16, kvd=_lib.PKV_F16), _lib.PKV_ERR_UNSUPPORTED),
    (dict(qd=9), _lib.PKV_ERR_INVALID_ARG),
    (dict(ps=24), _lib.PKV_ERR_INVALID_ARG),
    (dict(rows=-1), _lib.PKV_ERR_INVALID_ARG),
    (dict(maxq=-1), _lib.PKV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.PKV_ERR_INVALID_ARG),
    (dict(kvd=_lib.PKV_FP8_E4M3, ks=float("inf")), _lib.PKV_ERR_INVALID_ARG),
    (dict(hq=8, hkv=8, maxq=70000 * 16), _lib.PKV_ERR_UNSUPPORTED),      # row tiles beyond the grid
    (dict(S=70000), _lib.PKV_ERR_UNSUPPORTED),
    (dict(), _lib.PKV_ERR_INVALID_ARG),                                # NULL pointers
])
def test_multiquery_rejects(kw, status):
    assert multiquery(**kw) == status
    assert lib().pkv_last_error() != b""


def test_multiquery_empty_calls_and_workspace_check():
    assert multiquery(S=0) == _lib.PKV_OK
    assert multiquery(rows=0) == _lib.PKV_OK
    assert multiquery(maxq=0) == _lib.PKV_OK
    fake = ctypes.c_void_p(1 << 20)
    # 4 sequences x 2 kv-heads x 1 row tile: too few workgroups for one pass
    st = multiquery(out=fake, q=fake, k=fake, v=fake, bt=fake, cl=fake, qs=fake, mb=256, ps=512)
    assert st == _lib.PKV_ERR_WORKSPACE


def test_multiquery_partition_and_workspace_helpers():
    l = lib()
    # partition_size 0: the balanced schedule when one workgroup per
    # (sequence, kv-head, row tile) would not fill the chip: 64 x 8 x 1
    assert l.pkv_multiquery_partition_size(64, 4, 32, 8, 256, 0) == 0
    assert l.pkv_multiquery_partition_size(32, 8, 64, 8, 160, 0) == 0       # 32 x 8 x 4
    # 16 x 8 x 128 row tiles (512 rows, 4 per tile) fill it: one pass over the
    # context on the fixed grid
    assert l.pkv_multiquery_partition_size(16, 512, 32, 8, 2048, 0) == 2048 * 16
    # too many sequences for the balanced schedule's prefix sums: fixed
    assert l.pkv_multiquery_partition_size(4096, 1, 32, 8, 16, 0) > 0
    assert l.pkv_multiquery_partition_size(3000, 1, 4, 4, 16, 0) > 0
    assert l.pkv_multiquery_partition_size(16, 512, 32, 8, 2048, 64) == 64
    assert l.pkv_multiquery_partition_size(16, 512, 32, 8, 2048, 24) == -1
    # balanced: (m, l) and accumulator slots, two per wave of the grid, of
    # the 16 tile columns; the same for any row count
    W = 256 * 4
    want = 2 * W * 16 * 2 * 4 + 2 * W * 16 * 128 * 4
    assert l.pkv_multiquery_workspace_size(256, 64, 4, 32, 8, 128, 256, 0) == want
    assert l.pkv_multiquery_workspace_size(64, 64, 4, 32, 8, 128, 256, 0) == want
    # one fixed pass: no workspace
    assert l.pkv_multiquery_workspace_size(8192, 16, 512, 32, 8, 128, 2048, 0) == 0
    # fixed partitions of 512 over 4096 tokens: partials per row, head, partition
    n = l.pkv_multiquery_workspace_size(256, 64, 4, 32, 8, 128, 256, 512)
    assert n >= 256 * 32 * 8 * (128 + 2) * 4
    assert l.pkv_multiquery_workspace_size(-1, 64, 4, 32, 8, 128, 256, 512) == ctypes.c_size_t(-1).value


def test_int8_cache_is_a_scaled_byte_cache():
    l = lib()
    assert l.pkv_decode_algo_for(64, 8, 128, _lib.PKV_BF16, _lib.PKV_INT8) == _lib.PKV_ALGO_MFMA
    assert l.pkv_decode_algo_for(32, 32, 128, _lib.PKV_F16, _lib.PKV_INT8) == _lib.PKV_ALGO_VECTOR
    assert l.pkv_decode_partition_size(32, 64, 8, 128, 160, _lib.PKV_INT8, 0) == 0   # balanced
    assert l.pkv_kv_bytes_per_token(80, 8, 128, _lib.PKV_INT8) == 2 * 80 * 8 * 128
    # f32 q with an INT8 cache is not implemented; INT8 rows cannot be appended
    assert decode(qd=_lib.PKV_F32, kvd=_lib.PKV_INT8) == _lib.PKV_ERR_UNSUPPORTED
    st = lib().pkv_paged_cache_append(NULL, NULL, NULL, NULL, NULL, 3, 2, 64, 16, 4,
                                      _lib.PKV_INT8, _lib.PKV_INT8, 1.0, 1.0, NULL)
    assert st == _lib.PKV_ERR_UNSUPPORTED
    st = lib().pkv_paged_cache_append(NULL, NULL, NULL, NULL, NULL, 3, 2, 64, 16, 4,
                                      _lib.PKV_BF16, _lib.PKV_INT8, 0.0, 1.0, NULL)
    assert st == _lib.PKV_ERR_INVALID_ARG                  # INT8 needs scales > 0


def test_stream_read_probe_rejects_bad_arguments():
    l = lib()
    fake = ctypes.c_void_p(1 << 20)
    assert l.pkv_stream_read_probe(fake, 4096, fake, 1, fake, 0, NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert l.pkv_stream_read_probe(fake, 4096, fake, 1, fake, 65536, NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert l.pkv_stream_read_probe(fake, -1, fake, 1, fake, 4, NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert l.pkv_stream_read_probe(fake, 4096, fake, -1, fake, 4, NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert l.pkv_stream_read_probe(NULL, 4096, fake, 1, fake, 4, NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert l.pkv_stream_read_probe(ctypes.c_void_p((1 << 20) + 4), 4096, fake, 1, fake, 4,
                                   NULL, NULL, NULL) == _lib.PKV_ERR_INVALID_ARG
    assert b"stream_read_probe" in l.pkv_last_error()



def test_copy_blocks_rejects_pageable_host_memory():
    """Buffers no kernel can reach (pageable host memory) are refused before
    any launch, for the caches and for the pairs alike."""
    import numpy as np
    host = np.zeros(4096, np.uint8)
    pairs = np.array([0, 1], np.int32)
    hp, pp = host.ctypes.data, pairs.ctypes.data
    st = lib().pkv_copy_blocks(hp, hp, pp, 1, 2, 1024, NULL)
    assert st == _lib.PKV_ERR_INVALID_ARG
    assert b"device or pinned host memory" in lib().pkv_last_error()


def test_stream_workgroups_override_is_per_thread():
    """The grid override of one thread leaves other threads' workspace sizes
    (and grids) alone."""
    import threading
    l = lib()
    base = l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0)
    seen = {}

    def other():
        seen["size"] = l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0)

    assert l.pkv_set_stream_workgroups(1024) == _lib.PKV_OK
    try:
        th = threading.Thread(target=other)
        th.start()
        th.join()
        assert l.pkv_decode_workspace_size(64, 32, 8, 128, 256, _lib.PKV_BF16, 0) > base
    finally:
        assert l.pkv_set_stream_workgroups(0) == _lib.PKV_OK
    assert seen["size"] == base


def appending(**kw):
    fake = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced
    a = dict(out=fake, q=fake, kn=fake, vn=fake, slots=fake, k=fake, v=fake, bt=fake, cl=fake, S=4,
             hq=8, hkv=2, d=128, bs=16, nb=10, mb=4, scale=0.1, qd=_lib.PKV_BF16,
             kvd=_lib.PKV_FP8_E4M3, ks=0.5, vs=0.5, ps=0, ws=NULL, wsb=0, algo=0)
    a.update(kw)
    return lib().pkv_paged_decode_attention_appending(
        a["out"], a["q"], a["kn"], a["vn"], a["slots"], a["k"], a["v"], a["bt"], a["cl"], a["S"],
        a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["mb"], a["scale"], a["qd"], a["kvd"],
        a["ks"], a["vs"], a["ps"], a["ws"], a["wsb"], a["algo"], NULL, NULL, NULL, NULL)


@pytest.mark.parametrize("kw", [
    dict(kn=NULL), dict(vn=NULL), dict(slots=NULL),                     # the new rows
    dict(kn=ctypes.c_void_p((1 << 20) + 8)),                            # misaligned new rows
    dict(ks=0.0), dict(vs=float("nan")), dict(ks=float("inf")),         # one-byte scales
    dict(bs=32), dict(d=96), dict(hq=6, hkv=4), dict(out=NULL),         # the decode's own checks
    dict(mb=256, ps=512),                                               # workspace missing
])
def test_appending_decode_rejects_before_any_launch(kw):
    """pkv_paged_decode_attention_appending reports the append's and the
    decode's argument errors before it launches anything (the pointers here
    are never dereferenced)."""
    st = appending(**kw)
    assert st != _lib.PKV_OK
    assert lib().pkv_last_error() != b""


def test_appending_decode_scales_matter_only_for_one_byte_caches():
    # a bf16 cache ignores the scales: the call goes on to the decode's checks
    # (here a block size the kernels do not take), not to the scale check
    st = appending(kvd=_lib.PKV_BF16, ks=0.0, vs=0.0, bs=32)
    assert st == _lib.PKV_ERR_UNSUPPORTED


def test_appending_decode_of_zero_sequences_is_a_no_op():
    assert appending(S=0, kn=NULL, vn=NULL, slots=NULL) == _lib.PKV_OK
