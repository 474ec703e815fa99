"""ctypes front end of the fp64 CPU oracle in pkv_oracle.c.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py, never by the product package.  It shares no
code with the HIP path.

Arrays are numpy arrays holding raw element bits:
  'f32' -> float32, 'f16' / 'bf16' -> uint16, 'fp8' -> uint8 (OCP E4M3FN),
  'int8' -> int8 (symmetric codes, value = code * scale).
Cache arrays use the layout [num_blocks][num_kv_heads][block_size][head_dim].
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3, "int8": 4}
BITS_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
           "int8": np.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}

_lib = None


def build_oracle():
    """Compile pkv_oracle.c with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build_oracle()
    lib = ctypes.CDLL(_SO)
    P, I, D, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float
    I64 = ctypes.c_int64
    lib.orc_paged_decode.argtypes = [P, P, I, P, P, I, P, P, I, I, I, I, I, I, D, D, D]
    lib.orc_paged_decode.restype = I
    lib.orc_paged_decode_mt.argtypes = [P, P, I, P, P, I, P, P, I, I, I, I, I, I, D, D, D, I]
    lib.orc_paged_decode_mt.restype = I
    lib.orc_paged_multiquery.argtypes = [P, P, I, P, P, I, P, P, P, I, I, I, I, I, I, I, D, D, D]
    lib.orc_paged_multiquery.restype = I
    lib.orc_paged_multiquery_mt.argtypes = [P, P, I, P, P, I, P, P, P, I, I, I, I, I, I, I, D, D,
                                            D, I]
    lib.orc_paged_multiquery_mt.restype = I
    lib.orc_cache_append_channel.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, P]
    lib.orc_cache_append_channel.restype = I
    lib.orc_paged_decode_channel.argtypes = [P, P, I, P, P, I, P, P, I, I, I, I, I, I, D, P, P]
    lib.orc_paged_decode_channel.restype = I
    lib.orc_softmax_weights.argtypes = [P, I, I, P, I, P, I, P, P, I, I, I, I, I, I, D, D]
    lib.orc_softmax_weights.restype = I
    lib.orc_partition_stats.argtypes = [P, P, P, I, I, I, I, P, I, P, P, I, P, P,
                                        I, I, I, I, I, I, D, D, D]
    lib.orc_partition_stats.restype = I
    lib.orc_lse_merge.argtypes = [P, P, P, P, I, I]
    lib.orc_lse_merge.restype = None
    lib.orc_cache_append.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, F]
    lib.orc_cache_append.restype = I
    lib.orc_e4m3_encode_array.argtypes = [P, I64, P]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_int8_encode_array.argtypes = [P, I64, P]
    lib.orc_int8_encode_array.restype = None
    lib.orc_bits_to_f64.argtypes = [P, I, I64, P]
    lib.orc_bits_to_f64.restype = None
    lib.orc_kv_bytes_per_token.argtypes = [I, I, I, I]
    lib.orc_kv_bytes_per_token.restype = ctypes.c_uint64
    _lib = lib
    return lib


def default_threads():
    """Threads for the oracle's row-parallel entry points: OMP_NUM_THREADS if
    set, else the host's CPU count, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_bits(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != BITS_NP[dtype]:
        raise TypeError(f"{dtype} data must be given as {BITS_NP[dtype].__name__} bits, got {a.dtype}")
    return a


def to_f64(bits, dtype):
    """Exact widening of raw element bits to float64 (E4M3 via its definition)."""
    bits = _check_bits(bits, dtype)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().orc_bits_to_f64(_ptr(bits), DTYPES[dtype], bits.size, _ptr(out))
    return out


def e4m3_encode(x):
    """Nearest E4M3FN code of each float32 value, ties to even, saturating."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def int8_encode(x):
    """INT8 codes (as int8) of float32 values: nearest integer, ties to even,
    saturated to +-127, NaN -> 0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().orc_int8_encode_array(_ptr(x), x.size, _ptr(out))
    return out.view(np.int8)


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype):
    return int(_load().orc_kv_bytes_per_token(layers, kv_heads, head_dim, ELEM_BYTES[dtype]))


def cache_append(k_cache, v_cache, k_new, v_new, slot_mapping, new_dtype, kv_dtype,
                 k_scale=1.0, v_scale=1.0):
    """In-place append of new K/V rows [T][H_kv][d] at slot_mapping[T]."""
    k_cache = _check_bits(k_cache, kv_dtype)
    v_cache = _check_bits(v_cache, kv_dtype)
    k_new = _check_bits(k_new, new_dtype)
    v_new = _check_bits(v_new, new_dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    nb, hkv, bs, d = k_cache.shape
    T = slots.shape[0]
    assert k_new.shape == (T, hkv, d) and v_new.shape == (T, hkv, d)
    rc = _load().orc_cache_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                  _ptr(slots), T, hkv, d, bs, nb, DTYPES[new_dtype],
                                  DTYPES[kv_dtype], k_scale, v_scale)
    if rc != 0:
        raise ValueError(f"oracle cache_append failed ({rc})")
    return k_cache, v_cache


def _common(q, q_dtype, k_cache, kv_dtype, block_tables, context_lens):
    q = _check_bits(q, q_dtype)
    k_cache = _check_bits(k_cache, kv_dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    assert d == d2 and bt.shape[0] == S and cl.shape[0] == S
    return q, k_cache, bt, cl, S, hq, hkv, d, bs


def paged_decode(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                 scale, k_scale=1.0, v_scale=1.0, threads=None):
    """fp64 out[S][H_q][d] of single-query attention through the block table.
    threads: rows (sequence, q-head) shared among this many threads (None:
    default_threads(); 1: the serial loop).  The result is the same bit for
    bit: each row is computed by one thread with the same loops."""
    q, k_cache, bt, cl, S, hq, hkv, d, bs = _common(q, q_dtype, k_cache, kv_dtype,
                                                    block_tables, context_lens)
    v_cache = _check_bits(v_cache, kv_dtype)
    out = np.empty((S, hq, d), dtype=np.float64)
    nt = default_threads() if threads is None else int(threads)
    if nt <= 1:
        rc = _load().orc_paged_decode(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                      _ptr(v_cache), DTYPES[kv_dtype], _ptr(bt), _ptr(cl),
                                      S, hq, hkv, d, bs, bt.shape[1], scale, k_scale, v_scale)
    else:
        rc = _load().orc_paged_decode_mt(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                         _ptr(v_cache), DTYPES[kv_dtype], _ptr(bt), _ptr(cl),
                                         S, hq, hkv, d, bs, bt.shape[1], scale, k_scale,
                                         v_scale, nt)
    if rc != 0:
        raise ValueError(f"oracle paged_decode failed ({rc})")
    return out


def paged_multiquery(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                     query_start, scale, k_scale=1.0, v_scale=1.0, threads=None):
    """fp64 out[rows][H_q][d]: the rows query_start[s]..query_start[s+1]-1 of
    sequence s are its last positions and attend causally through the block
    table (row i of n sits at position ctx - n + i).  threads as for
    paged_decode."""
    q = _check_bits(q, q_dtype)
    k_cache = _check_bits(k_cache, kv_dtype)
    v_cache = _check_bits(v_cache, kv_dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    rows, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    S = cl.shape[0]
    assert d == d2 and bt.shape[0] == S and qs.shape[0] == S + 1
    out = np.empty((rows, hq, d), dtype=np.float64)
    nt = default_threads() if threads is None else int(threads)
    args = (_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache), _ptr(v_cache), DTYPES[kv_dtype],
            _ptr(bt), _ptr(cl), _ptr(qs), S, rows, hq, hkv, d, bs, bt.shape[1], scale, k_scale,
            v_scale)
    rc = (_load().orc_paged_multiquery(*args) if nt <= 1
          else _load().orc_paged_multiquery_mt(*args, nt))
    if rc != 0:
        raise ValueError(f"oracle paged_multiquery failed ({rc})")
    return out


def cache_append_channel(k_cache, v_cache, k_new, v_new, slot_mapping, new_dtype, kv_dtype,
                         k_scales, v_scales):
    """Append into a one-byte-code cache with one float32 scale per (kv-head,
    dim) channel: k_scales, v_scales [H_kv][d]."""
    k_cache = _check_bits(k_cache, kv_dtype)
    v_cache = _check_bits(v_cache, kv_dtype)
    k_new = _check_bits(k_new, new_dtype)
    v_new = _check_bits(v_new, new_dtype)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    nb, hkv, bs, d = k_cache.shape
    assert ks.shape == (hkv, d) and vs.shape == (hkv, d)
    rc = _load().orc_cache_append_channel(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                          _ptr(sm), sm.shape[0], hkv, d, bs, nb,
                                          DTYPES[new_dtype], DTYPES[kv_dtype], _ptr(ks), _ptr(vs))
    if rc != 0:
        raise ValueError(f"oracle cache_append_channel failed ({rc})")


def paged_decode_channel(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens,
                         scale, k_scales, v_scales):
    """fp64 decode over a cache with per-channel scales [H_kv][d] (as float64)."""
    q, k_cache, bt, cl, S, hq, hkv, d, bs = _common(q, q_dtype, k_cache, kv_dtype,
                                                    block_tables, context_lens)
    v_cache = _check_bits(v_cache, kv_dtype)
    ks = np.ascontiguousarray(k_scales, dtype=np.float64)
    vs = np.ascontiguousarray(v_scales, dtype=np.float64)
    assert ks.shape == (hkv, d) and vs.shape == (hkv, d)
    out = np.empty((S, hq, d), dtype=np.float64)
    rc = _load().orc_paged_decode_channel(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                          _ptr(v_cache), DTYPES[kv_dtype], _ptr(bt), _ptr(cl),
                                          S, hq, hkv, d, bs, bt.shape[1], scale, _ptr(ks),
                                          _ptr(vs))
    if rc != 0:
        raise ValueError(f"oracle paged_decode_channel failed ({rc})")
    return out


def softmax_weights(s, h, q, q_dtype, k_cache, kv_dtype, block_tables, context_lens,
                    scale, k_scale=1.0):
    q, k_cache, bt, cl, S, hq, hkv, d, bs = _common(q, q_dtype, k_cache, kv_dtype,
                                                    block_tables, context_lens)
    w = np.zeros(max(int(cl[s]), 1), dtype=np.float64)
    n = _load().orc_softmax_weights(_ptr(w), s, h, _ptr(q), DTYPES[q_dtype], _ptr(k_cache),
                                    DTYPES[kv_dtype], _ptr(bt), _ptr(cl), S, hq, hkv, d, bs,
                                    bt.shape[1], scale, k_scale)
    return w[:n]


def partition_stats(s, h, t0, t1, q, q_dtype, k_cache, v_cache, kv_dtype, block_tables,
                    context_lens, scale, k_scale=1.0, v_scale=1.0):
    """(m, l, acc[d]) of tokens [t0, t1) for one (sequence, q-head)."""
    q, k_cache, bt, cl, S, hq, hkv, d, bs = _common(q, q_dtype, k_cache, kv_dtype,
                                                    block_tables, context_lens)
    v_cache = _check_bits(v_cache, kv_dtype)
    m = np.zeros(1)
    l = np.zeros(1)
    acc = np.zeros(d)
    rc = _load().orc_partition_stats(_ptr(m), _ptr(l), _ptr(acc), s, h, t0, t1, _ptr(q),
                                     DTYPES[q_dtype], _ptr(k_cache), _ptr(v_cache),
                                     DTYPES[kv_dtype], _ptr(bt), _ptr(cl), S, hq, hkv, d, bs,
                                     bt.shape[1], scale, k_scale, v_scale)
    if rc != 0:
        raise ValueError(f"oracle partition_stats failed ({rc})")
    return float(m[0]), float(l[0]), acc


def lse_merge(m, l, acc):
    """Merge per-partition (m_p, l_p, acc_p[d]) into one output row."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    P, d = acc.shape
    out = np.empty(d)
    _load().orc_lse_merge(_ptr(out), _ptr(m), _ptr(l), _ptr(acc), P, d)
    return out
