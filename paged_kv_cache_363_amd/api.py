"""torch-facing binding of the C ABI: argument marshalling only.

Tensors supply device memory and the current HIP stream; every step of the
decode path runs in the library's kernels.  FP8 caches are uint8 (or
torch.float8_e4m3fn) tensors holding OCP E4M3FN codes; INT8 caches are int8
tensors of symmetric codes.
"""
import ctypes

import torch

from . import _lib
from ._lib import check, lib

_DT = {torch.float32: _lib.PKV_F32, torch.float16: _lib.PKV_F16,
       torch.bfloat16: _lib.PKV_BF16, torch.uint8: _lib.PKV_FP8_E4M3,
       torch.float8_e4m3fn: _lib.PKV_FP8_E4M3, torch.int8: _lib.PKV_INT8}
_ALGO = {"auto": _lib.PKV_ALGO_AUTO, "vector": _lib.PKV_ALGO_VECTOR, "mfma": _lib.PKV_ALGO_MFMA}
BLOCK_SIZE = 16


def dtype_code(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def kv_bytes_per_token(layers, kv_heads, head_dim, dtype):
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(lib().pkv_kv_bytes_per_token(layers, kv_heads, head_dim, code))


def paged_cache_append(k_cache, v_cache, k_new, v_new, slot_mapping, k_scale=1.0, v_scale=1.0,
                       stream=None):
    """Write k_new/v_new [T][H_kv][d] into the caches [NB][H_kv][16][d] at
    slot_mapping[T] (int64 device tensor; negative = skip)."""
    nb, hkv, bs, d = k_cache.shape
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError(f"k_new/v_new must be [{T}, {hkv}, {d}]")
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    check(lib().pkv_paged_cache_append(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"), T, hkv, d, bs, nb,
        dtype_code(k_new), dtype_code(k_cache), float(k_scale), float(v_scale),
        _stream(k_cache, stream)))


def paged_cache_append_per_channel(k_cache, v_cache, k_new, v_new, slot_mapping, k_scales,
                                   v_scales, stream=None):
    """Append into an FP8/INT8 cache with per-channel scales: k_scales,
    v_scales are float32 device tensors [H_kv][d]."""
    nb, hkv, bs, d = k_cache.shape
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError(f"k_new/v_new must be [{T}, {hkv}, {d}]")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if t.dtype != torch.float32 or tuple(t.shape) != (hkv, d):
            raise ValueError(f"{name} must be float32 [{hkv}, {d}]")
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    check(lib().pkv_paged_cache_append_per_channel(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping"), T, hkv, d, bs, nb,
        dtype_code(k_new), dtype_code(k_cache), _dev(k_scales, "k_scales"),
        _dev(v_scales, "v_scales"), _stream(k_cache, stream)))


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          kv_dtype=_lib.PKV_BF16, partition_size=0, context_lens=None):
    """partition_size for a decode call (pkv_decode_partition_size).  With the
    batch's context lengths on the host (context_lens: int sequence or numpy
    array) and partition_size 0, the choice weighs them
    (pkv_decode_partition_size_for_lengths)."""
    if context_lens is not None and partition_size == 0:
        import numpy as np
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        if cl.shape != (num_seqs,):
            raise ValueError("context_lens must hold num_seqs lengths")
        return int(lib().pkv_decode_partition_size_for_lengths(
            cl.ctypes.data, num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
            kv_dtype))
    return int(lib().pkv_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               max_blocks_per_seq, kv_dtype, partition_size))


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          kv_dtype=_lib.PKV_BF16, partition_size=0):
    n = lib().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_blocks_per_seq, kv_dtype, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise _lib.InvalidArg(_lib.PKV_ERR_INVALID_ARG, "bad decode workspace arguments")
    return int(n)


def decode_algo_for(num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype):
    a = int(lib().pkv_decode_algo_for(num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype))
    return {1: "vector", 2: "mfma"}.get(a)


def alloc_workspace(q, k_cache, block_tables, partition_size=0):
    S, hq, d = q.shape
    n = decode_workspace_size(S, hq, k_cache.shape[1], d, block_tables.shape[1],
                              dtype_code(k_cache), partition_size)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=1.0,
                           v_scale=1.0, partition_size=0, out=None, workspace=None, algo="auto",
                           stream=None, events=None):
    """out[S][H_q][d] (q dtype) = softmax(scale * q K^T) V over each sequence's
    context_lens[s] tokens, K/V gathered through block_tables [S][MB] (int32).
    events: optional (begin, mid, end) torch.cuda.Event triple recorded around
    the partition kernel and the reduction kernel."""
    S, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    mb = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(q, k_cache, block_tables, partition_size)
    evs = [None, None, None]
    if events is not None:
        evs = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
    check(lib().pkv_paged_decode_attention_profiled(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, hq, hkv, d,
        bs, nb, mb, float(scale), dtype_code(q), dtype_code(k_cache), float(k_scale),
        float(v_scale), int(partition_size), _dev(workspace, "workspace"), workspace.numel(),
        _ALGO[algo], _stream(q, stream), *evs))
    return out


def paged_decode_attention_appending(q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                     block_tables, context_lens, scale, k_scale=1.0, v_scale=1.0,
                                     partition_size=0, out=None, workspace=None, algo="auto",
                                     stream=None, events=None):
    """The decode step's append and attention in one call: the same result
    as paged_cache_append(k_cache, v_cache, k_new, v_new, slot_mapping, ...)
    followed by paged_decode_attention(...).  k_new, v_new [S][H_kv][d] in
    the q dtype; slot_mapping [S] int64, negative (no row) or the slot of the
    context's last token (pkv_paged_decode_attention_appending)."""
    S, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d):
        raise ValueError(f"k_new/v_new must be [{S}, {hkv}, {d}]")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("k_new and v_new must be in the q dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape[0] != S:
        raise TypeError("slot_mapping must be int64 [S]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    mb = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(q, k_cache, block_tables, partition_size)
    evs = [None, None, None]
    if events is not None:
        evs = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
    check(lib().pkv_paged_decode_attention_appending(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(slot_mapping, "slot_mapping"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, hq, hkv, d,
        bs, nb, mb, float(scale), dtype_code(q), dtype_code(k_cache), float(k_scale),
        float(v_scale), int(partition_size), _dev(workspace, "workspace"), workspace.numel(),
        _ALGO[algo], _stream(q, stream), *evs))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale,
                                   k_scale=1.0, v_scale=1.0, partition_size=0, out=None,
                                   algo="auto", stream=None):
    """paged_decode_attention without a workspace: the library keeps split
    contexts' partials in its static per-GPU scratch array
    (pkv_paged_decode_attention_noalloc).  `out` must be given by a caller
    that cannot allocate; calls overlapping in time on one GPU race."""
    S, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have one row per sequence")
    if out is None:
        out = torch.empty_like(q)
    check(lib().pkv_paged_decode_attention_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, hq, hkv, d,
        bs, nb, block_tables.shape[1], float(scale), dtype_code(q), dtype_code(k_cache),
        float(k_scale), float(v_scale), int(partition_size), _ALGO[algo], _stream(q, stream)))
    return out


def multiquery_partition_size(num_seqs, max_query_len, num_q_heads, num_kv_heads,
                              max_blocks_per_seq, partition_size=0, context_lens=None,
                              kv_dtype=_lib.PKV_BF16):
    """partition_size for a multi-query call (pkv_multiquery_partition_size).
    With the batch's context lengths on the host (context_lens) and
    partition_size 0, the choice weighs them
    (pkv_multiquery_partition_size_for_lengths)."""
    if context_lens is not None and partition_size == 0:
        import numpy as np
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        if cl.shape != (num_seqs,):
            raise ValueError("context_lens must hold num_seqs lengths")
        return int(lib().pkv_multiquery_partition_size_for_lengths(
            cl.ctypes.data, num_seqs, max_query_len, num_q_heads, num_kv_heads,
            max_blocks_per_seq, kv_dtype))
    return int(lib().pkv_multiquery_partition_size(num_seqs, max_query_len, num_q_heads,
                                                   num_kv_heads, max_blocks_per_seq,
                                                   partition_size))


def multiquery_workspace_size(num_rows, num_seqs, max_query_len, num_q_heads, num_kv_heads,
                              head_dim, max_blocks_per_seq, partition_size=0):
    n = lib().pkv_multiquery_workspace_size(num_rows, num_seqs, max_query_len, num_q_heads,
                                            num_kv_heads, head_dim, max_blocks_per_seq,
                                            partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise _lib.InvalidArg(_lib.PKV_ERR_INVALID_ARG, "bad multi-query workspace arguments")
    return int(n)


def paged_multiquery_attention(q, k_cache, v_cache, block_tables, context_lens, query_start,
                               max_query_len, scale, k_scale=1.0, v_scale=1.0, partition_size=0,
                               out=None, workspace=None, stream=None, events=None):
    """out[rows][H_q][d] (q dtype): rows query_start[s] .. query_start[s+1]-1
    of q (int32 device tensor [S+1]) are the last positions of sequence s and
    attend causally through block_tables [S][MB]; row i of n sits at position
    context_lens[s] - n + i.  max_query_len bounds the rows per sequence.
    events: optional (begin, mid, end) torch.cuda.Event triple recorded around
    the attention kernel and the partition reduction."""
    rows, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    S = context_lens.shape[0]
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                    (query_start, "query_start")):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("block_tables [S][MB], context_lens [S], query_start [S+1]")
    mb = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        n = multiquery_workspace_size(rows, S, max_query_len, hq, hkv, d, mb, partition_size)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    evs = [None, None, None]
    if events is not None:
        evs = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
    check(lib().pkv_paged_multiquery_attention_profiled(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
        _dev(query_start, "query_start"), S, rows, int(max_query_len), hq, hkv, d, bs, nb, mb,
        float(scale), dtype_code(q), dtype_code(k_cache), float(k_scale), float(v_scale),
        int(partition_size), _dev(workspace, "workspace"), workspace.numel(), _stream(q, stream),
        *evs))
    return out


def swap_blocks(dst_k, dst_v, src_k, src_v, src_dst_pairs, stream=None):
    """Copy block pairs[i][0] of (src_k, src_v) into block pairs[i][1] of
    (dst_k, dst_v); either side may be a pinned host tensor (swap out / in).
    src_dst_pairs: int32 tensor [n][2] on the device or in pinned memory."""
    if tuple(dst_k.shape[1:]) != tuple(src_k.shape[1:]) or dst_k.dtype != src_k.dtype:
        raise ValueError("the two caches must have the same block layout and dtype")
    for t, name in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"), (src_v, "src_v"),
                    (src_dst_pairs, "src_dst_pairs")):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a device tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if src_dst_pairs.dtype != torch.int32:
        raise TypeError("src_dst_pairs must be int32")
    dev = dst_k if dst_k.is_cuda else src_k
    block_bytes = dst_k[0].numel() * dst_k.element_size()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    check(lib().pkv_swap_blocks(ptr(dst_k), ptr(dst_v), dst_k.shape[0], ptr(src_k), ptr(src_v),
                                src_k.shape[0], ptr(src_dst_pairs), src_dst_pairs.shape[0],
                                block_bytes, _stream(dev, stream)))


def paged_decode_attention_per_channel(q, k_cache, v_cache, block_tables, context_lens, scale,
                                       k_scales, v_scales, partition_size=0, out=None,
                                       workspace=None, algo="auto", stream=None, events=None):
    """Decode over an FP8/INT8 cache with per-channel scales [H_kv][d]
    (float32 device tensors); otherwise as paged_decode_attention."""
    S, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    for t, name in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if t.dtype != torch.float32 or tuple(t.shape) != (hkv, d):
            raise ValueError(f"{name} must be float32 [{hkv}, {d}]")
    mb = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(q, k_cache, block_tables, partition_size)
    evs = [None, None, None]
    if events is not None:
        evs = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
    check(lib().pkv_paged_decode_attention_per_channel(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, hq, hkv, d,
        bs, nb, mb, float(scale), dtype_code(q), dtype_code(k_cache),
        _dev(k_scales, "k_scales"), _dev(v_scales, "v_scales"), int(partition_size),
        _dev(workspace, "workspace"), workspace.numel(), _ALGO[algo], _stream(q, stream), *evs))
    return out


def copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None):
    """Copy physical block pairs[i][0] into pairs[i][1] in both caches
    (src_dst_pairs: int32 device tensor [n][2])."""
    nb = k_cache.shape[0]
    block_bytes = k_cache[0].numel() * k_cache.element_size()
    if src_dst_pairs.dtype != torch.int32:
        raise TypeError("src_dst_pairs must be int32")
    n = src_dst_pairs.shape[0]
    check(lib().pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(src_dst_pairs, "src_dst_pairs"), n, nb, block_bytes,
                                _stream(k_cache, stream)))


def stream_read_probe(buf, tile_ids, sink, workgroups=256, stream=None, events=None):
    """Read the 4 KiB tiles of `buf` (a contiguous device tensor) listed in
    tile_ids (int32 device tensor) with the streaming-read probe: the
    achievable HBM read rate of paged decode's access pattern, for measuring
    the decode kernels against.  sink: uint32-sized device tensor of
    workgroups * 256 elements, overwritten.  events: optional (start, stop)
    torch.cuda.Event pair stamped by the probe kernel's dispatch."""
    if tile_ids.dtype != torch.int32:
        raise TypeError("tile_ids must be int32")
    if sink.numel() * sink.element_size() < workgroups * 256 * 4:
        raise ValueError("sink holds fewer than workgroups * 256 uint32")
    evs = [None, None]
    if events is not None:
        evs = [ctypes.c_void_p(e.cuda_event) if e is not None else None for e in events]
    check(lib().pkv_stream_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                      _dev(tile_ids, "tile_ids"), tile_ids.numel(),
                                      _dev(sink, "sink"), int(workgroups), _stream(buf, stream),
                                      *evs))
