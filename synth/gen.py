"""Seeded draws for a Config.  Every function here only draws and rounds.

Streams are independent numpy PCG64 generators keyed by (seed, stream id[,
sequence]), so any sequence's values can be regenerated on their own.
Rounding to bf16 goes through torch's float32 -> bfloat16 cast and to f16
through numpy's float32 -> float16 cast; both round to nearest even.
"""
import math

import numpy as np
import torch

from .configs import Config

_STREAM_CTX, _STREAM_ORDER, _STREAM_Q, _STREAM_K, _STREAM_V = 0, 1, 2, 3, 4
_STREAM_PREFIX_K, _STREAM_PREFIX_V, _STREAM_MISC = 5, 6, 7
_STREAM_STEP_K, _STREAM_STEP_V = 8, 9
_STREAM_QLEN, _STREAM_MQ_Q = 10, 11

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def rng(cfg_or_seed, *keys):
    seed = cfg_or_seed.seed if isinstance(cfg_or_seed, Config) else int(cfg_or_seed)
    return np.random.default_rng([seed, *keys])


def round_to(x_f32, dtype):
    """float32 numpy array -> torch CPU tensor of `dtype` ('f32'|'f16'|'bf16')."""
    x = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    if dtype == "f32":
        return x.clone()
    if dtype == "f16":
        return torch.from_numpy(x.numpy().astype(np.float16))
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    raise ValueError(dtype)


def bits(t):
    """Raw element bits of a CPU tensor as numpy (float32 / uint16 / uint8)."""
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.contiguous().numpy()
    raise TypeError(t.dtype)


def context_lens(cfg):
    """Post-append context lengths (the new token included), int32[S]."""
    S = cfg.num_seqs
    if cfg.ctx_kind == "list":
        c = np.array(cfg.ctx_params, dtype=np.int64)
        assert c.shape[0] == S
    elif cfg.ctx_kind == "fixed":
        c = np.full(S, cfg.ctx_params[0], dtype=np.int64)
    elif cfg.ctx_kind == "uniform":
        lo, hi = cfg.ctx_params
        c = rng(cfg, _STREAM_CTX).integers(lo, hi + 1, size=S)
    elif cfg.ctx_kind == "lognormal":
        mean, sigma, lo, hi = cfg.ctx_params
        mu = math.log(mean) - sigma * sigma / 2.0
        c = np.clip(np.rint(rng(cfg, _STREAM_CTX).lognormal(mu, sigma, size=S)), lo, hi)
    else:
        raise ValueError(cfg.ctx_kind)
    assert c.max() <= cfg.max_blocks_per_seq * cfg.block_size
    return c.astype(np.int32)


def block_demand(cfg, ctx):
    bs = cfg.block_size
    per_seq = [-(-int(n) // bs) for n in ctx]
    shared = cfg.shared_prefix // bs
    return sum(per_seq) - shared * (len(per_seq) - 1) if shared else sum(per_seq)


def num_blocks(cfg, ctx):
    if cfg.num_blocks:
        return cfg.num_blocks
    return int(math.ceil(cfg.pool_factor * block_demand(cfg, ctx)))


def free_order(cfg, nb):
    """Initial order of the pool's free queue: a seeded permutation."""
    return rng(cfg, _STREAM_ORDER).permutation(nb).astype(np.int32)


def queries(cfg):
    x = rng(cfg, _STREAM_Q).standard_normal(
        (cfg.num_seqs, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    return round_to(x, cfg.q_dtype)


def seq_kv(cfg, s, n):
    """K and V rows [n][H_kv][d] of the first n positions of sequence s, in
    cfg.new_dtype.  Positions below cfg.shared_prefix come from one stream
    shared by all sequences; the rest from the sequence's own stream."""
    shape_tail = (cfg.num_kv_heads, cfg.head_dim)
    p = min(cfg.shared_prefix, n)
    parts_k, parts_v = [], []
    if p:
        parts_k.append(rng(cfg, _STREAM_PREFIX_K).standard_normal((p,) + shape_tail, dtype=np.float32))
        parts_v.append(rng(cfg, _STREAM_PREFIX_V).standard_normal((p,) + shape_tail, dtype=np.float32))
    parts_k.append(rng(cfg, _STREAM_K, s).standard_normal((n - p,) + shape_tail, dtype=np.float32))
    parts_v.append(rng(cfg, _STREAM_V, s).standard_normal((n - p,) + shape_tail, dtype=np.float32))
    k = np.concatenate(parts_k) if len(parts_k) > 1 else parts_k[0]
    v = np.concatenate(parts_v) if len(parts_v) > 1 else parts_v[0]
    return round_to(k, cfg.new_dtype), round_to(v, cfg.new_dtype)


def step_kv(cfg):
    """The decode step's new K and V rows, [S][H_kv][d] in cfg.new_dtype; row s
    becomes position ctx[s]-1 of sequence s."""
    shape = (cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim)
    k = rng(cfg, _STREAM_STEP_K).standard_normal(shape, dtype=np.float32)
    v = rng(cfg, _STREAM_STEP_V).standard_normal(shape, dtype=np.float32)
    return round_to(k, cfg.new_dtype), round_to(v, cfg.new_dtype)


E4M3_MAX = 448.0  # largest finite E4M3 magnitude
INT8_MAX = 127.0  # largest symmetric INT8 code


def kv_scales(cfg, ctx):
    """Per-tensor scales for an FP8 or INT8 cache: amax over all K (resp. V)
    values of all sequences (prefill and step rows), divided by the largest
    code magnitude (448 for E4M3, 127 for INT8), as float32."""
    if cfg.kv_dtype not in ("fp8", "int8"):
        return 1.0, 1.0
    top = E4M3_MAX if cfg.kv_dtype == "fp8" else INT8_MAX
    k, v = step_kv(cfg)
    ak, av = float(k.float().abs().max()), float(v.float().abs().max())
    for s in range(cfg.num_seqs):
        if int(ctx[s]) <= 1:
            continue
        k, v = seq_kv(cfg, s, int(ctx[s]) - 1)
        ak = max(ak, float(k.float().abs().max()))
        av = max(av, float(v.float().abs().max()))
    return float(np.float32(ak / top)), float(np.float32(av / top))


def misc_normal(cfg, key, shape, dtype):
    """Extra N(0,1) tensors for edge-case tests (stream keyed by `key`)."""
    x = rng(cfg, _STREAM_MISC, key).standard_normal(shape, dtype=np.float32)
    return round_to(x, dtype)


def query_lens(mq, ctx):
    """Rows per sequence of a multi-query step, int32[S]: the workload's count,
    at most the sequence's context."""
    S = len(ctx)
    if mq.qlen_kind == "fixed":
        n = np.full(S, mq.qlen_params[0], dtype=np.int64)
    elif mq.qlen_kind == "uniform":
        lo, hi = mq.qlen_params
        n = rng(mq.seed, _STREAM_QLEN).integers(lo, hi + 1, size=S)
    else:
        raise ValueError(mq.qlen_kind)
    return np.minimum(n, np.asarray(ctx, dtype=np.int64)).astype(np.int32)


def query_start(qlens):
    """Row offsets int32[S+1] of the sequences' rows, in sequence order."""
    qs = np.zeros(len(qlens) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(qlens)
    return qs


def mq_queries(mq, cfg, rows):
    """Query rows [rows][H_q][d] of a multi-query step, in the q dtype."""
    x = rng(mq.seed, _STREAM_MQ_Q).standard_normal(
        (rows, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
    return round_to(x, cfg.q_dtype)
