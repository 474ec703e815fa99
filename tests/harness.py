"""Test orchestration shared by CPU and GPU tests.

`synth.scenario.build_state` replays a workload's pool operations on either
pool; `oracle_setup` then fills oracle-side caches with the oracle's own
append.
"""
import numpy as np

from synth import gen
from synth.scenario import build_state, table_array  # noqa: F401


def poison_bits(dtype):
    """NaN bit pattern used to fill never-written cache slots."""
    return {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F), "int8": np.int8(127)}[dtype]   # int8 has no NaN


def oracle_setup(cfg, seqs=None):
    """Oracle-side caches and metadata for cfg, built with the reference pool
    and the oracle's append.  `seqs` limits which sequences' K/V are written
    (others keep their table but their blocks stay poisoned)."""
    from oracle import oracle as orc
    from oracle.pool_ref import RefPool

    ctx = gen.context_lens(cfg)
    nb = gen.num_blocks(cfg, ctx)
    pool = RefPool(nb, cfg.block_size, gen.free_order(cfg, nb))
    st = build_state(cfg, pool, ctx)
    kd, nd = cfg.kv_dtype, cfg.new_dtype
    shape = (nb, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    kc = np.full(shape, poison_bits(kd), dtype=orc.BITS_NP[kd])
    vc = np.full(shape, poison_bits(kd), dtype=orc.BITS_NP[kd])
    k_scale, v_scale = gen.kv_scales(cfg, ctx)
    want = set(range(cfg.num_seqs)) if seqs is None else set(seqs)
    if cfg.shared_prefix:
        want.add(0)
    for s, p0, slots in st["prefill"]:
        if s not in want or not slots:
            continue
        k, v = gen.seq_kv(cfg, s, p0 + len(slots))
        orc.cache_append(kc, vc, gen.bits(k[p0:]), gen.bits(v[p0:]),
                         np.array(slots, np.int64), nd, kd, k_scale, v_scale)
    # the decode step's own append of the new token
    kn, vn = gen.step_kv(cfg)
    sl = st["step_slots"].copy()
    for s in range(cfg.num_seqs):
        if s not in want:
            sl[s] = -1
    orc.cache_append(kc, vc, gen.bits(kn), gen.bits(vn), sl, nd, kd, k_scale, v_scale)
    return dict(ctx=ctx, nb=nb, pool=pool, state=st, k_cache=kc, v_cache=vc,
                block_tables=table_array(cfg, st["tables"]), q=gen.queries(cfg),
                k_scale=k_scale, v_scale=v_scale, step_k=kn, step_v=vn)


def allclose_report(got, ref, atol, rtol):
    """Elementwise |got-ref| <= atol + rtol*|ref|; returns (ok, worst excess, max abs err)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    excess = err - bound
    ok = bool(np.all(np.isfinite(got)) and np.all(excess <= 0))
    return ok, float(np.max(excess)) if excess.size else 0.0, float(np.max(err)) if err.size else 0.0
