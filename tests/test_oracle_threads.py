"""The oracle's row-parallel entry points (rows shared among threads) give
the serial loop's result bit for bit: each (sequence, q-head) row, or
(query row, q-head) pair, is computed by one thread with the same loops in
the same order.  Checked on the tiny workload and on a slice of the
Qwen3-8B-shaped one, for decode and for multi-query rows."""
import numpy as np
import pytest

from harness import oracle_setup
from synth import CONFIGS, MQ_CONFIGS, gen


@pytest.mark.parametrize("name,seqs", [("c1_tiny_f32", None), ("c2_qwen3_8b_bf16", [0, 5, 63]),
                                       ("c4_llama3_70b_fp8", [3])])
def test_threaded_decode_is_bitwise_serial(name, seqs):
    from oracle import oracle as orc
    cfg = CONFIGS[name]
    o = oracle_setup(cfg, seqs)
    sel = list(range(cfg.num_seqs)) if seqs is None else seqs
    qb = gen.bits(o["q"])[sel]
    args = (qb, cfg.q_dtype, o["k_cache"], o["v_cache"], cfg.kv_dtype, o["block_tables"][sel],
            o["ctx"][sel], cfg.scale, o["k_scale"], o["v_scale"])
    serial = orc.paged_decode(*args, threads=1)
    for threads in (2, 3, 8):
        par = orc.paged_decode(*args, threads=threads)
        assert np.array_equal(serial.view(np.uint64), par.view(np.uint64)), threads


def test_threaded_multiquery_is_bitwise_serial():
    from oracle import oracle as orc
    mq = MQ_CONFIGS["mq_c2_mixed"]
    cfg = CONFIGS[mq.base]
    sel = [1, 2, 40]
    o = oracle_setup(cfg, sel)
    ql = gen.query_lens(mq, o["ctx"])[sel]
    qs = gen.query_start(ql)
    q = gen.bits(gen.misc_normal(cfg, 5, (int(qs[-1]), cfg.num_q_heads, cfg.head_dim),
                                 cfg.q_dtype))
    args = (q, cfg.q_dtype, o["k_cache"], o["v_cache"], cfg.kv_dtype, o["block_tables"][sel],
            o["ctx"][sel], qs, cfg.scale)
    serial = orc.paged_multiquery(*args, threads=1)
    for threads in (2, 5):
        par = orc.paged_multiquery(*args, threads=threads)
        assert np.array_equal(serial.view(np.uint64), par.view(np.uint64)), threads
