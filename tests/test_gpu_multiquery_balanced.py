"""Multi-query attention on small, hand-shaped batches against the fp64
oracle: every row of every sequence is compared element by element
(|gpu - ref| <= 2e-3 + 1e-2 |ref|), for the work-balanced schedule
(partition_size 0) and for the fixed grid (partitions of 64 tokens, and one
pass over the context).  The shapes put 1, 2 and 4 column tiles of 16
(row, q-head) columns in one wave, on both schedules.

The batches hold the cases the schedule has to get right:
  - a sequence without context (all its rows get zeros);
  - more rows than context tokens (the rows before position 0 get zeros);
  - sequences with no rows, one row, and rows that end a partial row tile;
  - contexts on and off 16-token block boundaries.
The balanced schedule runs with 4 to 4000 waves (pkv_set_stream_workgroups),
so that segments are kept whole by one wave, split between two, or spread
over many, and the merge kernel sees all of these.  Rows outside every
sequence must keep their contents."""
import numpy as np
import pytest
import torch

from gpu_harness import gpu_setup
from harness import allclose_report, oracle_setup
from oracle import oracle as orc
from synth import gen
from synth.configs import Config

pytestmark = pytest.mark.gpu

CTXS = [5, 3, 17, 40, 100, 16, 1, 300, 33]
QLS = [2, 6, 20, 1, 33, 0, 1, 40, 16]     # sequence 0 is given context 0 below
SHAPES = [
    # (q, kv, H_q, H_kv, d): g = 4, MHA (2 column tiles of 16 rows for 40
    # rows), g = 8 FP8, g = 12 INT8 d = 64, g = 20 (two head chunks); the
    # others take 4 column tiles
    ("bf16", "bf16", 32, 8, 128),
    ("f16", "f16", 16, 16, 128),
    ("bf16", "fp8", 64, 8, 128),
    ("bf16", "int8", 24, 2, 64),
    ("f16", "fp8", 40, 2, 128),
]
WORKGROUPS = [1, 7, 256, 1000]
# Block tables 8192 tokens wide (the contexts stay short): the fixed grid then
# also carries several column tiles per wave, as it does for long contexts.
MB = 512


@pytest.mark.parametrize("q,kv,hq,hkv,d", SHAPES)
def test_multiquery_batches_match_oracle(q, kv, hq, hkv, d):
    import paged_kv_cache_363_amd as pkv
    name = f"mqb_{q}_{kv}_{hq}_{hkv}_{d}"
    print(f"[case] balanced multiquery {name}", flush=True)
    cfg = Config(name=name, num_seqs=len(CTXS), num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 q_dtype=q, kv_dtype=kv, ctx_kind="list", ctx_params=tuple(CTXS),
                 seed=hq * 31 + d, max_blocks_per_seq=MB)
    st = gpu_setup(cfg)
    o = oracle_setup(cfg)
    S = cfg.num_seqs
    ctx = st["ctx"].copy()
    ctx[0] = 0
    ql = np.array(QLS, np.int32)
    qs = np.zeros(S + 1, np.int32)
    qs[0] = 2                                   # rows 0-1 belong to no sequence
    qs[1:] = 2 + np.cumsum(ql)
    rows = int(qs[-1]) + 3                      # and so do the last three
    maxq = int(ql.max())
    assert pkv.multiquery_partition_size(S, maxq, hq, hkv, cfg.max_blocks_per_seq) == 0
    qt = gen.misc_normal(cfg, 77, (rows, hq, d), q)
    ref = orc.paged_multiquery(gen.bits(qt)[2:int(qs[-1])], q, o["k_cache"], o["v_cache"], kv,
                               o["block_tables"], ctx, qs - 2, cfg.scale, o["k_scale"],
                               o["v_scale"])
    cl = torch.from_numpy(ctx).to("cuda")
    qs_dev = torch.from_numpy(qs).to("cuda")
    q_dev = qt.to("cuda")
    runs = [(w, 0) for w in WORKGROUPS] + [(0, 64), (0, 16 * cfg.max_blocks_per_seq)]
    try:
        for wgs, ps in runs:
            pkv.lib().pkv_set_stream_workgroups(wgs)
            out = torch.full_like(q_dev, 7.0)
            pkv.paged_multiquery_attention(q_dev, st["k_cache"], st["v_cache"],
                                           st["block_tables"], cl, qs_dev, maxq, cfg.scale,
                                           st["k_scale"], st["v_scale"], partition_size=ps,
                                           out=out)
            torch.cuda.synchronize()
            got = out.float().cpu()
            what = f"partition {ps}" if ps else f"{wgs} workgroups"
            assert torch.all(got[:2] == 7.0) and torch.all(got[int(qs[-1]):] == 7.0), what
            ok, excess, err = allclose_report(got[2:int(qs[-1])].numpy().astype(np.float64),
                                              ref, 2e-3, 1e-2)
            assert ok, f"{what}: max|err| {err}, worst excess {excess}"
            # the context-free sequence and the rows before position 0 are zeros
            assert torch.all(got[2:4] == 0.0)
            assert torch.all(got[int(qs[1]):int(qs[1]) + 3] == 0.0)
    finally:
        pkv.lib().pkv_set_stream_workgroups(0)
