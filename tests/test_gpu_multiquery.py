"""Multi-query attention parity: the HIP kernel (through the C ABI) against the
fp64 oracle, element by element.

Every workload reuses a decode workload's device cache (filled by the
library's append, the step's token included) and adds seeded query rows.
Every row of every sequence is checked against oracle.paged_multiquery.
For the 512-row chunks at the end of 32K contexts the full oracle would run
for hours, so six rows of each of the 16 sequences (the first, the last and
four interior ones) are checked against oracle.paged_decode over the row's
own prefix (a pinned identity: row i of n is the decode step of a context of
ctx - n + i + 1 tokens).  Tolerance as for decode:
|gpu - ref| <= 2e-3 + 1e-2 |ref| per element."""
import numpy as np
import pytest
import torch

from harness import allclose_report
from gpu_harness import gpu_state, oracle_ref
from synth import CONFIGS, MQ_CONFIGS, gen

pytestmark = pytest.mark.gpu

_MQ = {}


def mq_state(name):
    if name not in _MQ:
        mq = MQ_CONFIGS[name]
        cfg = CONFIGS[mq.base]
        st = gpu_state(mq.base)
        ql = gen.query_lens(mq, st["ctx"])
        qs = gen.query_start(ql)
        q = gen.mq_queries(mq, cfg, int(qs[-1]))
        _MQ[name] = dict(mq=mq, cfg=cfg, st=st, ql=ql, qs=qs, q=q,
                         q_dev=q.to("cuda"), qs_dev=torch.from_numpy(qs).to("cuda"))
    return _MQ[name]


def run_mq(m, partition_size=0, out=None):
    import paged_kv_cache_363_amd as pkv
    st, cfg = m["st"], m["cfg"]
    out = pkv.paged_multiquery_attention(
        m["q_dev"], st["k_cache"], st["v_cache"], st["block_tables"], st["context_lens"],
        m["qs_dev"], int(m["ql"].max(initial=0)), cfg.scale, st["k_scale"], st["v_scale"],
        partition_size=partition_size, out=out)
    torch.cuda.synchronize()
    return out


_MQ_REF = {}


def oracle_rows(m, seqs):
    """fp64 rows of the given sequences (oracle.paged_multiquery on the
    oracle-side caches), computed once per workload and sequence set."""
    from oracle import oracle as orc
    cfg = m["cfg"]
    key = (m["mq"].name, tuple(seqs))
    if key in _MQ_REF:
        return _MQ_REF[key]
    _, _, o = oracle_ref(cfg.name)
    qs, ql = m["qs"], m["ql"]
    sub_qs = np.zeros(len(seqs) + 1, np.int32)
    sub_qs[1:] = np.cumsum([int(ql[s]) for s in seqs])
    rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs]).astype(np.int64)
    qb = gen.bits(m["q"])[rows]
    ref = orc.paged_multiquery(qb, cfg.q_dtype, o["k_cache"], o["v_cache"], cfg.kv_dtype,
                               o["block_tables"][seqs], o["ctx"][seqs], sub_qs, cfg.scale,
                               o["k_scale"], o["v_scale"])
    _MQ_REF[key] = (rows, ref)
    return rows, ref


def check(got, ref, what):
    ok, excess, err = allclose_report(got, ref, 2e-3, 1e-2)
    assert ok, f"{what}: max|err| {err}, worst excess over bound {excess}"


CASES = [("mq_c2_verify4", 0), ("mq_c2_mixed", 0), ("mq_c2_mixed", 16), ("mq_c2_mixed", 512),
         ("mq_c2_mixed", 4096), ("mq_c3_chunk64", 0), ("mq_c3_chunk64", 128),
         ("mq_c4_verify8", 0), ("mq_c4_verify8", 2560), ("mq_c6_verify8", 0),
         ("mq_c6_verify8", 2560)]


@pytest.mark.parametrize("name,ps", CASES)
def test_multiquery_matches_oracle(name, ps):
    print(f"[case] multiquery {name} partition={ps}", flush=True)
    m = mq_state(name)
    seqs, _, _ = oracle_ref(m["cfg"].name)
    seqs = [s for s in seqs if m["ql"][s] > 0] or seqs
    rows, ref = oracle_rows(m, seqs)
    out = run_mq(m, ps)
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    check(got, ref, f"{name} ps={ps}")


_CHUNK_REF = {}


def chunk_rows_reference(m):
    """Rows (first, two near the start, two interior, last) of every sequence
    of the 512-row chunk workload, and their fp64 references: each row is
    the decode of its own prefix, so all of them go to the oracle as one
    decode batch whose 'sequences' are (sequence, row) pairs sharing the
    sequence's block table."""
    from oracle import oracle as orc
    if "c5" in _CHUNK_REF:
        return _CHUNK_REF["c5"]
    cfg = m["cfg"]
    seqs, _, o = oracle_ref(cfg.name)
    qb = gen.bits(m["q"])
    rows, tables, lens = [], [], []
    for s in seqs:
        n, ctx = int(m["ql"][s]), int(m["st"]["ctx"][s])
        for i in sorted({0, 1, 128, 255, 400, n - 1}):
            rows.append(int(m["qs"][s]) + i)
            tables.append(o["block_tables"][s])
            lens.append(ctx - n + i + 1)
    rows = np.array(rows, np.int64)
    ref = orc.paged_decode(qb[rows], cfg.q_dtype, o["k_cache"], o["v_cache"], cfg.kv_dtype,
                           np.stack(tables), np.array(lens, np.int32), cfg.scale,
                           o["k_scale"], o["v_scale"])
    _CHUNK_REF["c5"] = (rows, ref)
    return rows, ref


@pytest.mark.parametrize("ps", [0, 4096])
def test_long_context_chunk_rows_match_decode_over_their_prefix(ps):
    print(f"[case] multiquery mq_c5_chunk512 partition={ps}", flush=True)
    m = mq_state("mq_c5_chunk512")
    rows, ref = chunk_rows_reference(m)
    out = run_mq(m, ps).float().cpu().numpy().astype(np.float64)
    assert len(rows) == 6 * m["cfg"].num_seqs
    check(out[rows], ref, f"chunk rows partition={ps}")


def test_rows_outside_the_sequences_untouched_and_unplaced_rows_zero():
    """query_start beginning at row 2 leaves rows 0-1 and the trailing rows as
    they were; a sequence claiming more rows than its context gets zeros in the
    rows whose position is negative."""
    import paged_kv_cache_363_amd as pkv
    m = mq_state("mq_c2_verify4")
    st, cfg = m["st"], m["cfg"]
    S = cfg.num_seqs
    ctx0 = int(st["ctx"][0])
    ql = np.full(S, 2, np.int32)
    ql[0] = ctx0 + 3                      # three rows before position 0
    qs = np.zeros(S + 1, np.int32)
    qs[0] = 2
    qs[1:] = 2 + np.cumsum(ql)
    rows = int(qs[-1]) + 5
    q = gen.misc_normal(cfg, 91, (rows, cfg.num_q_heads, cfg.head_dim), cfg.q_dtype).to("cuda")
    out = torch.full_like(q, 7.0)
    pkv.paged_multiquery_attention(q, st["k_cache"], st["v_cache"], st["block_tables"],
                                   st["context_lens"], torch.from_numpy(qs).to("cuda"),
                                   int(ql.max()), cfg.scale, partition_size=0, out=out)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.all(o[:2] == 7.0) and torch.all(o[int(qs[-1]):] == 7.0)
    assert torch.all(o[2:5] == 0.0)
    assert torch.isfinite(o[5:int(qs[-1])]).all()
    # the first placed row of sequence 0 attends to token 0 only: its value row
    from oracle import oracle as orc
    _, _, oo = oracle_ref(cfg.name)
    if 0 in oracle_ref(cfg.name)[0]:
        ref = orc.paged_decode(gen.bits(q.cpu())[5:6], cfg.q_dtype, oo["k_cache"], oo["v_cache"],
                               cfg.kv_dtype, oo["block_tables"][0:1], np.array([1], np.int32),
                               cfg.scale)
        check(o[5:6].numpy().astype(np.float64), ref, "first placed row")


def test_one_row_per_sequence_matches_the_decode_oracle():
    import paged_kv_cache_363_amd as pkv
    cfg = CONFIGS["c2_qwen3_8b_bf16"]
    st = gpu_state(cfg.name)
    seqs, ref, _ = oracle_ref(cfg.name)
    qs = torch.arange(cfg.num_seqs + 1, dtype=torch.int32, device="cuda")
    out = pkv.paged_multiquery_attention(st["q"], st["k_cache"], st["v_cache"],
                                         st["block_tables"], st["context_lens"], qs, 1, cfg.scale)
    torch.cuda.synchronize()
    check(out.float().cpu().numpy().astype(np.float64)[seqs], ref, "one row per sequence")
