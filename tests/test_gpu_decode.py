"""Decode attention parity: the HIP kernels (through the C ABI) against the fp64
oracle on the five workloads, element by element.

Tolerances: f32 caches max|err| <= 1e-5; 16-bit and FP8 caches
|gpu - ref| <= 2e-3 + 1e-2 |ref| per element (outputs are rounded to the q
dtype, whose half-ulp is at most 2^-9 relative, and the MFMA path rounds the
softmax weights to the q dtype, about 2^-9 relative per weight).
Every output row of every sequence is compared, at the workloads' full sizes
and in every schedule, grid size and partition size below."""
import numpy as np
import pytest
import torch

from harness import allclose_report
from gpu_harness import gpu_state, oracle_ref
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def run_decode(st, algo="auto", partition_size=None):
    import paged_kv_cache_363_amd as pkv
    cfg = st["cfg"]
    ps = cfg.partition_size if partition_size is None else partition_size
    if ps == "plan":   # the host planner's choice for these lengths
        ps = pkv.decode_partition_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                       cfg.head_dim, cfg.max_blocks_per_seq,
                                       pkv.api.dtype_code(st["k_cache"]), 0,
                                       context_lens=st["context_lens"].cpu().numpy())
    out = pkv.paged_decode_attention(st["q"], st["k_cache"], st["v_cache"], st["block_tables"],
                                     st["context_lens"], cfg.scale, st["k_scale"], st["v_scale"],
                                     partition_size=ps, algo=algo)
    torch.cuda.synchronize()
    return out


def check_parity(name, out, seqs, ref):
    cfg = CONFIGS[name]
    got = out.float().cpu().numpy().astype(np.float64)[seqs]
    if cfg.kv_dtype == "f32":
        err = float(np.max(np.abs(got - ref)))
        assert np.all(np.isfinite(got)) and err <= 1e-5, f"{name}: max|err| {err}"
    else:
        ok, excess, err = allclose_report(got, ref, 2e-3, 1e-2)
        assert ok, f"{name}: max|err| {err}, worst excess over bound {excess}"


# (algo, partition): partition None = the workload's own setting; 0 with a
# 16-bit or FP8 cache = the balanced schedule; > 0 = fixed partitions + reduce
# (single pass when it covers max_blocks_per_seq * 16); "plan" = what the
# host planner picks for the workload's lengths
SCHEDULES = {
    "c1_tiny_f32": [("auto", None), ("vector", 16), ("auto", "plan")],
    "c2_qwen3_8b_bf16": [("auto", None), ("mfma", 0), ("mfma", 512), ("vector", 0),
                         ("auto", "plan")],
    "c3_llama2_7b_f16": [("auto", None), ("mfma", 0), ("mfma", 256), ("vector", 2048),
                         ("auto", "plan")],
    "c4_llama3_70b_fp8": [("auto", None), ("mfma", 0), ("mfma", 256), ("vector", 512),
                          ("mfma", 2560), ("auto", "plan")],
    "c5_long_shared_bf16": [("auto", None), ("mfma", 0), ("mfma", 512), ("vector", 1024),
                            ("auto", "plan")],
    "c6_llama3_70b_int8": [("auto", None), ("mfma", 0), ("mfma", 256), ("vector", 512),
                           ("mfma", 2560), ("auto", "plan")],
}
CASES = [(n, a, ps) for n in CONFIGS for a, ps in SCHEDULES[n]]


@pytest.mark.parametrize("name,algo,ps", CASES)
def test_decode_matches_oracle(name, algo, ps):
    print(f"[case] decode {name} algo={algo} partition={ps}", flush=True)
    st = gpu_state(name)
    seqs, ref, _ = oracle_ref(name)
    out = run_decode(st, algo, ps)
    check_parity(name, out, seqs, ref)


@pytest.mark.parametrize("wgs", [1, 3, 37, 512, 2048])
@pytest.mark.parametrize("name", ["c2_qwen3_8b_bf16", "c4_llama3_70b_fp8"])
def test_balanced_schedule_any_grid(name, wgs):
    """The balanced schedule cuts the work into as many shares as it has
    waves; every grid size must give the same answer (shares spanning many
    segments, segments spanning many shares, shares of one block)."""
    import paged_kv_cache_363_amd as pkv
    print(f"[case] balanced {name} workgroups={wgs}", flush=True)
    st = gpu_state(name)
    seqs, ref, _ = oracle_ref(name)
    pkv.lib().pkv_set_stream_workgroups(wgs)
    try:
        out = run_decode(st, "mfma", 0)
    finally:
        pkv.lib().pkv_set_stream_workgroups(0)
    check_parity(name, out, seqs, ref)


@pytest.mark.parametrize("wgs", [1, 3, 37, 512, 2048])
@pytest.mark.parametrize("name,ps", [("c2_qwen3_8b_bf16", 512), ("c2_qwen3_8b_bf16", 16),
                                     ("c4_llama3_70b_fp8", 256)])
def test_fixed_partitions_on_any_grid(name, ps, wgs):
    """Fixed partitions on the MFMA path run on the persistent grid: share
    boundaries move up to partition boundaries, each wave closes whole
    partitions into an LDS stash and writes it out when full (16-token
    partitions fill it many times per share), and the split-K reduction merges
    them.  Every grid size must give the oracle's answer, and the same bits as
    the default grid."""
    import paged_kv_cache_363_amd as pkv
    print(f"[case] fixed partitions {name} partition={ps} workgroups={wgs}", flush=True)
    st = gpu_state(name)
    seqs, ref, _ = oracle_ref(name)
    base = run_decode(st, "mfma", ps)
    pkv.lib().pkv_set_stream_workgroups(wgs)
    try:
        out = run_decode(st, "mfma", ps)
    finally:
        pkv.lib().pkv_set_stream_workgroups(0)
    check_parity(name, out, seqs, ref)
    # a partition's (m, l, acc) does not depend on which wave computed it
    assert torch.equal(out.view(torch.int16), base.view(torch.int16))


def test_balanced_schedule_ignores_stale_workspace():
    """The workspace only carries partials written and read within one call:
    a workspace full of garbage or left by earlier calls gives the same
    result, bit for bit."""
    import paged_kv_cache_363_amd as pkv
    name = "c2_qwen3_8b_bf16"
    st = gpu_state(name)
    cfg = st["cfg"]
    ws = pkv.alloc_workspace(st["q"], st["k_cache"], st["block_tables"], 0)
    outs = []
    for fill in (None, 0xFF, 0x00, 0x5A):
        if fill is not None:
            ws.fill_(fill)
        outs.append(pkv.paged_decode_attention(st["q"], st["k_cache"], st["v_cache"],
                                               st["block_tables"], st["context_lens"], cfg.scale,
                                               workspace=ws, algo="mfma"))
        torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("ps", [16, 64, 128, 512, 1024, 4096])
@pytest.mark.parametrize("algo", ["vector", "mfma"])
def test_partition_sizes_agree_with_oracle(ps, algo):
    name = "c2_qwen3_8b_bf16"
    print(f"[case] partition {ps} {algo}", flush=True)
    st = gpu_state(name)
    seqs, ref, _ = oracle_ref(name)
    out = run_decode(st, algo, partition_size=ps)
    check_parity(name, out, seqs, ref)


def test_tiny_config_all_outputs_and_single_pass():
    import paged_kv_cache_363_amd as pkv
    name = "c1_tiny_f32"
    cfg = CONFIGS[name]
    assert pkv.decode_workspace_size(4, 4, 2, 64, cfg.max_blocks_per_seq, 0, 0) == 0
    st = gpu_state(name)
    seqs, ref, _ = oracle_ref(name)
    assert seqs == [0, 1, 2, 3]
    for ps in (0, 16, 32):
        out = run_decode(st, "vector", ps)
        check_parity(name, out, seqs, ref)
