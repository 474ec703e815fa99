"""The decode entry point that allocates nothing
(pkv_paged_decode_attention_noalloc, through the C ABI) against the
workspace entry point on the same inputs: the same schedule and kernels, so
the same bits, and the oracle's tolerance on every row.  Two calls in a row
share the static scratch, the second on a smaller input; a schedule needing
more scratch than the array holds is refused before any launch."""
import numpy as np
import pytest
import torch

from harness import allclose_report
from gpu_harness import gpu_state, oracle_ref
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def both(st, cfg, seqs, ps):
    import paged_kv_cache_363_amd as pkv
    q = st["q"][seqs].contiguous()
    bt = st["block_tables"][seqs].contiguous()
    cl = st["context_lens"][seqs].contiguous()
    ref = pkv.paged_decode_attention(q, st["k_cache"], st["v_cache"], bt, cl, cfg.scale,
                                     st["k_scale"], st["v_scale"], partition_size=ps)
    out = torch.full_like(q, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    pkv.paged_decode_attention_noalloc(q, st["k_cache"], st["v_cache"], bt, cl, cfg.scale,
                                       st["k_scale"], st["v_scale"], partition_size=ps, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out, ref


@pytest.mark.parametrize("name,ps", [("c2_qwen3_8b_bf16", 0), ("c5_long_shared_bf16", 512),
                                     ("c4_llama3_70b_fp8", 256)])
def test_noalloc_matches_workspace_entry_point_twice(name, ps):
    print(f"[case] noalloc {name} partition={ps}", flush=True)
    cfg = CONFIGS[name]
    st = gpu_state(name)
    seqs_all, ref_all, _ = oracle_ref(name)
    full = list(range(cfg.num_seqs))
    small = full[: max(1, cfg.num_seqs // 4)][::-1]   # fewer sequences, another order
    for seqs in (full, small):
        out, ref = both(st, cfg, seqs, ps)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        got = out.float().cpu().numpy().astype(np.float64)
        ok, excess, err = allclose_report(got, ref_all[seqs], 2e-3, 1e-2)
        assert ok, f"{name}: max|err| {err}, worst excess {excess}"


def test_noalloc_refuses_schedules_beyond_the_scratch():
    import paged_kv_cache_363_amd as pkv
    cfg = CONFIGS["c2_qwen3_8b_bf16"]
    st = gpu_state(cfg.name)
    need = pkv.decode_workspace_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                     cfg.head_dim, cfg.max_blocks_per_seq, 2, 16)
    assert need > pkv.api.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(st["q"], 7.0)
    with pytest.raises(pkv.WorkspaceError, match="static scratch"):
        pkv.paged_decode_attention_noalloc(st["q"], st["k_cache"], st["v_cache"],
                                           st["block_tables"], st["context_lens"], cfg.scale,
                                           partition_size=16, out=out)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)   # nothing launched
