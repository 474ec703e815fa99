"""The decode step's append and attention in one call
(pkv_paged_decode_attention_appending) against the two calls it stands for:
pkv_paged_cache_append of the step's new rows, then the decode.  Both start
from identical caches that do not hold the step's token yet; afterwards the
caches must be identical bit for bit, and so must the outputs (the append
and the decode each already match the oracle: tests/test_gpu_append.py,
tests/test_gpu_decode.py).

Cases:
  - the planner's schedule and the balanced one (E4M3, INT8, bf16, f16 and
    f32 caches): on the MFMA kernels (fixed partitions, balanced grid,
    partitions on the persistent grid) the decode kernel appends the rows
    itself, on the vector kernel the call runs the append kernel first;
  - 512-token partitions on the persistent grid, and the 32K shared-prefix
    workload;
  - sequences without a new row (negative slot; their context stops before
    the step's token);
  - slots of earlier tokens of a sequence's own blocks (the row of token
    ctx-2, or of token ctx-17 in the block before the last);
  - 2100 short sequences with 16-token partitions: beyond the persistent
    grid's 2048 sequences the fixed-partition kernel runs several
    partitions, the last one holding the new token."""
import numpy as np
import pytest
import torch

from gpu_harness import gpu_setup
from synth import CONFIGS
from synth.configs import Config

pytestmark = pytest.mark.gpu


def raw(t):
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def run_both(st, ps, algo="auto", skip_every=0, back=0):
    """back > 0: every sequence with at least back + 1 tokens rewrites the row
    of token ctx - 1 - back instead (a slot of its own private blocks that
    is not the last token's, in the last block or an earlier one)."""
    import paged_kv_cache_363_amd as pkv
    cfg = st["cfg"]
    slots = st["step"]["slots"].clone()
    ctx = st["context_lens"].clone()
    if back:
        t = (ctx.long() - 1 - back)
        ok = t >= 0
        tc = t.clamp(min=0)
        bt = st["block_tables"].long()
        blk = bt.gather(1, (tc // 16).unsqueeze(1)).squeeze(1)
        slots = torch.where(ok, blk * 16 + tc % 16, slots)
    if skip_every:
        idx = torch.arange(0, cfg.num_seqs, skip_every, device=slots.device)
        slots[idx] = -1
        ctx[idx] -= 1      # without its new row a sequence's context ends before it
    k1, v1 = st["k_cache"].clone(), st["v_cache"].clone()
    k2, v2 = st["k_cache"].clone(), st["v_cache"].clone()
    kn, vn = st["step"]["k"], st["step"]["v"]
    pkv.paged_cache_append(k1, v1, kn, vn, slots, st["k_scale"], st["v_scale"])
    ref = pkv.paged_decode_attention(st["q"], k1, v1, st["block_tables"], ctx, cfg.scale,
                                     st["k_scale"], st["v_scale"], partition_size=ps, algo=algo)
    got = pkv.paged_decode_attention_appending(st["q"], kn, vn, slots, k2, v2,
                                               st["block_tables"], ctx, cfg.scale,
                                               st["k_scale"], st["v_scale"], partition_size=ps,
                                               algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(raw(k1), raw(k2)) and torch.equal(raw(v1), raw(v2)), "caches differ"
    assert torch.equal(raw(ref), raw(got)), \
        f"outputs differ: max|diff| {(ref.float() - got.float()).abs().max().item()}"


def planner_ps(st):
    import paged_kv_cache_363_amd as pkv
    cfg = st["cfg"]
    return pkv.decode_partition_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                     cfg.head_dim, cfg.max_blocks_per_seq,
                                     {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3, "int8": 4}[
                                         cfg.kv_dtype], 0, context_lens=st["ctx"])


_ST = {}


def state(name):
    if name not in _ST:
        _ST[name] = gpu_setup(CONFIGS[name], step_append=False)
    return _ST[name]


@pytest.mark.parametrize("name", ["c4_llama3_70b_fp8", "c6_llama3_70b_int8", "c2_qwen3_8b_bf16",
                                  "c3_llama2_7b_f16", "c1_tiny_f32"])
@pytest.mark.parametrize("skip_every", [0, 3])
def test_appending_decode_equals_append_then_decode(name, skip_every):
    if name not in CONFIGS:
        pytest.skip(f"no workload {name}")
    print(f"[case] appending decode {name} skip_every={skip_every}", flush=True)
    st = state(name)
    run_both(st, planner_ps(st), skip_every=skip_every)   # the planner's schedule
    run_both(st, 0, skip_every=skip_every)                # the balanced one where it applies


@pytest.mark.parametrize("name", ["c4_llama3_70b_fp8", "c2_qwen3_8b_bf16"])
@pytest.mark.parametrize("back", [1, 16])
def test_appending_decode_rewriting_an_earlier_token(name, back):
    if name not in CONFIGS:
        pytest.skip(f"no workload {name}")
    print(f"[case] appending decode {name} rewriting token ctx-1-{back}", flush=True)
    st = state(name)
    # one partition per context (the fixed-partition kernel), the balanced
    # grid, and 512-token partitions on the persistent grid
    for ps in (16 * st["cfg"].max_blocks_per_seq, 0, 512):
        run_both(st, ps, algo="mfma", back=back)


@pytest.mark.parametrize("name", ["c2_qwen3_8b_bf16", "c6_llama3_70b_int8"])
def test_appending_decode_in_partition_mode(name):
    if name not in CONFIGS:
        pytest.skip(f"no workload {name}")
    print(f"[case] appending decode {name}, 512-token partitions", flush=True)
    st = state(name)
    run_both(st, 512, algo="mfma")
    run_both(st, 512, algo="mfma", skip_every=4)


def test_appending_decode_long_shared_prefix():
    name = "c5_long_shared_bf16"
    if name not in CONFIGS:
        pytest.skip(f"no workload {name}")
    print(f"[case] appending decode {name} (its 512-token partitions, then balanced)", flush=True)
    st = gpu_setup(CONFIGS[name], step_append=False)
    run_both(st, CONFIGS[name].partition_size, algo="mfma")
    run_both(st, 0, algo="mfma")


def test_appending_decode_on_the_fixed_kernel_beyond_the_persistent_grid():
    print("[case] appending decode 2100 sequences, 16-token partitions", flush=True)
    rs = np.random.default_rng(31)
    ctxs = tuple(int(x) for x in rs.integers(1, 41, 2100))
    cfg = Config(name="append_many", num_seqs=len(ctxs), num_q_heads=8, num_kv_heads=2,
                 head_dim=128, q_dtype="bf16", kv_dtype="bf16", ctx_kind="list",
                 ctx_params=ctxs, seed=2100, max_blocks_per_seq=4)
    st = gpu_setup(cfg, step_append=False)
    run_both(st, 16, algo="mfma")
    run_both(st, 16, algo="mfma", skip_every=5)


@pytest.mark.parametrize("q_dtype,kv_dtype", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "fp8"),
                                              ("f16", "int8")])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_appending_decode_every_dtype_and_head_dim_on_every_mfma_schedule(q_dtype, kv_dtype,
                                                                          head_dim):
    """One element of each new row per lane (head_dim 64) or two (128), for
    16-bit copies and one-byte encodings, on the fixed-partition kernel (one
    pass), the balanced grid and 64-token partitions on the persistent grid
    (the fixed kernel's several partitions: the 2100-sequence test), and the
    vector kernel (append kernel first)."""
    print(f"[case] appending decode {q_dtype}/{kv_dtype} d={head_dim}", flush=True)
    rs = np.random.default_rng(head_dim + len(kv_dtype))
    ctxs = tuple(int(x) for x in rs.integers(1, 300, 24))
    cfg = Config(name="append_dtypes", num_seqs=len(ctxs), num_q_heads=8, num_kv_heads=2,
                 head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype, ctx_kind="list",
                 ctx_params=ctxs, seed=77 + head_dim, max_blocks_per_seq=19)
    st = gpu_setup(cfg, step_append=False)
    for ps in (16 * cfg.max_blocks_per_seq, 0, 64):
        run_both(st, ps, algo="mfma")
    run_both(st, 0, algo="mfma", skip_every=5, back=3)
    # the vector kernel: one pass, and 64-token partitions with the reduction
    for ps in (16 * cfg.max_blocks_per_seq, 64):
        run_both(st, ps, algo="vector")
    run_both(st, 64, algo="vector", skip_every=5, back=3)
