"""The decode workloads: shapes, dtypes, context-length mixes and seeds.

Shapes follow the models the pages use as examples (Qwen3-8B: 32 q-heads /
8 KV heads / head_dim 128; Llama-2-7B: 32 / 32 / 128; Llama-3-70B: 64 / 8 /
128 with FP8 KV).  The pages never publish a kernel-level benchmark, so every
input is synthetic: q, K and V are drawn N(0, 1) in float32 and rounded
(round-to-nearest-even) to the storage type.
"""
from dataclasses import dataclass
import math


@dataclass(frozen=True)
class Config:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str            # 'f32' | 'f16' | 'bf16' (also the output dtype)
    kv_dtype: str           # 'f32' | 'f16' | 'bf16' | 'fp8' | 'int8'
    ctx_kind: str           # 'list' | 'uniform' | 'lognormal' | 'fixed'
    ctx_params: tuple
    seed: int
    max_blocks_per_seq: int
    num_blocks: int = 0      # 0: ceil(pool_factor * demand)
    pool_factor: float = 1.25
    shared_prefix: int = 0   # tokens shared by every sequence (whole blocks)
    partition_size: int = 0  # 0: library's choice
    block_size: int = 16
    description: str = ""

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def new_dtype(self):
        """dtype of the K/V rows handed to cache-append (q dtype for FP8 and
        INT8 caches)."""
        return self.q_dtype if self.kv_dtype in ("fp8", "int8") else self.kv_dtype

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads


CONFIGS = {
    "c1_tiny_f32": Config(
        name="c1_tiny_f32", num_seqs=4, num_q_heads=4, num_kv_heads=2, head_dim=64,
        q_dtype="f32", kv_dtype="f32", ctx_kind="list", ctx_params=(5, 16, 17, 45),
        seed=1001, max_blocks_per_seq=3, num_blocks=16,
        description="tiny fp32, contexts {5,16,17,45}, GQA 2, 16-block pool"),
    "c2_qwen3_8b_bf16": Config(
        name="c2_qwen3_8b_bf16", num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        q_dtype="bf16", kv_dtype="bf16", ctx_kind="uniform", ctx_params=(256, 4096),
        seed=1002, max_blocks_per_seq=256,
        description="Qwen3-8B-shaped layer, bf16, batch 64, contexts U[256,4096]"),
    "c3_llama2_7b_f16": Config(
        name="c3_llama2_7b_f16", num_seqs=256, num_q_heads=32, num_kv_heads=32, head_dim=128,
        q_dtype="f16", kv_dtype="f16", ctx_kind="lognormal", ctx_params=(300.0, 0.6, 16, 2048),
        seed=1003, max_blocks_per_seq=128,
        description="Llama-2-7B-shaped MHA, fp16, batch 256, lognormal contexts mean 300"),
    "c4_llama3_70b_fp8": Config(
        name="c4_llama3_70b_fp8", num_seqs=32, num_q_heads=64, num_kv_heads=8, head_dim=128,
        q_dtype="bf16", kv_dtype="fp8", ctx_kind="fixed", ctx_params=(2560,),
        seed=1004, max_blocks_per_seq=160,
        description="Llama-3-70B-shaped layer, E4M3 KV (per-tensor scale), bf16 q/out, ctx 2560"),
    "c6_llama3_70b_int8": Config(
        name="c6_llama3_70b_int8", num_seqs=32, num_q_heads=64, num_kv_heads=8, head_dim=128,
        q_dtype="bf16", kv_dtype="int8", ctx_kind="fixed", ctx_params=(2560,),
        seed=1006, max_blocks_per_seq=160,
        description="Llama-3-70B-shaped layer, INT8 KV (symmetric, per-tensor scale), bf16 q/out, "
                    "ctx 2560"),
    "c5_long_shared_bf16": Config(
        name="c5_long_shared_bf16", num_seqs=16, num_q_heads=32, num_kv_heads=8, head_dim=128,
        q_dtype="bf16", kv_dtype="bf16", ctx_kind="fixed", ctx_params=(32768,),
        seed=1005, max_blocks_per_seq=2048, shared_prefix=2048, partition_size=512,
        description="32K-context bf16, 2048-token prefix shared by 16 tables, 512-token partitions"),
}


@dataclass(frozen=True)
class MQConfig:
    """A multi-query step on a decode workload's cache: each sequence's last
    qlen positions (a chunk of a prompt, or draft tokens under verification)
    attend causally in one pass.  The cache state, lengths and tables are the
    base workload's; only the query rows are new."""
    name: str
    base: str                # key of CONFIGS
    qlen_kind: str           # 'fixed' | 'uniform'
    qlen_params: tuple
    seed: int
    description: str = ""


MQ_CONFIGS = {
    "mq_c2_verify4": MQConfig(
        name="mq_c2_verify4", base="c2_qwen3_8b_bf16", qlen_kind="fixed", qlen_params=(4,),
        seed=2002, description="speculative verify, 4 rows per sequence (3 drafts + 1), "
                               "Qwen3-8B-shaped bf16 cache, batch 64"),
    "mq_c2_mixed": MQConfig(
        name="mq_c2_mixed", base="c2_qwen3_8b_bf16", qlen_kind="uniform", qlen_params=(0, 16),
        seed=2012, description="mixed batch, 0..16 rows per sequence (decode rows, drafts, "
                               "small chunks), Qwen3-8B-shaped bf16 cache"),
    "mq_c3_chunk64": MQConfig(
        name="mq_c3_chunk64", base="c3_llama2_7b_f16", qlen_kind="fixed", qlen_params=(64,),
        seed=2003, description="64-token prompt chunks (at most the context) on the "
                               "Llama-2-7B-shaped fp16 MHA cache, batch 256"),
    "mq_c4_verify8": MQConfig(
        name="mq_c4_verify8", base="c4_llama3_70b_fp8", qlen_kind="fixed", qlen_params=(8,),
        seed=2004, description="speculative verify, 8 rows per sequence, Llama-3-70B-shaped "
                               "E4M3 cache, batch 32"),
    "mq_c6_verify8": MQConfig(
        name="mq_c6_verify8", base="c6_llama3_70b_int8", qlen_kind="fixed", qlen_params=(8,),
        seed=2006, description="speculative verify, 8 rows per sequence, Llama-3-70B-shaped "
                               "INT8 cache, batch 32"),
    "mq_c5_chunk512": MQConfig(
        name="mq_c5_chunk512", base="c5_long_shared_bf16", qlen_kind="fixed", qlen_params=(512,),
        seed=2005, description="512-token prompt chunk at the end of each 32K context, bf16, "
                               "batch 16"),
}
