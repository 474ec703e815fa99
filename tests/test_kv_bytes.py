"""KV-cache size formula against the pages' worked numbers: bytes per token =
2 x layers x kv_heads x head_dim x element bytes ("Transformer 推理优化：KV
Cache、PagedAttention 与 vLLM", section 2.5; "推理加速三板斧", section 2.2)."""
import json
import math
import os

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        return json.load(f)


def test_qwen3_8b_bytes_per_token_and_table():
    g = _g()["qwen3_8b"]
    b = orc.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype"])
    assert b == g["bytes_per_token"] == 147456
    unit = {"MiB": 2 ** 20, "GiB": 2 ** 30}
    for row in g["per_request"]:
        size = b * row["tokens"] / unit[row["unit"]]
        # the page prints these rounded ("~288 MB", "~1.1 GB", "~4.5 GB")
        assert abs(size - row["approx"]) <= 0.05 * row["approx"]


def test_llama3_70b_sizes_and_concurrency():
    g = _g()["llama3_70b"]
    b = orc.kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype"])
    assert b == 327680
    for row, conc in zip(g["per_request"], g["max_concurrency"]):
        gb = b * row["tokens"] / 1e9
        # the page truncates to one decimal (1.342 -> 1.3, 2.684 -> 2.6, 10.737 -> 10.7)
        assert math.floor(gb * 10) / 10 == row["approx"]
        assert math.floor(g["budget_gb"] * 1e9 / (b * row["tokens"])) == conc


def test_fp8_halves_the_cache():
    assert orc.kv_bytes_per_token(80, 8, 128, "fp8") * 2 == orc.kv_bytes_per_token(80, 8, 128, "f16")
