"""Pins for the oracle's multi-query attention (a chunk of a prompt, or draft
tokens under verification, attending through the block table).

Against: torch's scaled_dot_product_attention in float64 with an explicit
causal mask that ends at each query's position (an independent library
routine); the pinned single-query oracle (a one-row chunk is a decode step,
and every row is a decode step over its own prefix); closed forms (the first
row of a chunk that is the whole context sees only token 0)."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from test_oracle_attention import _bits, random_case


def chunk_rows(rs, S, hq, d, qlens, tdt):
    qs = np.zeros(S + 1, np.int32)
    qs[1:] = np.cumsum(qlens)
    q = torch.from_numpy(rs.standard_normal((int(qs[-1]), hq, d)).astype(np.float32)).to(tdt)
    return q, qs


def sdpa_causal(q, qs, ks, vs, ctx, scale):
    """Row r of sequence s: torch SDPA over that sequence's contiguous K/V with
    the mask t <= ctx - n + i."""
    out = np.zeros((q.shape[0], q.shape[1], q.shape[2]))
    for s in range(len(ctx)):
        r0, n = int(qs[s]), int(qs[s + 1] - qs[s])
        if n == 0:
            continue
        qq = q[r0:r0 + n].double().permute(1, 0, 2)[None]     # [1, Hq, n, d]
        kk = ks[s].double().permute(1, 0, 2)[None]             # [1, Hkv, ctx, d]
        vv = vs[s].double().permute(1, 0, 2)[None]
        pos = int(ctx[s]) - n + torch.arange(n)
        mask = torch.arange(int(ctx[s]))[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask[None, None], scale=scale, enable_gqa=True)
        out[r0:r0 + n] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 4, 4, 64),
                                            ("f32", 8, 2, 64)])
def test_matches_library_sdpa_with_causal_mask(dtype, hq, hkv, d):
    rs = np.random.default_rng(21)
    ctxs = [1, 5, 16, 17, 45, 100, 33]
    qlens = [1, 3, 16, 0, 45, 7, 1]      # a whole-context chunk, an empty one, ...
    c = random_case(rs, ctxs, hq, hkv, d, dtype)
    q, qs = chunk_rows(rs, len(ctxs), hq, d, qlens, c["q"].dtype)
    scale = 1.0 / math.sqrt(d)
    got = orc.paged_multiquery(_bits(q), dtype, c["kc"], c["vc"], dtype, c["bt"], c["ctx"],
                               qs, scale)
    ref = sdpa_causal(q, qs, c["ks"], c["vs"], c["ctx"], scale)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_one_row_per_sequence_is_the_decode_step():
    rs = np.random.default_rng(22)
    ctxs = [3, 16, 17, 64, 90]
    c = random_case(rs, ctxs, 8, 2, 64, "bf16")
    qs = np.arange(len(ctxs) + 1, dtype=np.int32)
    qb = _bits(c["q"])
    got = orc.paged_multiquery(qb, "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], qs, 0.125)
    ref = orc.paged_decode(qb, "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], 0.125)
    assert np.max(np.abs(got - ref)) < 1e-13


def test_every_row_is_a_decode_over_its_prefix():
    rs = np.random.default_rng(23)
    ctxs = [20, 50, 33]
    qlens = [8, 50, 5]
    c = random_case(rs, ctxs, 16, 4, 64, "bf16")
    q, qs = chunk_rows(rs, len(ctxs), 16, 64, qlens, torch.bfloat16)
    qb = _bits(q)
    got = orc.paged_multiquery(qb, "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], qs, 0.125)
    for s in range(len(ctxs)):
        n = qlens[s]
        for i in range(n):
            r = int(qs[s]) + i
            p = ctxs[s] - n + i
            ref = orc.paged_decode(qb[r:r + 1], "bf16", c["kc"], c["vc"], "bf16",
                                   c["bt"][s:s + 1], np.array([p + 1], np.int32), 0.125)
            assert np.max(np.abs(got[r] - ref[0])) < 1e-13


def test_first_row_of_a_whole_context_chunk_is_its_value():
    rs = np.random.default_rng(24)
    c = random_case(rs, [37], 8, 2, 64, "bf16")
    q, qs = chunk_rows(rs, 1, 8, 64, [37], torch.bfloat16)
    got = orc.paged_multiquery(_bits(q), "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"],
                               qs, 0.125)
    v0 = c["vs"][0][0].double().numpy()          # [Hkv][d]
    for h in range(8):
        assert np.array_equal(got[0, h], v0[h // 4])


def test_rows_past_the_context_and_unowned_rows_are_zero():
    rs = np.random.default_rng(25)
    c = random_case(rs, [4, 9], 4, 2, 64, "f32")
    # sequence 0 claims 6 rows for 4 tokens: its first 2 rows have no position;
    # rows 0..1 belong to nobody (query_start starts at 2)
    qs = np.array([2, 8, 10], np.int32)
    q = torch.from_numpy(rs.standard_normal((12, 4, 64)).astype(np.float32))
    got = orc.paged_multiquery(_bits(q), "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"],
                               qs, 0.125)
    assert not got[0:2].any() and not got[10:12].any()
    assert not got[2:4].any() and np.all(got[4:10] != 0)
