"""Pins for the oracle's decode attention, split-K merge and append.

Each check is against something other than the oracle's own formula:
torch's scaled_dot_product_attention (an independent library routine, run in
float64 on contiguous K/V), closed forms, the pages' worked block-table
example, and invariants the pages state (paging changes only where K/V live;
shared prefix blocks give the same result as private copies)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t):
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().view(torch.uint8).numpy()


NAN_BITS = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F), "int8": np.int8(127)}   # int8 has no NaN: a large code
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def place(tables, seq_vals, nb, hkv, bs, d, dtype):
    """Scatter contiguous per-sequence K (or V) rows [n][H][d] (raw bits) into a
    NaN-poisoned paged cache, token t of sequence s going to physical block
    tables[s][t // bs], slot t % bs."""
    cache = np.full((nb, hkv, bs, d), NAN_BITS[dtype], dtype=orc.BITS_NP[dtype])
    for s, rows in enumerate(seq_vals):
        for t in range(rows.shape[0]):
            cache[tables[s][t // bs], :, t % bs, :] = rows[t]
    return cache


def sdpa_ref(q, ks, vs, scale):
    """torch SDPA (float64, GQA) per sequence on contiguous K/V [n][H_kv][d]."""
    outs = []
    for s in range(q.shape[0]):
        qq = q[s].double()[None, :, None, :]              # [1, Hq, 1, d]
        kk = ks[s].double().permute(1, 0, 2)[None]         # [1, Hkv, n, d]
        vv = vs[s].double().permute(1, 0, 2)[None]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale,
                                                              enable_gqa=True)
        outs.append(o[0, :, 0, :])
    return torch.stack(outs).numpy()


def random_case(rs, ctxs, hq, hkv, d, dtype, bs=16, slack=3, tdt=None):
    S = len(ctxs)
    nblk = [-(-n // bs) for n in ctxs]
    nb = sum(nblk) + slack
    perm = rs.permutation(nb)
    tables, i = [], 0
    for s in range(S):
        tables.append(perm[i:i + nblk[s]].tolist())
        i += nblk[s]
    tdt = tdt or TDT[dtype]
    q = torch.from_numpy(rs.standard_normal((S, hq, d)).astype(np.float32)).to(tdt)
    ks = [torch.from_numpy(rs.standard_normal((n, hkv, d)).astype(np.float32)).to(tdt) for n in ctxs]
    vs = [torch.from_numpy(rs.standard_normal((n, hkv, d)).astype(np.float32)).to(tdt) for n in ctxs]
    mb = max(max(nblk), 1)
    bt = np.full((S, mb), -1, np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    kc = place(tables, [_bits(k) for k in ks], nb, hkv, bs, d, dtype)
    vc = place(tables, [_bits(v) for v in vs], nb, hkv, bs, d, dtype)
    return dict(q=q, ks=ks, vs=vs, tables=tables, bt=bt, kc=kc, vc=vc,
                ctx=np.array(ctxs, np.int32), nb=nb)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 2, 64), ("bf16", 32, 8, 128),
                                            ("f16", 8, 8, 128), ("bf16", 64, 8, 128)])
def test_paged_matches_library_sdpa(dtype, hq, hkv, d):
    rs = np.random.default_rng(11)
    c = random_case(rs, [1, 5, 16, 17, 45, 100], hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    got = orc.paged_decode(_bits(c["q"]), dtype, c["kc"], c["vc"], dtype, c["bt"], c["ctx"], scale)
    ref = sdpa_ref(c["q"], c["ks"], c["vs"], scale)
    assert np.all(np.isfinite(got))  # NaN-poisoned tails and free blocks never leak in
    assert np.max(np.abs(got - ref)) < 1e-12


def test_gqa_mapping_is_consecutive():
    """q-head h reads kv-head h // g: with two kv-heads holding very different
    values, a modulo mapping would give a different answer."""
    rs = np.random.default_rng(5)
    c = random_case(rs, [20], 4, 2, 64, "f32")
    got = orc.paged_decode(_bits(c["q"]), "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"], 0.125)
    ref = sdpa_ref(c["q"], c["ks"], c["vs"], 0.125)
    wrong = sdpa_ref(c["q"][:, [0, 2, 1, 3]], c["ks"], c["vs"], 0.125)[:, [0, 2, 1, 3]]
    assert np.max(np.abs(got - ref)) < 1e-12
    assert np.max(np.abs(got - wrong)) > 1e-3


def test_p1_block_table_example():
    """The pages' worked example: 8 physical blocks, sequence A (45 tokens) in
    blocks [2,5,0], sequence B (20 tokens) in [7,3], blocks 1,4,6 free."""
    with open(os.path.join(GOLDEN, "p1_block_table.json")) as f:
        g = json.load(f)
    A, B = g["sequences"]["A"], g["sequences"]["B"]
    bs, nb = g["block_size"], g["num_blocks"]
    rs = np.random.default_rng(2)
    hq, hkv, d = 4, 2, 64
    ks = [torch.from_numpy(rs.standard_normal((n, hkv, d)).astype(np.float32)) for n in (A["tokens"], B["tokens"])]
    vs = [torch.from_numpy(rs.standard_normal((n, hkv, d)).astype(np.float32)) for n in (A["tokens"], B["tokens"])]
    q = torch.from_numpy(rs.standard_normal((2, hq, d)).astype(np.float32))
    tables = [A["table"], B["table"]]
    kc = place(tables, [k.numpy() for k in ks], nb, hkv, bs, d, "f32")
    vc = place(tables, [v.numpy() for v in vs], nb, hkv, bs, d, "f32")
    # the layout string of the page: which logical block sits in each physical block
    used = {b for t in tables for b in t}
    assert sorted(set(range(nb)) - used) == g["free"]
    for phys, label in enumerate(g["physical_layout"]):
        if label == "free":
            assert np.all(np.isnan(kc[phys]))
        else:
            seq, j = label.split("_")
            assert tables[0 if seq == "A" else 1][int(j)] == phys
    bt = np.full((2, 3), -1, np.int32)
    bt[0, :3] = tables[0]
    bt[1, :2] = tables[1]
    got = orc.paged_decode(q.numpy(), "f32", kc, vc, "f32", bt, [A["tokens"], B["tokens"]], 0.125)
    ref = sdpa_ref(q, ks, vs, 0.125)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_single_token_returns_its_value_exactly():
    rs = np.random.default_rng(8)
    c = random_case(rs, [1, 1], 8, 2, 128, "bf16")
    got = orc.paged_decode(_bits(c["q"]), "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], 0.1)
    for s in range(2):
        for h in range(8):
            assert np.array_equal(got[s, h], c["vs"][s][0, h // 4].double().numpy())


def test_zero_query_gives_mean_of_values():
    rs = np.random.default_rng(9)
    c = random_case(rs, [37], 2, 1, 64, "f32")
    q0 = np.zeros((1, 2, 64), np.float32)
    got = orc.paged_decode(q0, "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"], 0.125)
    mean = c["vs"][0][:, 0, :].double().mean(0).numpy()
    assert np.max(np.abs(got[0, 0] - mean)) < 1e-14


def test_equal_keys_give_mean_of_values():
    rs = np.random.default_rng(10)
    c = random_case(rs, [29], 2, 1, 64, "f32")
    k_row = rs.standard_normal((1, 64)).astype(np.float32)
    ks = [torch.from_numpy(np.broadcast_to(k_row, (29, 1, 64)).copy())]
    kc = place(c["tables"], [ks[0].numpy()], c["nb"], 1, 16, 64, "f32")
    got = orc.paged_decode(_bits(c["q"]), "f32", kc, c["vc"], "f32", c["bt"], c["ctx"], 0.125)
    mean = c["vs"][0][:, 0, :].double().mean(0).numpy()
    assert np.max(np.abs(got[0] - mean)) < 1e-14


def test_dominant_logit_selects_its_value():
    rs = np.random.default_rng(12)
    c = random_case(rs, [50], 1, 1, 64, "f32")
    j = 33
    kj = c["ks"][0][j, 0].double().numpy()
    q = (200.0 * kj / np.linalg.norm(kj)).astype(np.float32)[None, None, :]
    got = orc.paged_decode(q, "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"], 1.0)
    assert np.max(np.abs(got[0, 0] - c["vs"][0][j, 0].double().numpy())) < 1e-9


def test_empty_context_gives_zeros():
    rs = np.random.default_rng(13)
    c = random_case(rs, [7, 3], 2, 1, 64, "f32")
    got = orc.paged_decode(_bits(c["q"]), "f32", c["kc"], c["vc"], "f32", c["bt"],
                           np.array([0, 3], np.int32), 0.125)
    assert np.all(got[0] == 0.0)


def test_weights_sum_to_one_and_match_library_softmax():
    rs = np.random.default_rng(14)
    c = random_case(rs, [300], 4, 2, 128, "bf16")
    scale = 1 / math.sqrt(128)
    for h in range(4):
        w = orc.softmax_weights(0, h, _bits(c["q"]), "bf16", c["kc"], "bf16", c["bt"], c["ctx"], scale)
        assert abs(w.sum() - 1.0) < 1e-12 and np.all(w >= 0)
        logits = (c["ks"][0][:, h // 2, :].double() @ c["q"][0, h].double()) * scale
        assert np.max(np.abs(w - torch.softmax(logits, 0).numpy())) < 1e-14


def test_physical_permutation_invariance_is_bitwise():
    rs = np.random.default_rng(15)
    c = random_case(rs, [45, 20, 77], 4, 2, 64, "bf16", slack=5)
    base = orc.paged_decode(_bits(c["q"]), "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], 0.125)
    for trial in range(3):
        perm = rs.permutation(c["nb"])        # physical block b moves to perm[b]
        kc = np.empty_like(c["kc"])
        vc = np.empty_like(c["vc"])
        kc[perm] = c["kc"]
        vc[perm] = c["vc"]
        bt = np.where(c["bt"] >= 0, perm[np.maximum(c["bt"], 0)], -1).astype(np.int32)
        got = orc.paged_decode(_bits(c["q"]), "bf16", kc, vc, "bf16", bt, c["ctx"], 0.125)
        assert np.array_equal(got, base)


def test_shared_prefix_equals_private_copy():
    """Two tables pointing at the same prefix blocks give exactly the result
    of tables whose prefix blocks are private copies."""
    rs = np.random.default_rng(16)
    hkv, d, bs = 2, 64, 16
    pre = rs.standard_normal((32, hkv, d)).astype(np.float32)
    tails = [rs.standard_normal((n, hkv, d)).astype(np.float32) for n in (9, 20)]
    vpre = rs.standard_normal((32, hkv, d)).astype(np.float32)
    vtails = [rs.standard_normal((n, hkv, d)).astype(np.float32) for n in (9, 20)]
    kseq = [np.concatenate([pre, t]) for t in tails]
    vseq = [np.concatenate([vpre, t]) for t in vtails]
    shared = [[0, 1, 2], [0, 1, 3, 4]]
    private = [[5, 6, 2], [7, 8, 3, 4]]
    q = rs.standard_normal((2, 4, d)).astype(np.float32)
    ctx = np.array([41, 52], np.int32)
    outs = []
    for tables in (shared, private):
        kc = place(tables, kseq, 9, hkv, bs, d, "f32")
        vc = place(tables, vseq, 9, hkv, bs, d, "f32")
        bt = np.full((2, 4), -1, np.int32)
        for s, t in enumerate(tables):
            bt[s, :len(t)] = t
        outs.append(orc.paged_decode(q, "f32", kc, vc, "f32", bt, ctx, 0.125))
    assert np.array_equal(outs[0], outs[1])


def test_fp8_cache_with_scales_matches_library():
    """E4M3 codes times the per-tensor scales (different for K and V, so a
    swap would show) against torch's own E4M3 decode feeding SDPA."""
    rs = np.random.default_rng(17)
    hq, hkv, d = 16, 2, 128
    ctxs = [30, 64]
    c = random_case(rs, ctxs, hq, hkv, d, "bf16")
    kcodes = [rs.integers(0, 256, (n, hkv, d)).astype(np.uint8) for n in ctxs]
    vcodes = [rs.integers(0, 256, (n, hkv, d)).astype(np.uint8) for n in ctxs]
    for a in kcodes + vcodes:
        a[(a & 0x7F) == 0x7F] = 0x3C  # no NaN codes in live slots
    ksc, vsc = 0.0123, 0.37
    kc = place(c["tables"], kcodes, c["nb"], hkv, 16, d, "fp8")
    vc = place(c["tables"], vcodes, c["nb"], hkv, 16, d, "fp8")
    got = orc.paged_decode(_bits(c["q"]), "bf16", kc, vc, "fp8", c["bt"], c["ctx"],
                           1 / math.sqrt(d), ksc, vsc)
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    ref = sdpa_ref(c["q"], [dec(a) * ksc for a in kcodes], [dec(a) * vsc for a in vcodes],
                   1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_int8_cache_with_scales_matches_library():
    """INT8 codes times the per-tensor scales (different for K and V) against
    torch's dequantisation (int8 -> float64 times scale) feeding SDPA."""
    rs = np.random.default_rng(19)
    hq, hkv, d = 16, 2, 128
    ctxs = [30, 64, 1]
    c = random_case(rs, ctxs, hq, hkv, d, "bf16")
    kcodes = [rs.integers(-127, 128, (n, hkv, d)).astype(np.int8) for n in ctxs]
    vcodes = [rs.integers(-127, 128, (n, hkv, d)).astype(np.int8) for n in ctxs]
    ksc, vsc = 0.0123, 0.037
    kc = place(c["tables"], kcodes, c["nb"], hkv, 16, d, "int8")
    vc = place(c["tables"], vcodes, c["nb"], hkv, 16, d, "int8")
    got = orc.paged_decode(_bits(c["q"]), "bf16", kc, vc, "int8", c["bt"], c["ctx"],
                           1 / math.sqrt(d), ksc, vsc)
    dec = lambda a: torch.from_numpy(a).double()
    ref = sdpa_ref(c["q"], [dec(a) * ksc for a in kcodes], [dec(a) * vsc for a in vcodes],
                   1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12
    # one token: the output is its value row exactly (code * v_scale)
    assert np.array_equal(got[2], (vcodes[2][0].astype(np.float64) * vsc)[
        np.arange(hq) // (hq // hkv)])


def test_block_size_is_a_parameter():
    rs = np.random.default_rng(18)
    c = random_case(rs, [13, 40], 2, 1, 64, "f32", bs=8)
    got = orc.paged_decode(c["q"].numpy(), "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"], 0.125)
    ref = sdpa_ref(c["q"], c["ks"], c["vs"], 0.125)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("part", [16, 48, 512, None])
def test_partition_merge_equals_direct(part):
    rs = np.random.default_rng(19)
    c = random_case(rs, [700], 4, 1, 64, "bf16")
    args = (_bits(c["q"]), "bf16", c["kc"], c["vc"], "bf16", c["bt"], c["ctx"], 0.125)
    direct = orc.paged_decode(*args)
    n = 700
    bounds = list(range(0, n, part)) + [n] if part else [0, 130, 131, 400, n]
    for h in range(4):
        ms, ls, accs = [], [], []
        for t0, t1 in zip(bounds[:-1], bounds[1:]):
            m, l, acc = orc.partition_stats(0, h, t0, t1, *args)
            ms.append(m)
            ls.append(l)
            accs.append(acc)
        merged = orc.lse_merge(ms, ls, np.stack(accs))
        assert np.max(np.abs(merged - direct[0, h])) < 1e-12


def test_partition_stats_single_token_and_empty_merge():
    rs = np.random.default_rng(20)
    c = random_case(rs, [20], 1, 1, 64, "f32")
    args = (c["q"].numpy(), "f32", c["kc"], c["vc"], "f32", c["bt"], c["ctx"], 0.125)
    m, l, acc = orc.partition_stats(0, 0, 7, 8, *args)
    z = 0.125 * float(c["ks"][0][7, 0].double() @ c["q"][0, 0].double())
    assert abs(m - z) < 1e-13 and l == 1.0
    assert np.array_equal(acc, c["vs"][0][7, 0].double().numpy())
    assert np.all(orc.lse_merge([-np.inf], [0.0], np.zeros((1, 64))) == 0.0)
    # an empty partition among live ones changes nothing
    m2, l2, acc2 = orc.partition_stats(0, 0, 0, 20, *args)
    merged = orc.lse_merge([m2, -np.inf], [l2, 0.0], np.stack([acc2, np.zeros(64)]))
    direct = orc.paged_decode(*args)[0, 0]
    assert np.max(np.abs(merged - direct)) < 1e-14
