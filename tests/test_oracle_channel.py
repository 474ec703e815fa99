"""Pins for the oracle's per-channel scales ("大语言模型推理引擎深度剖析", section
4.3: each head dimension of K and V quantised on its own): attention against
torch's dequantisation (code * scale[kv_head][dim]) feeding SDPA, the
reduction to the pinned per-tensor oracle when every channel has the same
scale, and the append's codes against numpy / torch per channel.  Scales
differ per channel, per kv-head and between K and V, so a transposed or
swapped index would show."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from test_oracle_attention import _bits, place, random_case, sdpa_ref


def _codes(rs, kv, shape):
    if kv == "int8":
        return rs.integers(-127, 128, shape).astype(np.int8)
    a = rs.integers(0, 256, shape).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x3C
    return a


def _dequant(kv, a, sc):
    x = torch.from_numpy(a).double() if kv == "int8" else \
        torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    return x * torch.from_numpy(sc)[None]          # [n][H_kv][d] * [H_kv][d]


@pytest.mark.parametrize("kv", ["fp8", "int8"])
def test_channel_decode_matches_library(kv):
    rs = np.random.default_rng(41)
    hq, hkv, d = 16, 2, 64
    ctxs = [30, 64, 1, 17]
    c = random_case(rs, ctxs, hq, hkv, d, "bf16")
    kcodes = [_codes(rs, kv, (n, hkv, d)) for n in ctxs]
    vcodes = [_codes(rs, kv, (n, hkv, d)) for n in ctxs]
    ks = rs.uniform(0.001, 0.05, (hkv, d))
    vs = rs.uniform(0.01, 0.5, (hkv, d))
    kc = place(c["tables"], kcodes, c["nb"], hkv, 16, d, kv)
    vc = place(c["tables"], vcodes, c["nb"], hkv, 16, d, kv)
    got = orc.paged_decode_channel(_bits(c["q"]), "bf16", kc, vc, kv, c["bt"], c["ctx"],
                                   1 / math.sqrt(d), ks, vs)
    ref = sdpa_ref(c["q"], [_dequant(kv, a, ks) for a in kcodes],
                   [_dequant(kv, a, vs) for a in vcodes], 1 / math.sqrt(d))
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("kv", ["fp8", "int8"])
def test_equal_channel_scales_are_the_per_tensor_oracle(kv):
    rs = np.random.default_rng(42)
    hq, hkv, d = 8, 2, 64
    ctxs = [20, 45]
    c = random_case(rs, ctxs, hq, hkv, d, "bf16")
    kc = place(c["tables"], [_codes(rs, kv, (n, hkv, d)) for n in ctxs], c["nb"], hkv, 16, d, kv)
    vc = place(c["tables"], [_codes(rs, kv, (n, hkv, d)) for n in ctxs], c["nb"], hkv, 16, d, kv)
    qb = _bits(c["q"])
    got = orc.paged_decode_channel(qb, "bf16", kc, vc, kv, c["bt"], c["ctx"], 0.125,
                                   np.full((hkv, d), 0.03), np.full((hkv, d), 0.2))
    ref = orc.paged_decode(qb, "bf16", kc, vc, kv, c["bt"], c["ctx"], 0.125, 0.03, 0.2)
    assert np.max(np.abs(got - ref)) < 1e-13


@pytest.mark.parametrize("kv", ["fp8", "int8"])
def test_channel_append_codes(kv):
    rs = np.random.default_rng(43)
    nb, hkv, bs, d = 3, 2, 16, 64
    dt = np.int8 if kv == "int8" else np.uint8
    kc = np.full((nb, hkv, bs, d), 5, dt)
    vc = kc.copy()
    T = 10
    x = (rs.standard_normal((T, hkv, d)) * 3).astype(np.float32)
    y = (rs.standard_normal((T, hkv, d)) * 3).astype(np.float32)
    ks = rs.uniform(0.005, 0.05, (hkv, d)).astype(np.float32)
    vs = rs.uniform(0.01, 0.1, (hkv, d)).astype(np.float32)
    slots = rs.permutation(nb * bs)[:T].astype(np.int64)
    orc.cache_append_channel(kc, vc, x, y, slots, "f32", kv, ks, vs)
    for new, cache, sc in ((x, kc, ks), (y, vc, vs)):
        inv = (np.float32(1.0) / sc).astype(np.float32)
        p = (new * inv[None]).astype(np.float32)
        if kv == "int8":
            ref = np.clip(np.rint(p), -127, 127).astype(np.int8)
        else:
            ref = torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            ref = np.where(np.abs(p) >= 464.0, np.where(p < 0, 0xFE, 0x7E), ref).astype(np.uint8)
        for t, sl in enumerate(slots):
            assert np.array_equal(cache[sl // bs, :, sl % bs, :], ref[t])
