"""Pins for the oracle's cache-append: only the addressed rows change, they
hold the new token's K/V ("Transformer 推理优化：KV Cache、PagedAttention 与
vLLM", section 2.2: each step computes and stores only the new token's K and
V), and E4M3 caches hold torch's own E4M3 cast of x * (1/scale)."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

CANARY = {"f32": np.float32(-12345.5), "f16": np.uint16(0xABCD), "bf16": np.uint16(0xC0DE),
          "fp8": np.uint8(0x5A)}


def _rand_bits(rs, shape, dtype):
    x = rs.standard_normal(shape).astype(np.float32)
    if dtype == "f32":
        return x
    t = torch.from_numpy(x).to({"f16": torch.float16, "bf16": torch.bfloat16}[dtype])
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_append_writes_exactly_the_addressed_rows(dtype):
    rs = np.random.default_rng(30)
    nb, hkv, bs, d = 6, 3, 16, 64
    kc = np.full((nb, hkv, bs, d), CANARY[dtype], dtype=orc.BITS_NP[dtype])
    vc = kc.copy()
    slots = np.array([37, -1, 0, 95, 16], np.int64)  # 37 = block 2 slot 5; 95 = block 5 slot 15
    kn = _rand_bits(rs, (5, hkv, d), dtype)
    vn = _rand_bits(rs, (5, hkv, d), dtype)
    orc.cache_append(kc, vc, kn, vn, slots, dtype, dtype)
    expect_k = np.full_like(kc, CANARY[dtype])
    expect_v = np.full_like(vc, CANARY[dtype])
    for t, where in enumerate([(2, 5), None, (0, 0), (5, 15), (1, 0)]):
        if where is None:
            continue
        blk, off = where
        expect_k[blk, :, off, :] = kn[t]
        expect_v[blk, :, off, :] = vn[t]
    assert np.array_equal(kc.view(np.uint8), expect_k.view(np.uint8))
    assert np.array_equal(vc.view(np.uint8), expect_v.view(np.uint8))


def test_append_rejects_out_of_range_slot():
    kc = np.zeros((2, 1, 16, 64), np.float32)
    with pytest.raises(ValueError):
        orc.cache_append(kc, kc.copy(), np.zeros((1, 1, 64), np.float32),
                         np.zeros((1, 1, 64), np.float32), np.array([32]), "f32", "f32")


@pytest.mark.parametrize("new_dtype", ["bf16", "f16", "f32"])
def test_fp8_append_matches_torch_cast(new_dtype):
    rs = np.random.default_rng(31)
    nb, hkv, bs, d = 4, 2, 16, 128
    kc = np.full((nb, hkv, bs, d), CANARY["fp8"], np.uint8)
    vc = kc.copy()
    T = 20
    kn = _rand_bits(rs, (T, hkv, d), new_dtype)
    vn = _rand_bits(rs, (T, hkv, d), new_dtype)
    slots = rs.permutation(nb * bs)[:T].astype(np.int64)
    k_scale, v_scale = float(np.float32(0.0091)), float(np.float32(3.7))
    orc.cache_append(kc, vc, kn, vn, slots, new_dtype, "fp8", k_scale, v_scale)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[new_dtype]
    for new, cache, sc in ((kn, kc, k_scale), (vn, vc, v_scale)):
        x = torch.from_numpy(new.view(np.int16) if new_dtype != "f32" else new)
        x = x.view(tdt).float() if new_dtype != "f32" else x
        inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(sc, dtype=torch.float32)
        y = (x * inv).float()
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        ref = np.where(np.abs(y.numpy()) >= 464.0, np.where(y.numpy() < 0, 0xFE, 0x7E), ref)
        for t, sl in enumerate(slots):
            assert np.array_equal(cache[sl // bs, :, sl % bs, :], ref[t])
    written = np.zeros((nb, bs), bool)
    written[slots // bs, slots % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~written] == CANARY["fp8"])


@pytest.mark.parametrize("new_dtype", ["bf16", "f16", "f32"])
def test_int8_append_is_numpy_rint_of_the_scaled_value(new_dtype):
    rs = np.random.default_rng(32)
    nb, hkv, bs, d = 4, 2, 16, 64
    kc = np.full((nb, hkv, bs, d), 99, np.int8)
    vc = kc.copy()
    T = 20
    kn = _rand_bits(rs, (T, hkv, d), new_dtype)
    vn = _rand_bits(rs, (T, hkv, d), new_dtype)
    slots = rs.permutation(nb * bs)[:T].astype(np.int64)
    k_scale, v_scale = float(np.float32(0.021)), float(np.float32(0.5))
    orc.cache_append(kc, vc, kn, vn, slots, new_dtype, "int8", k_scale, v_scale)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[new_dtype]
    for new, cache, sc in ((kn, kc, k_scale), (vn, vc, v_scale)):
        x = torch.from_numpy(new.view(np.int16) if new_dtype != "f32" else new)
        x = x.view(tdt).float() if new_dtype != "f32" else x
        inv = np.float32(1.0) / np.float32(sc)
        y = x.numpy().astype(np.float32) * inv
        ref = np.clip(np.rint(y), -127, 127).astype(np.int8)
        if sc == k_scale:
            assert np.any(np.abs(y) > 127)      # K: 1/0.021 ~ 47.6 saturates the tails
        for t, sl in enumerate(slots):
            assert np.array_equal(cache[sl // bs, :, sl % bs, :], ref[t])
    written = np.zeros((nb, bs), bool)
    written[slots // bs, slots % bs] = True
    assert np.all(kc.transpose(0, 2, 1, 3)[~written] == 99)
