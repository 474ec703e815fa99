"""Swapping blocks to pinned host memory and back ("大语言模型推理引擎深度剖析",
section 3.3): the bookkeeping of pkv_seq_swap and the copies of
pkv_swap_blocks.  Block copies are byte copies, so everything here is
checked bit for bit: the host blocks equal the device blocks they came from,
and a decode after swapping out, clobbering the freed device blocks and
swapping back into other blocks equals the decode before (the result does
not depend on where the blocks sit)."""
import numpy as np
import pytest
import torch

from gpu_harness import gpu_setup
from synth import CONFIGS

pytestmark = pytest.mark.gpu


def _bytes(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("name", ["c2_qwen3_8b_bf16", "c4_llama3_70b_fp8", "c5_long_shared_bf16"])
def test_swap_out_clobber_swap_in_is_exact(name):
    import paged_kv_cache_363_amd as pkv
    print(f"[case] swap {name}", flush=True)
    cfg = CONFIGS[name]
    st = gpu_setup(cfg)
    pool, tables = st["pool"], st["state"]["tables"]
    ws = pkv.alloc_workspace(st["q"], st["k_cache"], st["block_tables"], cfg.partition_size)

    def decode():
        out = pkv.paged_decode_attention(st["q"], st["k_cache"], st["v_cache"],
                                         st["block_tables"], st["context_lens"], cfg.scale,
                                         st["k_scale"], st["v_scale"],
                                         partition_size=cfg.partition_size, workspace=ws)
        torch.cuda.synchronize()
        return out

    before = decode()
    moved = list(range(0, cfg.num_seqs, 2))[:8]
    n_host = sum(len(tables[s]) for s in moved)
    host = pkv.BlockPool(n_host, 16)
    shape = (n_host,) + tuple(st["k_cache"].shape[1:])
    hk = torch.empty(shape, dtype=st["k_cache"].dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=st["k_cache"].dtype, pin_memory=True)
    host_tables, out_pairs = {}, []
    for s in moved:
        host_tables[s], pairs = pool.seq_swap(host, tables[s])
        out_pairs += pairs
    p_out = torch.tensor(out_pairs, dtype=torch.int32, device="cuda")
    pkv.swap_blocks(hk, hv, st["k_cache"], st["v_cache"], p_out)
    torch.cuda.synchronize()
    src = torch.tensor([a for a, _ in out_pairs], device="cuda")
    dst = torch.tensor([b for _, b in out_pairs])
    assert torch.equal(_bytes(hk[dst]), _bytes(st["k_cache"][src].cpu()))
    assert torch.equal(_bytes(hv[dst]), _bytes(st["v_cache"][src].cpu()))

    # the released device blocks are reused by someone else: clobber them
    freed = sorted(set(a for a, _ in out_pairs) & set(pool.free_list()))
    if freed:
        idx = torch.tensor(freed, device="cuda")
        st["k_cache"][idx] = st["k_cache"][idx].view(torch.uint8).fill_(0x7F).view(
            st["k_cache"].dtype)
        st["v_cache"][idx] = st["v_cache"][idx].view(torch.uint8).fill_(0x7F).view(
            st["v_cache"].dtype)
    # take some free device blocks first so the way back lands elsewhere
    pool.seq_create(16 * min(4, pool.num_free()))
    in_pairs = []
    bt = st["block_tables"].cpu().numpy()
    for s in moved:
        tables[s], pairs = host.seq_swap(pool, host_tables[s])
        in_pairs += pairs
        bt[s, :len(tables[s])] = tables[s]
    p_in = torch.tensor(in_pairs, dtype=torch.int32, device="cuda")
    pkv.swap_blocks(st["k_cache"], st["v_cache"], hk, hv, p_in)
    st["block_tables"].copy_(torch.from_numpy(bt))
    torch.cuda.synchronize()
    assert host.num_free() == n_host
    after = decode()
    assert torch.equal(_bytes(after), _bytes(before))


def test_swap_skips_pairs_outside_either_pool():
    import paged_kv_cache_363_amd as pkv
    a = torch.arange(4 * 2 * 16 * 64, dtype=torch.float32, device="cuda").view(4, 2, 16, 64)
    b = torch.full((3, 2, 16, 64), -1.0, pin_memory=True)
    c = torch.full((3, 2, 16, 64), -1.0, pin_memory=True)
    pairs = torch.tensor([[0, 2], [3, 3], [4, 0], [-1, 1], [1, 0]], dtype=torch.int32,
                         device="cuda")
    pkv.swap_blocks(b, c, a, a, pairs)
    torch.cuda.synchronize()
    assert torch.equal(b[2], a[0].cpu()) and torch.equal(b[0], a[1].cpu())
    assert torch.all(b[1] == -1.0) and torch.equal(c[2], a[0].cpu())


def test_pageable_host_memory_is_refused_before_launch():
    from paged_kv_cache_363_amd import _lib
    a = torch.zeros((2, 2, 16, 64), device="cuda")
    host = np.zeros((2, 2, 16, 64), np.float32)        # pageable: no kernel may touch it
    pairs = torch.tensor([[0, 0]], dtype=torch.int32, device="cuda")
    st = _lib.lib().pkv_swap_blocks(host.ctypes.data, host.ctypes.data, 2, a.data_ptr(),
                                    a.data_ptr(), 2, pairs.data_ptr(), 1, 2 * 16 * 64 * 4, None)
    assert st == _lib.PKV_ERR_INVALID_ARG
    assert b"pinned" in _lib.lib().pkv_last_error()
