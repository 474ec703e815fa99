"""Logits that climb block after block, by steps below and above the online
softmax's rebasing threshold (8 in base-2 units), with falls in between: the
matrix-core kernels keep their reference maximum through small rises and
move it on large ones, and every schedule must still give the oracle's
attention.  The multi-query kernels take the same caches with 16 query rows
per sequence (four column tiles), whose columns cross the threshold on
different blocks.  Inputs are built on the host (seeded), written straight
into the caches in their [block][kv-head][16][d] layout; the oracle reads the
same bits."""
import numpy as np
import pytest
import torch

from harness import allclose_report
from oracle import oracle as orc
from synth import gen

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16}
HKV, G, D, S = 2, 4, 128, 3


def levels(nblk, rs):
    """Per-block logit level (base-2 units, roughly): rises of 0.5-7.5 and of
    9-20 in random order, and falls of up to 15."""
    lv, x = [], 0.0
    for _ in range(nblk):
        r = rs.random()
        if r < 0.5:
            x += rs.uniform(0.5, 7.5)
        elif r < 0.8:
            x += rs.uniform(9.0, 20.0)
        else:
            x -= rs.uniform(0.0, 15.0)
        lv.append(x)
    return np.array(lv)


def build(dt, seed):
    rs = np.random.default_rng(seed)
    ctx = np.array([16 * 37 + 5, 16 * 64, 16 * 9 + 1], np.int32)
    nblk = (ctx + 15) // 16
    mb = int(nblk.max())
    nb = int(nblk.sum()) + 7
    ids = rs.permutation(nb).astype(np.int32)
    bt = np.full((S, mb), -1, np.int32)
    k = np.full((nb, HKV, 16, D), np.nan, np.float32)
    v = np.full((nb, HKV, 16, D), np.nan, np.float32)
    q = np.empty((S, HKV * G, D), np.float32)
    scale = 1.0 / np.sqrt(D)
    used = 0
    for s in range(S):
        bt[s, :nblk[s]] = ids[used:used + nblk[s]]
        used += nblk[s]
        for h in range(HKV):
            u = rs.standard_normal(D)
            u /= np.linalg.norm(u)
            for j in range(G):
                q[s, h * G + j] = 8.0 * u + 0.1 * rs.standard_normal(D)
            # logit ~ scale * 8 * a per token, in base-2 units ~ 1.02 a
            a = np.repeat(levels(nblk[s], rs), 16)[:ctx[s]] + rs.uniform(-0.5, 0.5, ctx[s])
            kt = a[:, None] * u[None, :] + 0.05 * rs.standard_normal((ctx[s], D))
            vt = rs.standard_normal((ctx[s], D))
            for t in range(ctx[s]):
                k[bt[s, t // 16], h, t % 16] = kt[t]
                v[bt[s, t // 16], h, t % 16] = vt[t]
    kc = torch.from_numpy(k).to(TORCH[dt])
    vc = torch.from_numpy(v).to(TORCH[dt])
    qt = torch.from_numpy(q).to(TORCH[dt])
    ref = orc.paged_decode(gen.bits(qt), dt, gen.bits(kc), gen.bits(vc), dt, bt, ctx, scale)
    return dict(k=kc, v=vc, q=qt, bt=bt, ctx=ctx, scale=scale, mb=mb, ref=ref)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ps", [0, 128, 1024])
def test_rising_logits_match_oracle(dt, ps):
    import paged_kv_cache_363_amd as pkv
    print(f"[case] rebase {dt} partition={ps}", flush=True)
    b = build(dt, 4242 + ps)
    dev = "cuda"
    out = pkv.paged_decode_attention(b["q"].to(dev), b["k"].to(dev), b["v"].to(dev),
                                     torch.from_numpy(b["bt"]).to(dev),
                                     torch.from_numpy(b["ctx"]).to(dev), b["scale"],
                                     partition_size=ps, algo="mfma")
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ok, excess, err = allclose_report(got, b["ref"], 2e-3, 1e-2)
    assert ok, f"max|err| {err}, worst excess {excess}"


NROWS = 16   # query rows per sequence: four column tiles of 4 rows x 4 heads


def build_mq(dt, seed):
    """The caches of build() with NROWS query rows per sequence, the last
    positions of its context.  Row i's q is the sequence's direction scaled
    by 1 + 0.15 i, so its logits follow the same levels with steeper rises
    and the columns of one wave cross the rebasing threshold on different
    blocks (some keep their reference while others move)."""
    b = build(dt, seed)
    rs = np.random.default_rng(seed + 1)
    q1 = b["q"].float().numpy()            # [S][H_q][D], 8 u per kv-head + noise
    q = np.empty((S * NROWS, HKV * G, D), np.float32)
    for s in range(S):
        for i in range(NROWS):
            q[s * NROWS + i] = q1[s] * (1.0 + 0.15 * i) + 0.05 * rs.standard_normal((HKV * G, D))
    qt = torch.from_numpy(q).to(TORCH[dt])
    qs = (np.arange(S + 1) * NROWS).astype(np.int32)
    ref = orc.paged_multiquery(gen.bits(qt), dt, gen.bits(b["k"]), gen.bits(b["v"]), dt, b["bt"],
                               b["ctx"], qs, b["scale"])
    return dict(b, q=qt, qs=qs, ref=ref)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ps", [0, 128, 16 * 64])
def test_rising_logits_multiquery_match_oracle(dt, ps):
    import paged_kv_cache_363_amd as pkv
    print(f"[case] rebase multiquery {dt} partition={ps}", flush=True)
    b = build_mq(dt, 5151 + ps)
    dev = "cuda"
    out = pkv.paged_multiquery_attention(b["q"].to(dev), b["k"].to(dev), b["v"].to(dev),
                                         torch.from_numpy(b["bt"]).to(dev),
                                         torch.from_numpy(b["ctx"]).to(dev),
                                         torch.from_numpy(b["qs"]).to(dev), NROWS, b["scale"],
                                         partition_size=ps)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ok, excess, err = allclose_report(got, b["ref"], 2e-3, 1e-2)
    assert ok, f"max|err| {err}, worst excess {excess}"
