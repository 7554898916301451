"""Decode against a paged KV cache (block table over a shared page pool), on the GPU.

Each case scatters seeded contiguous caches into a pool in a random page order, runs the paged
entry point, and checks it against the oracle's decode of the cache read back through the table
(bf16 tolerance 2e-2), and bit for bit against the contiguous entry point on the original caches
(the same kernels with the same split-K slices see the same rows in the same order).
"""
import sys

import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).to(DEV)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


@pytest.mark.parametrize("page", [32, 64, 256])
def test_v1_paged_decode(page):
    B, L, H = 3, 1000, 4
    lens = [1000, 1, 517]
    note(f"v1 paged decode B={B} L={L} H={H} page={page} lens={lens}")
    q1, q2 = rand((B, H, 64), 10 + page), rand((B, H, 64), 11 + page)
    k1, k2, v = rand((B, L, H, 64), 12 + page), rand((B, L, H, 64), 13 + page), rand((B, L, H, 128), 14 + page)
    lam = torch.linspace(0.2, 0.8, H)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    (pk1, pk2, pv), table = W.scatter_to_pages((k1, k2, v), page, seed=page)
    out = da.diffattn_decode_paged(q1, q2, pk1, pk2, pv, table, lam.to(DEV), cache_lens=lens_t, max_len=L)
    contig = da.diffattn_decode(q1, q2, k1, k2, v, lam.to(DEV), cache_lens=lens_t)
    torch.cuda.synchronize()
    assert torch.equal(out, contig)
    t = table.cpu().numpy()
    ref = oracle.decode(f64(q1), f64(q2), oracle.gather_pages(f64(pk1), t, L, page),
                        oracle.gather_pages(f64(pk2), t, L, page), oracle.gather_pages(f64(pv), t, L, page),
                        lam.numpy(), cache_lens=lens)
    assert maxerr(f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("page,hq,hkv", [(32, 16, 4), (128, 16, 4), (64, 64, 8), (64, 32, 2), (32, 48, 2)])
def test_v2_paged_decode(page, hq, hkv):
    B, L = 3, 1500
    lens = [1500, 33, 640]
    note(f"v2 paged decode B={B} L={L} hq={hq} hkv={hkv} page={page} lens={lens}")
    q = rand((B, hq, 128), 20 + page + hq)
    k, v = rand((B, L, hkv, 128), 21 + page + hq), rand((B, L, hkv, 128), 22 + page + hq)
    lam = torch.rand((B, hq // 2), generator=torch.Generator().manual_seed(23 + page))
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    (pk, pv), table = W.scatter_to_pages((k, v), page, seed=page + hq)
    out = da.diffattn_v2_decode_paged(q, pk, pv, table, lam.to(DEV), cache_lens=lens_t, max_len=L)
    contig = da.diffattn_v2_decode(q, k, v, lam.to(DEV), cache_lens=lens_t)
    torch.cuda.synchronize()
    assert torch.equal(out, contig)
    t = table.cpu().numpy()
    ref = oracle.v2_decode(f64(q), oracle.gather_pages(f64(pk), t, L, page), oracle.gather_pages(f64(pv), t, L, page),
                           lam.numpy(), cache_lens=lens)
    assert maxerr(f64(out), ref) <= TOL_BF16


def test_paged_table_with_padding_and_no_lens():
    # a block table wider than needed (its extra entries hold garbage) and cache_lens = NULL
    B, L, H, page = 2, 256, 2, 64
    note(f"v1 paged decode, wide table, no lengths B={B} L={L} page={page}")
    q1, q2 = rand((B, H, 64), 30), rand((B, H, 64), 31)
    k1, k2, v = rand((B, L, H, 64), 32), rand((B, L, H, 64), 33), rand((B, L, H, 128), 34)
    lam = torch.tensor([0.3, 0.6])
    (pk1, pk2, pv), table = W.scatter_to_pages((k1, k2, v), page, seed=35)
    wide = torch.full((B, table.shape[1] + 5), 123456, dtype=torch.int32, device=DEV)
    wide[:, :table.shape[1]] = table
    out = da.diffattn_decode_paged(q1, q2, pk1, pk2, pv, wide, lam.to(DEV), max_len=L)
    contig = da.diffattn_decode(q1, q2, k1, k2, v, lam.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, contig)


def test_full_v2_paged_decode_64k():
    # the V2 decode workload (B=32, 64K cache, 64q/8kv heads, d=128) in 256-token pages, in the
    # launch configuration the benchmark times: equal to the contiguous path bit for bit, and
    # sampled pairs against the oracle
    c = W.V2_DECODE_64K
    note(f"full v2 paged decode: {c.name}, page 256")
    x = W.v2_decode_inputs(c, device=DEV)
    (pk, pv), table = W.scatter_to_pages((x["k"], x["v"]), 256, seed=77)
    lam = x["lam"].to(DEV)
    out = da.diffattn_v2_decode_paged(x["q"], pk, pv, table, lam, max_len=c.L)
    contig = da.diffattn_v2_decode(x["q"], x["k"], x["v"], lam)
    torch.cuda.synchronize()
    assert torch.equal(out, contig)
    rng = np.random.default_rng(78)
    h, group = c.hq // 2, c.hq // c.hkv
    got = out.float().cpu().numpy()
    for b, p in zip(rng.integers(0, c.B, 6), rng.integers(0, h, 6)):
        b, p = int(b), int(p)
        g = (2 * p) // group
        # the pair's KV head only: query heads 2p, 2p+1 of one group read KV head g
        ref = oracle.v2_decode(f64(x["q"][b:b + 1, 2 * p:2 * p + 2]), f64(x["k"][b:b + 1, :, g:g + 1]),
                               f64(x["v"][b:b + 1, :, g:g + 1]), lam[b:b + 1, p:p + 1].cpu().numpy())
        assert maxerr(got[b, p], ref[0, 0]) <= TOL_BF16, (b, p)
    del x, pk, pv
    torch.cuda.empty_cache()
