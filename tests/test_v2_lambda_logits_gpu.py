"""DIFF V2 with lambda taken in-kernel from its logits (lambda = sigmoid(W_lambda x)), on the GPU:
forward and decode, MFMA and generic kernels, contiguous and paged caches, against the oracle's
logits path (bf16 tolerance 2e-2, fp32 1e-5)."""
import sys

import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def rand(shape, seed, dtype=torch.bfloat16):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(dtype).to(DEV)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


@pytest.mark.parametrize("N,hq,hkv,d,dtype,tol", [
    (300, 16, 4, 128, torch.bfloat16, TOL_BF16),     # MFMA kernel
    (129, 8, 2, 64, torch.bfloat16, TOL_BF16),       # generic kernel (d = 64)
    (40, 4, 2, 16, torch.float32, TOL_F32),          # generic kernel, fp32
])
def test_v2_forward_logits(N, hq, hkv, d, dtype, tol):
    B = 2
    note(f"v2 forward, lambda logits: B={B} N={N} hq={hq} hkv={hkv} d={d} {dtype}")
    q, k, v = rand((B, N, hq, d), 1, dtype), rand((B, N, hkv, d), 2, dtype), rand((B, N, hkv, d), 3, dtype)
    z = W.lambda_logits((B, N, hq // 2), seed=4)
    out = da.diffattn_v2_fwd(q, k, v, z.to(DEV), causal=True, lam_logits=True)
    torch.cuda.synchronize()
    ref = oracle.v2_forward(f64(q), f64(k), f64(v), z.numpy(), causal=True, lam_logits=True)
    assert maxerr(f64(out), ref) <= tol


@pytest.mark.parametrize("hq,hkv,d,dtype,tol", [
    (16, 4, 128, torch.bfloat16, TOL_BF16),          # split-K MFMA kernel
    (8, 2, 64, torch.bfloat16, TOL_BF16),            # generic kernel
    (4, 2, 16, torch.float32, TOL_F32),
])
def test_v2_decode_logits(hq, hkv, d, dtype, tol):
    B, L = 3, 700
    lens = [700, 5, 333]
    note(f"v2 decode, lambda logits: B={B} L={L} hq={hq} hkv={hkv} d={d} {dtype}")
    q, k, v = rand((B, hq, d), 5, dtype), rand((B, L, hkv, d), 6, dtype), rand((B, L, hkv, d), 7, dtype)
    z = W.lambda_logits((B, hq // 2), seed=8)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = da.diffattn_v2_decode(q, k, v, z.to(DEV), cache_lens=lens_t, lam_logits=True)
    torch.cuda.synchronize()
    ref = oracle.v2_decode(f64(q), f64(k), f64(v), z.numpy(), cache_lens=lens, lam_logits=True)
    assert maxerr(f64(out), ref) <= tol
    if d == 128:
        (pk, pv), table = W.scatter_to_pages((k, v), 64, seed=9)
        paged = da.diffattn_v2_decode_paged(q, pk, pv, table, z.to(DEV), cache_lens=lens_t, max_len=L,
                                            lam_logits=True)
        torch.cuda.synchronize()
        assert torch.equal(paged, out)


def test_v2_logits_equal_values_at_closed_form_points():
    # logit ln 3 is lambda 3/4 exactly in real arithmetic; the two modes agree to fp32 rounding
    B, N, hq, hkv = 1, 64, 8, 2
    q, k, v = rand((B, N, hq, 128), 10), rand((B, N, hkv, 128), 11), rand((B, N, hkv, 128), 12)
    z = torch.full((B, N, hq // 2), float(np.log(3.0)), device=DEV)
    a = da.diffattn_v2_fwd(q, k, v, z, causal=True, lam_logits=True)
    b = da.diffattn_v2_fwd(q, k, v, torch.full_like(z, 0.75), causal=True)
    torch.cuda.synchronize()
    assert maxerr(f64(a), f64(b)) <= 1e-2


def test_full_v2_8k_logits():
    # the V2 prefill workload with lambda logits, in the launch configuration the benchmark times
    cfg = W.V2_GQA_8K
    x = W.v2_inputs(cfg, device=DEV)
    z = W.lambda_logits((cfg.B, cfg.N, cfg.hq // 2), seed=cfg.seed + 2000)
    note(f"full {cfg.name}, lambda logits")
    out = da.diffattn_v2_fwd(x["q"], x["k"], x["v"], z.to(DEV), causal=True, lam_logits=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    rows = np.array([(int(b), int(p), int(i)) for b, p, i in zip(rng.integers(0, cfg.B, 24),
                                                                 rng.integers(0, cfg.hq // 2, 24),
                                                                 rng.integers(0, cfg.N, 24))]
                    + [(0, 0, 0), (cfg.B - 1, cfg.hq // 2 - 1, cfg.N - 1)])
    ref = oracle.v2_forward(*(x[k].float().cpu().numpy() for k in ("q", "k", "v")), z.numpy(), causal=True,
                            rows=rows, lam_logits=True)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert maxerr(got, ref) <= TOL_BF16
