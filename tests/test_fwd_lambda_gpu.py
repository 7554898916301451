"""The V1 forward with lambda computed from its re-parameterisation in the same kernel: it must
give exactly what diffattn_lambda followed by diffattn_fwd gives (same lambda arithmetic), and
match the oracle (bf16 tolerance 2e-2, fp32 1e-5)."""
import sys

import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def rand(shape, seed, dtype, scale=1.0):
    return (torch.randn(shape, generator=torch.Generator().manual_seed(seed)) * scale).to(dtype).to(DEV)


@pytest.mark.parametrize("N,H,d,dv,dtype,tol,lam_dim", [
    (300, 3, 64, 128, torch.bfloat16, 2e-2, 64),     # MFMA kernel, lambda in the kernel
    (129, 2, 64, 128, torch.bfloat16, 2e-2, 200),    # lam_dim past one wave's lanes
    (77, 2, 32, 48, torch.bfloat16, 2e-2, 32),       # generic kernel after the lambda kernel
    (40, 2, 8, 16, torch.float32, 1e-5, 8),
    (4100, 1, 64, 128, torch.bfloat16, 2e-2, 64),    # 4096 keys and more: the max-ilp build of the kernels
])
def test_fused_lambda_equals_separate_calls(N, H, d, dv, dtype, tol, lam_dim):
    B, layer = 2, 5
    note(f"fused lambda forward N={N} H={H} d={d} dv={dv} {dtype} lam_dim={lam_dim}")
    q1, q2, k1, k2 = (rand((B, N, H, d), 10 + i, dtype) for i in range(4))
    v = rand((B, N, H, dv), 14, dtype)
    vecs = [rand((H, lam_dim), 20 + i, torch.float32, 0.1) for i in range(4)]
    out, lam = da.diffattn_fwd_lambda(q1, q2, k1, k2, v, *vecs, layer, causal=True, epilogue=True)
    lam_sep = da.diffattn_lambda(*vecs, layer)
    sep = da.diffattn_fwd(q1, q2, k1, k2, v, lam_sep, causal=True, epilogue=True,
                          lambda_init_value=da.lambda_init(layer))
    torch.cuda.synchronize()
    assert torch.equal(lam, lam_sep)
    assert torch.equal(out, sep)
    ref_lam = oracle.lam(*(f64(x) for x in vecs), layer)
    ref = oracle.v1_forward(*(f64(x) for x in (q1, q2, k1, k2, v)), ref_lam, causal=True, epilogue=True,
                            lambda_init_value=oracle.lambda_init(layer))
    assert np.max(np.abs(f64(out) - ref)) <= tol
    assert np.max(np.abs(f64(lam) - ref_lam)) <= 1e-5


def test_full_fused_lambda_2k():
    # the V1 prefill workload: the single-kernel step gives the two-call step's output bit for bit
    cfg = W.V1_PREFILL_2K
    x = W.v1_inputs(cfg, device=DEV)
    vecs = [x[k].to(DEV) for k in ("lq1", "lk1", "lq2", "lk2")]
    note(f"full fused lambda: {cfg.name}")
    out, lam = da.diffattn_fwd_lambda(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], *vecs, cfg.layer, causal=True,
                                      epilogue=True)
    lam_sep = da.diffattn_lambda(*vecs, cfg.layer)
    sep = da.diffattn_fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam_sep, causal=True, epilogue=True,
                          lambda_init_value=da.lambda_init(cfg.layer))
    torch.cuda.synchronize()
    assert torch.equal(lam, lam_sep)
    assert torch.equal(out, sep)
