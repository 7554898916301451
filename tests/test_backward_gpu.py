"""GPU parity of the V1 training forward's saved statistics and of the backward pass, against the
fp64 oracle (oracle.v1_train_stats, oracle.v1_backward, oracle.lambda_backward)."""
import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
import workloads as W
from tolerances import grad_excess

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(f"[case] {msg}", flush=True)


def rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(shape, generator=g)).to(torch.bfloat16).to(DEV)


def f64(x):
    return x.double().cpu().numpy() if isinstance(x, torch.Tensor) else x



def close(got, ref, name):
    e = grad_excess(got, ref)
    note(f"{name}: worst error / bound = {e:.3f}")
    assert e <= 1.0, (name, e)


def case(B, Nq, Nk, H, seed, causal=True, epilogue=True, norm=False, qscale=1.0):
    q1 = rand((B, Nq, H, 64), seed, qscale)
    q2 = rand((B, Nq, H, 64), seed + 1, qscale)
    k1 = rand((B, Nk, H, 64), seed + 2)
    k2 = rand((B, Nk, H, 64), seed + 3)
    v = rand((B, Nk, H, 128), seed + 4)
    dy = rand((B, Nq, H, 128), seed + 5)
    lam = torch.linspace(0.2, 0.9, H)
    w = (0.75 + 0.5 * torch.rand((128,), generator=torch.Generator().manual_seed(seed + 6))) if norm else None
    return dict(q1=q1, q2=q2, k1=k1, k2=k2, v=v, dy=dy, lam=lam, w=w, causal=causal, epilogue=epilogue)


def run(c, li=0.8):
    note(f"bwd case q={tuple(c['q1'].shape)} k={tuple(c['k1'].shape)} causal={c['causal']} epi={c['epilogue']}")
    w = None if c["w"] is None else c["w"].to(DEV)
    out, lse, maps = da.diffattn_fwd_train(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["lam"].to(DEV),
                                           causal=c["causal"], epilogue=c["epilogue"], lambda_init_value=li,
                                           norm_w=w)
    g = da.diffattn_bwd(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["dy"], c["lam"].to(DEV), lse, maps,
                        causal=c["causal"], epilogue=c["epilogue"], lambda_init_value=li, norm_w=w)
    torch.cuda.synchronize()
    ref = oracle.v1_backward(*(f64(c[k]) for k in ("q1", "q2", "k1", "k2", "v")), c["lam"].numpy(), f64(c["dy"]),
                             causal=c["causal"], epilogue=c["epilogue"], lambda_init_value=li,
                             g=None if c["w"] is None else c["w"].numpy())
    return out, lse, maps, g, ref


@pytest.mark.parametrize("N,causal", [(1, True), (31, True), (33, False), (100, True), (257, True), (300, False)])
def test_train_stats(N, causal):
    c = case(2, N, N, 2, 3000 + N, causal=causal)
    out, lse, maps = da.diffattn_fwd_train(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["lam"].to(DEV),
                                           causal=causal, epilogue=True)
    plain = da.diffattn_fwd(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["lam"].to(DEV), causal=causal,
                            epilogue=True)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)                     # training outputs leave the output unchanged
    rl, rm = oracle.v1_train_stats(*(f64(c[k]) for k in ("q1", "q2", "k1", "k2", "v")), causal=causal)
    assert np.max(np.abs(f64(lse) - rl)) <= 2e-3 * max(1.0, np.max(np.abs(rl)))
    assert np.max(np.abs(f64(maps) - rm)) <= 2e-2


@pytest.mark.parametrize("N", [1, 31, 33, 100, 257])
def test_bwd_causal_epilogue(N):
    out, lse, maps, g, ref = run(case(2, N, N, 2, 3100 + N, causal=True, epilogue=True, norm=True))
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        close(g[k], ref[k], k)
    close(g["dlam"], ref["dlam"], "dlam")
    close(g["dnorm_w"], ref["dg"], "dnorm_w")


@pytest.mark.parametrize("B,H,N", [(3, 5, 97), (2, 7, 65)])
def test_bwd_batches_and_heads(B, H, N):
    # several (batch, head) slices, row counts that leave a row pass block part full: the
    # per-block partials of dlambda and dL/dw and their fixed-order sums over batch and heads
    out, lse, maps, g, ref = run(case(B, N, N, H, 3400 + 10 * B + H, causal=True, epilogue=True, norm=True))
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        close(g[k], ref[k], k)
    close(g["dlam"], ref["dlam"], "dlam")
    close(g["dnorm_w"], ref["dg"], "dnorm_w")


@pytest.mark.parametrize("Nq,Nk,causal", [(64, 64, False), (70, 130, True), (40, 200, False), (300, 260, False), (200, 330, True)])
def test_bwd_noepi_and_rect(Nq, Nk, causal):
    out, lse, maps, g, ref = run(case(1, Nq, Nk, 3, 3200 + Nq + Nk, causal=causal, epilogue=False))
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        close(g[k], ref[k], k)
    close(g["dlam"], ref["dlam"], "dlam")
    assert g["dnorm_w"] is None


def test_bwd_large_logits():
    out, lse, maps, g, ref = run(case(1, 160, 160, 2, 3300, causal=True, epilogue=True, qscale=6.0))
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        close(g[k], ref[k], k)


def test_bwd_deterministic():
    c = case(1, 200, 200, 2, 3400)
    _, lse, maps = da.diffattn_fwd_train(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["lam"].to(DEV))
    g1 = da.diffattn_bwd(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["dy"], c["lam"].to(DEV), lse, maps)
    g2 = da.diffattn_bwd(c["q1"], c["q2"], c["k1"], c["k2"], c["v"], c["dy"], c["lam"].to(DEV), lse, maps)
    torch.cuda.synchronize()
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "dlam", "dnorm_w"):
        assert torch.equal(g1[k], g2[k]), k


def test_lambda_bwd():
    rng = np.random.default_rng(60)
    vecs = [rng.normal(0, 0.1, (16, 64)).astype(np.float32) for _ in range(4)]
    dl = rng.standard_normal(16).astype(np.float32)
    got = da.diffattn_lambda_bwd(*(torch.from_numpy(x).to(DEV) for x in vecs), torch.from_numpy(dl).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.lambda_backward(*vecs, dl)
    for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
        assert np.max(np.abs(got[k].cpu().numpy() - ref[k])) <= 1e-5, k


def test_full_v1_prefill_2k_backward_sampled():
    # the 2K configuration's shapes, one batch entry and two heads (the oracle's N^2 rows per head)
    cfg = W.V1_PREFILL_2K
    x = W.v1_inputs(cfg, device=DEV, B=1)
    H = 2
    sl = lambda t: t[:, :, :H].contiguous()
    q1, q2, k1, k2, v = (sl(x[k]) for k in ("q1", "q2", "k1", "k2", "v"))
    dy = rand(tuple(v.shape[:3]) + (128,), 3500)
    lam = torch.tensor([0.5, 0.7], device=DEV)
    li = da.lambda_init(cfg.layer)
    note(f"full-length backward N={cfg.N} H={H}")
    out, lse, maps = da.diffattn_fwd_train(q1, q2, k1, k2, v, lam, causal=True, epilogue=True, lambda_init_value=li)
    g = da.diffattn_bwd(q1, q2, k1, k2, v, dy, lam, lse, maps, causal=True, epilogue=True, lambda_init_value=li)
    torch.cuda.synchronize()
    ref = oracle.v1_backward(*(f64(t) for t in (q1, q2, k1, k2, v)), lam.cpu().numpy(), f64(dy), causal=True,
                             epilogue=True, lambda_init_value=li)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv"):
        close(g[k], ref[k], k)
    close(g["dlam"], ref["dlam"], "dlam")
