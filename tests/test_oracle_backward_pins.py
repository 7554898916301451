"""Pins for the oracle's gradients: central finite differences of the (pinned) forward oracle, and
the special case lambda = 0, no norm, which is ordinary attention's gradient from torch autograd.

The backward formulas are the chain rule through the definition of differential attention
("Differential Transformer: Noise-Canceling Attention by Subtraction", sections "The mechanism"
and "Making lambda learnable and stable"); these tests check them against derivatives taken
numerically, so a dropped term, a sign or a transposed operand shows up.
"""
import numpy as np
import pytest
import torch

import oracle


def _loss(x, dy, lam, causal, epilogue, li, g, scale=None):
    y = oracle.v1_forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, causal=causal,
                          epilogue=epilogue, lambda_init_value=li, g=g, scale=scale)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("causal,epilogue,nq,nk", [(True, True, 5, 5), (False, True, 4, 6),
                                                   (True, False, 4, 7), (False, False, 5, 5)])
def test_backward_matches_finite_differences(causal, epilogue, nq, nk):
    rng = np.random.default_rng(20 + nq + nk + 2 * causal + epilogue)
    B, H, d, dv = 1, 2, 3, 4
    x = {k: rng.standard_normal((B, nq, H, d)) for k in ("q1", "q2")}
    x.update({k: rng.standard_normal((B, nk, H, d)) for k in ("k1", "k2")})
    x["v"] = rng.standard_normal((B, nk, H, dv))
    lam = np.array([0.35, 0.8])
    g = rng.uniform(0.5, 1.5, dv) if epilogue else None
    li = 0.6
    dy = rng.standard_normal((B, nq, H, dv))
    got = oracle.v1_backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, dy, causal=causal,
                             epilogue=epilogue, lambda_init_value=li, g=g)
    h = 1e-6
    for name in ("q1", "q2", "k1", "k2", "v"):
        num = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {k: a.copy() for k, a in x.items()}
            xm = {k: a.copy() for k, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (_loss(xp, dy, lam, causal, epilogue, li, g) -
                        _loss(xm, dy, lam, causal, epilogue, li, g)) / (2 * h)
        assert np.allclose(got["d" + name], num, atol=2e-7, rtol=0), name
    for hd in range(H):
        lp, lm = lam.copy(), lam.copy()
        lp[hd] += h
        lm[hd] -= h
        num = (_loss(x, dy, lp, causal, epilogue, li, g) - _loss(x, dy, lm, causal, epilogue, li, g)) / (2 * h)
        assert got["dlam"][hd] == pytest.approx(num, abs=2e-7)
    if epilogue:
        for c in range(dv):
            gp, gm = g.copy(), g.copy()
            gp[c] += h
            gm[c] -= h
            num = (_loss(x, dy, lam, causal, epilogue, li, gp) - _loss(x, dy, lam, causal, epilogue, li, gm)) / (2 * h)
            assert got["dg"][c] == pytest.approx(num, abs=2e-7)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_lambda_zero_is_attention_gradient(causal):
    # lambda = 0 and no norm: map 1 is ordinary attention, whose gradients torch autograd gives;
    # map 2 then gets no gradient, and dlambda = -sum dy . (A2 V)
    rng = np.random.default_rng(30 + causal)
    B, N, H, d, dv = 2, 9, 2, 5, 6
    q1, q2, k1, k2 = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    v = rng.standard_normal((B, N, H, dv))
    dy = rng.standard_normal((B, N, H, dv))
    got = oracle.v1_backward(q1, q2, k1, k2, v, np.zeros(H), dy, causal=causal, epilogue=False)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tq, tk, tv = t(q1), t(k1), t(v)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    o.backward(torch.from_numpy(dy).permute(0, 2, 1, 3))
    back = lambda a: a.grad.permute(0, 2, 1, 3).numpy()
    assert np.allclose(got["dq1"], back(tq), atol=1e-12, rtol=0)
    assert np.allclose(got["dk1"], back(tk), atol=1e-12, rtol=0)
    assert np.allclose(got["dv"], back(tv), atol=1e-12, rtol=0)
    assert np.all(got["dq2"] == 0) and np.all(got["dk2"] == 0)
    with torch.no_grad():
        o2 = torch.nn.functional.scaled_dot_product_attention(t(q2), t(k2), t(v), is_causal=causal)
    ref = -np.einsum("bhnc,bhnc->h", torch.from_numpy(dy).permute(0, 2, 1, 3).numpy(), o2.numpy())
    assert np.allclose(got["dlam"], ref, atol=1e-12, rtol=0)


def test_backward_cancelling_maps_give_no_value_gradient():
    # identical maps with lambda = 1: o = 0 whatever V is, so dV = 0 exactly
    rng = np.random.default_rng(40)
    B, N, H, d, dv = 1, 8, 1, 4, 4
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, dv))
    dy = rng.standard_normal((B, N, H, dv))
    got = oracle.v1_backward(q, q, k, k, v, [1.0], dy, causal=True, epilogue=False)
    assert np.all(got["dv"] == 0.0)
    # and the two maps' query gradients are equal and opposite
    assert np.allclose(got["dq1"], -got["dq2"], atol=1e-15, rtol=0)


def test_lambda_backward_matches_finite_differences():
    rng = np.random.default_rng(50)
    H, dim = 3, 5
    vecs = [rng.normal(0, 0.3, (H, dim)) for _ in range(4)]
    dlam = rng.standard_normal(H)
    got = oracle.lambda_backward(*vecs, dlam)
    h = 1e-6
    for i, name in enumerate(("dlq1", "dlk1", "dlq2", "dlk2")):
        num = np.zeros((H, dim))
        for idx in np.ndindex(H, dim):
            vp = [a.copy() for a in vecs]
            vm = [a.copy() for a in vecs]
            vp[i][idx] += h
            vm[i][idx] -= h
            num[idx] = (np.sum(dlam * oracle.lam(*vp, 12)) - np.sum(dlam * oracle.lam(*vm, 12))) / (2 * h)
        assert np.allclose(got[name], num, atol=1e-8, rtol=0), name


# ------------------------------------------------------------------------------------------------
# DIFF V2 ("softmax can't say zero", section "DIFF V2: what the authors changed"): per-row lambda,
# query heads 2p and 2p+1 sharing the group's K and V, no norm
# ------------------------------------------------------------------------------------------------

def _v2_loss(x, dy, lam, causal, logits):
    y = oracle.v2_forward(x["q"], x["k"], x["v"], lam, causal=causal, lam_logits=logits)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("causal,logits", [(True, False), (False, False), (True, True)])
def test_v2_backward_matches_finite_differences(causal, logits):
    # one KV head shared by two pairs (a group of four query heads), so dK and dV must add up
    # over every head of the group
    rng = np.random.default_rng(40 + 2 * causal + logits)
    B, N, H2, hkv, d = 1, 5, 4, 1, 3
    x = {"q": rng.standard_normal((B, N, H2, d)), "k": rng.standard_normal((B, N, hkv, d)),
         "v": rng.standard_normal((B, N, hkv, d))}
    lam = rng.standard_normal((B, N, H2 // 2)) if logits else rng.uniform(0.1, 0.9, (B, N, H2 // 2))
    dy = rng.standard_normal((B, N, H2 // 2, d))
    got = oracle.v2_backward(x["q"], x["k"], x["v"], lam, dy, causal=causal, lam_logits=logits)
    h = 1e-6
    for name in ("q", "k", "v"):
        num = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {k: a.copy() for k, a in x.items()}
            xm = {k: a.copy() for k, a in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (_v2_loss(xp, dy, lam, causal, logits) - _v2_loss(xm, dy, lam, causal, logits)) / (2 * h)
        assert np.allclose(got["d" + name], num, atol=2e-7, rtol=0), name
    num = np.zeros_like(lam)
    for idx in np.ndindex(*lam.shape):
        lp, lm = lam.copy(), lam.copy()
        lp[idx] += h
        lm[idx] -= h
        num[idx] = (_v2_loss(x, dy, lp, causal, logits) - _v2_loss(x, dy, lm, causal, logits)) / (2 * h)
    assert np.allclose(got["dlam"], num, atol=2e-7, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_v2_backward_lambda_zero_is_gqa_attention_gradient(causal):
    # lambda = 0: each pair's output is query head 2p's GQA attention; torch autograd of SDPA over
    # the KV heads repeated per query head gives dQ of the even heads and, summed, dK and dV
    rng = np.random.default_rng(50 + causal)
    B, N, H2, hkv, d = 2, 8, 8, 2, 5
    q = rng.standard_normal((B, N, H2, d))
    k, v = rng.standard_normal((B, N, hkv, d)), rng.standard_normal((B, N, hkv, d))
    dy = rng.standard_normal((B, N, H2 // 2, d))
    got = oracle.v2_backward(q, k, v, np.zeros((B, N, H2 // 2)), dy, causal=causal)
    group = H2 // hkv
    tq = torch.from_numpy(q[:, :, 0::2]).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    rep = lambda a: a.repeat_interleave(group // 2, dim=1)     # KV head of each even query head
    o = torch.nn.functional.scaled_dot_product_attention(tq, rep(tk), rep(tv), is_causal=causal)
    o.backward(torch.from_numpy(dy).permute(0, 2, 1, 3))
    assert np.allclose(got["dq"][:, :, 0::2], tq.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    assert np.all(got["dq"][:, :, 1::2] == 0)
    assert np.allclose(got["dk"], tk.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    assert np.allclose(got["dv"], tv.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)


def test_v2_train_stats_definitions():
    # maps are the two heads' own attention outputs (lambda = 0 and the forward's difference),
    # and the weights exp2(c s - lse) of each row sum to one
    rng = np.random.default_rng(60)
    B, N, H2, hkv, d = 1, 7, 4, 2, 4
    q = rng.standard_normal((B, N, H2, d))
    k, v = rng.standard_normal((B, N, hkv, d)), rng.standard_normal((B, N, hkv, d))
    lse, maps = oracle.v2_train_stats(q, k, v, causal=True)
    lam = rng.uniform(0, 1, (B, N, H2 // 2))
    out = oracle.v2_forward(q, k, v, lam, causal=True)
    assert np.allclose(out, maps[..., 0, :] - lam[..., None] * maps[..., 1, :], atol=1e-13, rtol=0)
    c = np.log2(np.e) / np.sqrt(d)
    for p in range(H2 // 2):
        for m in range(2):
            s = q[0, :, 2 * p + m] @ k[0, :, (2 * p) // (H2 // hkv)].T
            w = np.exp2(c * s - lse[0, p, :, m][:, None]) * np.tri(N)
            assert np.allclose(w.sum(axis=1), 1.0, atol=1e-13)


def test_v2_backward_query_suffix():
    # the last Nq query rows against all keys give those rows' dQ and dlambda, and the complete dK
    # and dV of the keys only they see, exactly as the full problem does
    rng = np.random.default_rng(70)
    B, N, H2, hkv, d, M = 1, 12, 4, 2, 3, 4
    q = rng.standard_normal((B, N, H2, d))
    k, v = rng.standard_normal((B, N, hkv, d)), rng.standard_normal((B, N, hkv, d))
    lam = rng.uniform(0, 1, (B, N, H2 // 2))
    dy = rng.standard_normal((B, N, H2 // 2, d))
    full = oracle.v2_backward(q, k, v, lam, dy, causal=True)
    part = oracle.v2_backward(q[:, -M:], k, v, lam[:, -M:], dy[:, -M:], causal=True)
    assert np.allclose(part["dq"], full["dq"][:, -M:], atol=1e-13, rtol=0)
    assert np.allclose(part["dlam"], full["dlam"][:, -M:], atol=1e-13, rtol=0)
    assert np.allclose(part["dk"][:, -M:], full["dk"][:, -M:], atol=1e-13, rtol=0)
    assert np.allclose(part["dv"][:, -M:], full["dv"][:, -M:], atol=1e-13, rtol=0)
