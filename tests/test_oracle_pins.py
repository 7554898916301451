"""Pins for the fp64 oracle: facts the pages and mathematics fix, independent of the oracle's code.

Each test names the passage (page title, section) it checks against. None of
them re-derives a value by calling the oracle's own formula a second way; they
use printed values, closed forms, invariants, or library routines that the
method reduces to in a special case.
"""
import concurrent.futures as cf
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _weights(z1, z2, lam):
    """The oracle's differential weight row for arbitrary logits z1, z2 (length n).

    d = 1 with q = 1 and k_j = z_j makes the logit of key j exactly z_j (scale 1);
    V = identity makes the output row equal the weight row.
    """
    n = len(z1)
    one = np.ones((1, 1))
    return oracle._head(one, one, np.asarray(z1, float)[:, None], np.asarray(z2, float)[:, None],
                        _eye(n), np.array([lam]), False, 1.0, None)[0]


_EYES = {}


def _eye(n):
    if n not in _EYES:
        _EYES[n] = np.eye(n)
    return _EYES[n]


# ----------------------------------------------------------------------------------------------
# lambda schedule and re-parameterisation
# ("softmax can't say zero", section "lambda, re-parameterised";
#  "Noise-Canceling Attention by Subtraction", section "Making lambda learnable and stable")
# ----------------------------------------------------------------------------------------------

def test_lambda_init_table():
    t = _load("lambda_schedule.json")
    for l, want, want1m in zip(t["layers"], t["lambda_init_2dp"], t["one_minus_lambda_init_2dp"]):
        got = oracle.lambda_init(l)
        assert round(got, 2) == pytest.approx(want, abs=1e-12), (l, got)
        assert round(1.0 - got, 2) == pytest.approx(want1m, abs=1e-12), (l, got)


def test_lambda_init_endpoints():
    # about 0.2 at the first layer, tending to 0.8 with depth; strictly increasing.
    assert oracle.lambda_init(1) == pytest.approx(0.2, abs=1e-15)
    assert oracle.lambda_init(200) == pytest.approx(0.8, abs=1e-15)
    vals = [oracle.lambda_init(l) for l in range(1, 40)]
    assert all(b > a for a, b in zip(vals, vals[1:]))


def test_lambda_zero_vectors_give_lambda_init():
    z = np.zeros((3, 64))
    for layer in (1, 12, 24):
        got = oracle.lam(z, z, z, z, layer)
        assert np.all(got == oracle.lambda_init(layer))


def test_lambda_sign_of_each_term():
    # Only map-1 vectors nonzero: lambda exceeds lambda_init by exp(dot)-1 > 0;
    # only map-2 vectors nonzero: lambda falls below lambda_init. A swapped sign fails.
    a = np.full((1, 4), 0.5)
    z = np.zeros((1, 4))
    li = oracle.lambda_init(5)
    up = oracle.lam(a, a, z, z, 5)[0]
    down = oracle.lam(z, z, a, a, 5)[0]
    assert up == pytest.approx(li + math.e - 1.0, rel=1e-14)      # dot = 4 * 0.25 = 1
    assert down == pytest.approx(li - (math.e - 1.0), rel=1e-14)


def test_lambda_init_spread_monte_carlo():
    t = _load("lambda_schedule.json")["init_spread"]
    rng = np.random.default_rng(12345)
    n, dim, std = 50_000, t["head_dim"], t["vector_std"]
    vecs = [rng.normal(0.0, std, size=(n, dim)) for _ in range(4)]
    lam = oracle.lam(*vecs, layer=28)
    dots = np.sum(vecs[0] * vecs[1], axis=1)
    assert np.std(dots) == pytest.approx(t["dot_std_approx"], abs=0.002)
    assert np.std(lam) == pytest.approx(t["lambda_std_measured"], abs=0.002)
    assert np.mean(lam) == pytest.approx(oracle.lambda_init(28), abs=0.003)


# ----------------------------------------------------------------------------------------------
# softmax per map: the needle closed form ("softmax can't say zero", "Why softmax can't say zero")
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [32, 4096, 65536])
def test_needle_closed_form(n):
    gaps = _load("needle_gaps.json")
    printed = dict(zip(gaps["n"], gaps["printed_half_weight_gap"]))[n]
    lam = 0.7
    for D in (printed, 2.5, 8.0):
        # map 1: one key at logit D, the rest at 0; map 2: every logit 0; V one-hot on the needle.
        z1 = np.zeros(n)
        z1[n // 3] = D
        q = np.array([[D * math.sqrt(4.0), 0, 0, 0]])      # d = 4, default scale 1/2
        k1 = np.zeros((n, 4))
        k1[n // 3, 0] = 1.0
        v = np.zeros((n, 1))
        v[n // 3, 0] = 1.0
        o = oracle._head(q, np.zeros((1, 4)), k1, np.zeros((n, 4)), v, np.array([lam]), False,
                         0.5, None)[0, 0]
        want = math.exp(D) / (math.exp(D) + n - 1) - lam / n
        # a sum of n rounded terms: relative error below n * 2^-52
        assert o == pytest.approx(want, rel=n * 2.0 ** -52, abs=1e-15)
    # the printed gap keeps half the weight on the needle, to the gap's printed rounding
    assert math.log(n - 1) == pytest.approx(printed, abs=0.005)
    k1 = np.zeros((n, 1))
    k1[0, 0] = printed
    v = np.zeros((n, 1))
    v[0, 0] = 1.0
    w0 = oracle._head(np.ones((1, 1)), np.ones((1, 1)), k1, np.zeros((n, 1)), v, np.array([0.0]),
                      False, 1.0, None)[0, 0]
    assert w0 == pytest.approx(0.5, abs=0.0025)


# ----------------------------------------------------------------------------------------------
# the difference: row sums and signs
# ("softmax can't say zero", "The row no longer sums to one"; the glossary's seeded example)
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_row_sums_are_one_minus_lambda(causal):
    rng = np.random.default_rng(7)
    B, N, H, d, dv = 1, 37, 3, 5, 4
    q1, q2, k1, k2 = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    v = rng.standard_normal((B, N, H, dv))
    v[..., 0] = 1.0
    lam = np.array([0.8, -0.3, 1.7])
    o = oracle.v1_forward(q1, q2, k1, k2, v, lam, causal=causal, epilogue=False)
    for h in range(H):
        assert np.allclose(o[0, :, h, 0], 1.0 - lam[h], atol=1e-13, rtol=0)


def test_glossary_worked_example():
    t = _load("glossary_worked_example.json")
    n, d, lam = t["n"], t["d"], t["lam"]
    torch.manual_seed(t["torch_seed"])
    q1, k1, q2, k2 = torch.randn(4, n, d).double().numpy()
    v = torch.randn(n, 2 * d).double().numpy()
    # V = identity exposes the weight matrix itself
    W = oracle._head(q1, q2, k1, k2, np.eye(n), np.full(n, lam), False, 1 / math.sqrt(d), None)
    assert f"{W.sum(axis=1)[0]:.2f}" == t["printed_row_sum"]
    assert np.allclose(W.sum(axis=1), 1 - lam, atol=1e-13)
    assert int((W < 0).sum()) == t["printed_negative_count"]
    assert W.size == t["printed_total_weights"]
    assert np.min(np.abs(W)) > 1e-3                 # the count is not a rounding accident
    # and the output with the real V is W @ V
    o = oracle._head(q1, q2, k1, k2, v, np.full(n, lam), False, 1 / math.sqrt(d), None)
    assert np.allclose(o, W @ v, atol=1e-13)


# ----------------------------------------------------------------------------------------------
# the toy: needle plus correlated noise ("softmax can't say zero", "The analogy, and where it breaks")
# ----------------------------------------------------------------------------------------------

def _toy_trial(n, rho, gap, sigma, lam, seeds):
    def one(seed):
        rng = np.random.default_rng(seed)
        c, e = rng.standard_normal((2, n))
        z1 = sigma * c
        z1[0] += gap
        z2 = sigma * (rho * c + math.sqrt(1 - rho ** 2) * e)
        single = _weights(z1, z2, 0.0)          # lambda = 0: map 1 alone
        diff = _weights(z1, z2, lam)
        return (abs(single[0]) / np.abs(single).sum(), abs(diff[0]) / np.abs(diff).sum(),
                single[0], diff[0])
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        res = np.array(list(ex.map(one, seeds)))
    return res.mean(axis=0)


def test_toy_table_n32():
    t = _load("toy_table.json")
    s = t["setup"]
    for row in t["rows_n32"]:
        got = _toy_trial(32, row["rho"], s["gap"], s["sigma"], s["lam"], range(1000))
        assert round(got[0], 3) == pytest.approx(row["share_single"], abs=1e-9), row
        assert round(got[1], 3) == pytest.approx(row["share_diff"], abs=1e-9), row
        assert round(got[2], 3) == pytest.approx(row["needle_single"], abs=1e-9), row
        assert round(got[3], 3) == pytest.approx(row["needle_diff"], abs=1e-9), row


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_toy_table_growing_n(idx):
    t = _load("toy_table.json")
    s = t["setup"]
    row = t["rows_rho09"][idx]
    got = _toy_trial(row["n"], 0.9, s["gap"], s["sigma"], s["lam"], range(1000))
    assert round(got[0], 3) == pytest.approx(row["share_single"], abs=1e-9), row
    assert round(got[1], 3) == pytest.approx(row["share_diff"], abs=1e-9), row


# ----------------------------------------------------------------------------------------------
# special cases that reduce to a library routine, and invariants
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_lambda_zero_is_standard_attention(causal):
    # lambda = 0 leaves map 1 alone: ordinary scaled-dot-product attention
    # ("Noise-Canceling Attention by Subtraction", section "The mechanism").
    rng = np.random.default_rng(3)
    B, N, H, d, dv = 2, 29, 2, 6, 12
    q1, q2, k1, k2 = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    v = rng.standard_normal((B, N, H, dv))
    o = oracle.v1_forward(q1, q2, k1, k2, v, np.zeros(H), causal=causal, epilogue=False)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q1), t(k1), t(v), is_causal=causal)
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)


def test_common_mode_cancels():
    # identical maps and lambda = 1: the difference is exactly zero
    # ("Noise-Canceling Attention by Subtraction", introduction: shared noise cancels).
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 20, 2, 4))
    k = rng.standard_normal((1, 20, 2, 4))
    v = rng.standard_normal((1, 20, 2, 8))
    o = oracle.v1_forward(q, q, k, k, v, np.ones(2), causal=True, epilogue=False)
    assert np.all(o == 0.0)


def test_brute_force_tiny():
    # Per-element sums on tiny inputs, spelled out over every (i, j, c) with Python floats.
    rng = np.random.default_rng(5)
    N, d, dv, lam = 5, 3, 4, 0.6
    q1, q2, k1, k2 = (rng.standard_normal((N, d)) for _ in range(4))
    v = rng.standard_normal((N, dv))
    for causal in (False, True):
        o = oracle._head(q1, q2, k1, k2, v, np.full(N, lam), causal, 1 / math.sqrt(d), None)
        for i in range(N):
            keys = range(i + 1) if causal else range(N)
            e1 = [math.exp(sum(q1[i, c] * k1[j, c] for c in range(d)) / math.sqrt(d)) for j in keys]
            e2 = [math.exp(sum(q2[i, c] * k2[j, c] for c in range(d)) / math.sqrt(d)) for j in keys]
            for c in range(dv):
                want = sum((a / sum(e1) - lam * b / sum(e2)) * v[j, c]
                           for a, b, j in zip(e1, e2, keys))
                assert o[i, c] == pytest.approx(want, abs=1e-13)


def test_causal_prefix_property():
    rng = np.random.default_rng(6)
    N, d, dv = 24, 4, 6
    q1, q2, k1, k2 = (rng.standard_normal((1, N, 1, d)) for _ in range(4))
    v = rng.standard_normal((1, N, 1, dv))
    full = oracle.v1_forward(q1, q2, k1, k2, v, [0.5], causal=True, epilogue=True,
                             lambda_init_value=0.3)
    for i in (0, 1, 7, N - 1):
        part = oracle.v1_forward(*(x[:, :i + 1] for x in (q1, q2, k1, k2, v)), [0.5], causal=True,
                                 epilogue=True, lambda_init_value=0.3)
        assert np.array_equal(full[0, i], part[0, i])


def test_noncausal_key_permutation_invariance():
    rng = np.random.default_rng(8)
    N, d, dv = 19, 4, 6
    q1, q2, k1, k2 = (rng.standard_normal((1, N, 1, d)) for _ in range(4))
    v = rng.standard_normal((1, N, 1, dv))
    perm = rng.permutation(N)
    a = oracle.v1_forward(q1, q2, k1, k2, v, [0.8], causal=False, epilogue=False)
    b = oracle.v1_forward(q1, q2, k1[:, perm], k2[:, perm], v[:, perm], [0.8], causal=False,
                          epilogue=False)
    assert np.allclose(a, b, atol=1e-13, rtol=0)


def test_rmsnorm_scale_closed_form():
    # With unit weight the epilogue output satisfies mean_c out^2 = (1-li)^2 ms/(ms+eps);
    # a weight g scales channel c by g_c.
    rng = np.random.default_rng(9)
    N, d, dv, li, eps = 16, 4, 8, 0.37, 1e-3
    args = [rng.standard_normal((1, N, 1, d)) for _ in range(4)] + [rng.standard_normal((1, N, 1, dv))]
    raw = oracle.v1_forward(*args, [0.8], causal=True, epilogue=False)[0, :, 0]
    out = oracle.v1_forward(*args, [0.8], causal=True, epilogue=True, lambda_init_value=li,
                            eps=eps)[0, :, 0]
    ms = np.mean(raw ** 2, axis=1)
    assert np.allclose(np.mean(out ** 2, axis=1), (1 - li) ** 2 * ms / (ms + eps), rtol=1e-12)
    assert np.allclose(out / raw, ((1 - li) / np.sqrt(ms + eps))[:, None], rtol=1e-12)
    g = rng.uniform(0.5, 2.0, dv)
    outg = oracle.v1_forward(*args, [0.8], causal=True, epilogue=True, lambda_init_value=li,
                             eps=eps, g=g)[0, :, 0]
    assert np.allclose(outg, out * g[None, :], rtol=1e-12)


def test_decode_is_last_causal_row():
    rng = np.random.default_rng(10)
    B, L, H, d, dv = 2, 33, 3, 4, 8
    q1, q2, k1, k2 = (rng.standard_normal((B, L, H, d)) for _ in range(4))
    v = rng.standard_normal((B, L, H, dv))
    lam = np.array([0.2, 0.5, 0.8])
    fwd = oracle.v1_forward(q1, q2, k1, k2, v, lam, causal=True, epilogue=True,
                            lambda_init_value=0.8)
    dec = oracle.decode(q1[:, -1], q2[:, -1], k1, k2, v, lam, epilogue=True, lambda_init_value=0.8)
    assert np.array_equal(dec, fwd[:, -1])
    # a shorter cache length per batch entry is the same as truncating the cache
    lens = np.array([L, 10])
    dec2 = oracle.decode(q1[:, 9], q2[:, 9], k1, k2, v, lam, cache_lens=lens, epilogue=True,
                         lambda_init_value=0.8)
    assert np.array_equal(dec2[1], fwd[1, 9])


# ----------------------------------------------------------------------------------------------
# V2 ("softmax can't say zero", "DIFF V2: what the authors changed"; "Differential Transformer V2")
# ----------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_v2_lambda_zero_is_gqa_attention(causal):
    # lambda = 0 leaves the even query heads' ordinary GQA attention; heads of one
    # group are contiguous, so query head j reads KV head j // (2h / h_kv).
    rng = np.random.default_rng(11)
    B, N, hq, hkv, d = 2, 21, 8, 2, 6
    q = rng.standard_normal((B, N, hq, d))
    k = rng.standard_normal((B, N, hkv, d))
    v = rng.standard_normal((B, N, hkv, d))
    o = oracle.v2_forward(q, k, v, np.zeros((B, N, hq // 2)), causal=causal)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    rep = hq // hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k).repeat_interleave(rep, dim=1), t(v).repeat_interleave(rep, dim=1),
        is_causal=causal).permute(0, 2, 1, 3).numpy()
    assert np.allclose(o, ref[:, :, 0::2], atol=1e-12, rtol=0)
    # lambda = 1 with the odd heads' output known: o = even - odd
    lam1 = oracle.v2_forward(q, k, v, np.ones((B, N, hq // 2)), causal=causal)
    assert np.allclose(lam1, ref[:, :, 0::2] - ref[:, :, 1::2], atol=1e-12, rtol=0)


def test_v2_per_token_lambda_and_cancel():
    rng = np.random.default_rng(12)
    B, N, hq, hkv, d = 1, 15, 4, 1, 4
    q = rng.standard_normal((B, N, hq, d))
    q[:, :, 1] = q[:, :, 0]                                 # pair 0: identical maps
    k = rng.standard_normal((B, N, hkv, d))
    v = rng.standard_normal((B, N, hkv, d))
    lam = rng.uniform(0, 1, (B, N, hq // 2))
    lam[:, :, 0] = 1.0
    o = oracle.v2_forward(q, k, v, lam, causal=True)
    assert np.all(o[:, :, 0] == 0.0)
    # row sums of the weights are 1 - lambda per token: ones in V's channel 0
    v1 = v.copy()
    v1[..., 0] = 1.0
    o1 = oracle.v2_forward(q, k, v1, lam, causal=True)
    assert np.allclose(o1[0, :, 1, 0], 1.0 - lam[0, :, 1], atol=1e-13)


def test_v2_uniform_attention_rms():
    # Uniform attention over n unit-RMS, uncorrelated values has output RMS near 1/sqrt(n)
    # ("softmax can't say zero", "DIFF V2": the reason V2 drops the per-head norm).
    rng = np.random.default_rng(13)
    n, d = 4096, 64
    q = np.zeros((1, n, 2, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    rows = np.array([[0, 0, n - 1]])
    o = oracle.v2_forward(q, k, v, np.zeros((1, n, 1)), causal=True, rows=rows)
    rms = np.sqrt(np.mean(o ** 2))
    assert rms == pytest.approx(1 / math.sqrt(n), rel=0.25)


def test_v2_decode_single_query_gqa_attention():
    # V2 decode with lambda = 0 is one query of ordinary GQA attention over the cache prefix
    # (a library routine), and with lambda = 1 it is the difference of the pair's two heads.
    rng = np.random.default_rng(14)
    B, L, hq, hkv, d = 3, 37, 8, 2, 6
    q = rng.standard_normal((B, hq, d))
    kc = rng.standard_normal((B, L, hkv, d))
    vc = rng.standard_normal((B, L, hkv, d))
    lens = np.array([L, 1, 20])
    rep = hq // hkv
    refs = []
    for b in range(B):
        n = lens[b]
        qq = torch.from_numpy(q[b])[:, None, :]                               # [hq, 1, d]
        kk = torch.from_numpy(kc[b, :n]).permute(1, 0, 2).repeat_interleave(rep, dim=0)
        vv = torch.from_numpy(vc[b, :n]).permute(1, 0, 2).repeat_interleave(rep, dim=0)
        refs.append(torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0].numpy())
    ref = np.stack(refs)                                                       # [B, hq, d]
    o0 = oracle.v2_decode(q, kc, vc, np.zeros((B, hq // 2)), cache_lens=lens)
    assert np.allclose(o0, ref[:, 0::2], atol=1e-12, rtol=0)
    o1 = oracle.v2_decode(q, kc, vc, np.ones((B, hq // 2)), cache_lens=lens)
    assert np.allclose(o1, ref[:, 0::2] - ref[:, 1::2], atol=1e-12, rtol=0)
    # a cache of length 1 returns that row's value for every head: weights are exactly 1
    assert np.allclose(o0[1], vc[1, 0][[(2 * p) // rep for p in range(hq // 2)]], atol=1e-15, rtol=0)


def test_v2_decode_is_last_causal_row():
    # decoding the last token against the full cache is the last row of the causal V2 forward
    rng = np.random.default_rng(15)
    B, N, hq, hkv, d = 2, 29, 4, 2, 5
    q = rng.standard_normal((B, N, hq, d))
    k = rng.standard_normal((B, N, hkv, d))
    v = rng.standard_normal((B, N, hkv, d))
    lam = rng.uniform(0, 1, (B, N, hq // 2))
    fwd = oracle.v2_forward(q, k, v, lam, causal=True)
    dec = oracle.v2_decode(q[:, -1], k, v, lam[:, -1])
    assert np.array_equal(dec, fwd[:, -1])


# ------------------------------------------------------------------------------------------------
# Paged caches: the gather that reads a page pool through a block table
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("L,page", [(100, 32), (96, 32), (300, 64), (5, 256)])
def test_gather_pages_round_trip(L, page):
    # the seeded scatter (an input generator, written separately) followed by the gather gives the
    # contiguous cache back exactly, for ragged last pages too
    import workloads as W
    c = torch.randn(3, L, 2, 8, generator=torch.Generator().manual_seed(L + page))
    pool, table = W.scatter_to_pages(c, page, seed=L * page)
    assert table.shape == (3, (L + page - 1) // page)
    assert len(set(table.flatten().tolist())) == table.numel()          # no page shared
    back = oracle.gather_pages(pool.numpy(), table.numpy(), L, page)
    assert np.array_equal(back, c.numpy())


def test_gather_pages_identity_table():
    # sequence b's pages stored consecutively: the pool is the contiguous cache cut into pages
    B, L, page = 2, 128, 32
    c = np.arange(B * L * 3 * 4, dtype=np.float64).reshape(B, L, 3, 4)
    pool = c.reshape(B * L // page, page, 3, 4)
    table = np.arange(B * L // page).reshape(B, L // page)
    assert np.array_equal(oracle.gather_pages(pool, table, L, page), c)
    # a shorter length reads a prefix, and entries past it are never used
    table2 = table.copy()
    table2[:, -1] = 10 ** 6
    assert np.array_equal(oracle.gather_pages(pool, table2, L - page, page), c[:, :L - page])


# ------------------------------------------------------------------------------------------------
# DIFF V2 lambda from logits: lambda = sigmoid(W x) ("softmax can't say zero", section "DIFF V2:
# what the authors changed"), pinned at points where the sigmoid has a closed form
# ------------------------------------------------------------------------------------------------

def _v2_small(seed):
    rng = np.random.default_rng(seed)
    B, N, H2, hkv, d = 2, 9, 4, 2, 8
    return rng.standard_normal((B, N, H2, d)), rng.standard_normal((B, N, hkv, d)), rng.standard_normal((B, N, hkv, d))


@pytest.mark.parametrize("z,lam_value", [(0.0, 0.5), (math.log(3.0), 0.75), (-math.log(3.0), 0.25),
                                         (math.log(0.25), 0.2)])
def test_v2_logits_closed_form_points(z, lam_value):
    q, k, v = _v2_small(11)
    B, N = q.shape[:2]
    out_z = oracle.v2_forward(q, k, v, np.full((B, N, 2), z), causal=True, lam_logits=True)
    out_v = oracle.v2_forward(q, k, v, np.full((B, N, 2), lam_value), causal=True)
    assert np.max(np.abs(out_z - out_v)) < 1e-14


def test_v2_logits_saturate():
    # a large positive logit gives lambda = 1 (the full difference), a large negative one gives
    # lambda = 0: the pair's first head alone, i.e. plain GQA attention of head 2p
    q, k, v = _v2_small(12)
    B, N = q.shape[:2]
    hi = oracle.v2_forward(q, k, v, np.full((B, N, 2), 60.0), causal=True, lam_logits=True)
    one = oracle.v2_forward(q, k, v, np.ones((B, N, 2)), causal=True)
    assert np.max(np.abs(hi - one)) < 1e-12
    lo = oracle.v2_forward(q, k, v, np.full((B, N, 2), -800.0), causal=True, lam_logits=True)
    zero = oracle.v2_forward(q, k, v, np.zeros((B, N, 2)), causal=True)
    assert np.array_equal(lo, zero)


def test_v2_decode_logits_match_forward_last_row():
    q, k, v = _v2_small(13)
    B, N = q.shape[:2]
    z = np.random.default_rng(14).standard_normal((B, N, 2)) * 3
    fwd = oracle.v2_forward(q, k, v, z, causal=True, lam_logits=True)
    dec = oracle.v2_decode(q[:, -1], k, v, z[:, -1], lam_logits=True)
    assert np.max(np.abs(fwd[:, -1] - dec)) < 1e-13
