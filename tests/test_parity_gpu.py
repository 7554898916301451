"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Tolerances: max |GPU - oracle| <= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs (bf16 in,
fp32 accumulate, bf16 out). Small cases are checked element by element everywhere; the full-size
workloads are checked on sampled rows the oracle computes one by one, in the same launch
configuration the benchmark times.
"""
import math
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


def rand(shape, seed, dtype, device=DEV, scale=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype).to(device)


def v1_case(B, Nq, Nk, H, d, dv, dtype, seed, causal, epilogue, lam=None, li=0.8, norm=False,
            scale=None, eps=1e-5, qscale=1.0):
    q1 = rand((B, Nq, H, d), seed, dtype, scale=qscale)
    q2 = rand((B, Nq, H, d), seed + 1, dtype, scale=qscale)
    k1 = rand((B, Nk, H, d), seed + 2, dtype)
    k2 = rand((B, Nk, H, d), seed + 3, dtype)
    v = rand((B, Nk, H, dv), seed + 4, dtype)
    lam = torch.linspace(0.2, 0.9, H) if lam is None else torch.as_tensor(lam, dtype=torch.float32)
    # norm weight in [0.75, 1.25): outputs stay O(1), where bf16 rounding is far below the tolerance
    w = 0.75 + 0.5 * torch.rand((dv,), generator=torch.Generator().manual_seed(seed + 5)) if norm else None
    note(f"v1 case B={B} Nq={Nq} Nk={Nk} H={H} d={d} dv={dv} {dtype} causal={causal} epi={epilogue}")
    out = da.diffattn_fwd(q1, q2, k1, k2, v, lam.to(DEV), causal=causal, epilogue=epilogue,
                          lambda_init_value=li, norm_w=None if w is None else w.to(DEV), eps=eps,
                          scale=0.0 if scale is None else scale)
    torch.cuda.synchronize()
    ref = oracle.v1_forward(f64(q1), f64(q2), f64(k1), f64(k2), f64(v), lam.numpy(), causal=causal,
                            epilogue=epilogue, lambda_init_value=li,
                            g=None if w is None else w.numpy(), eps=eps, scale=scale)
    return f64(out), ref


def maxerr(a, b):
    return float(np.max(np.abs(a - b)))


# ------------------------------------------------------------------------------------------------
# fp32 (generic kernel)
# ------------------------------------------------------------------------------------------------

def test_fp32_single_head_config():
    cfg = W.FP32_SINGLE_HEAD
    x = W.v1_inputs(cfg, device=DEV)
    lam = x["lam_fixed"].to(DEV)
    note("fp32 single head N=64 d=8 dv=16")
    out = da.diffattn_fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, causal=False, epilogue=False)
    torch.cuda.synchronize()
    ref = oracle.v1_forward(f64(x["q1"]), f64(x["q2"]), f64(x["k1"]), f64(x["k2"]), f64(x["v"]),
                            lam.cpu().numpy(), causal=False, epilogue=False)
    assert maxerr(f64(out), ref) <= TOL_F32


@pytest.mark.parametrize("N", [1, 2, 5, 63, 64, 65, 130])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_shapes(N, causal):
    out, ref = v1_case(2, N, N, 3, 8, 16, torch.float32, 100 + N, causal, epilogue=causal)
    assert maxerr(out, ref) <= TOL_F32


def test_fp32_rect_and_options():
    out, ref = v1_case(1, 7, 50, 2, 24, 40, torch.float32, 7, causal=True, epilogue=True, norm=True,
                       scale=0.3, li=0.35, eps=1e-3)
    assert maxerr(out, ref) <= TOL_F32
    out, ref = v1_case(2, 33, 20, 2, 16, 32, torch.float32, 8, causal=False, epilogue=False)
    assert maxerr(out, ref) <= TOL_F32


# ------------------------------------------------------------------------------------------------
# bf16 V1 prefill (MFMA kernel: d = 64, dv = 128)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 300])
def test_bf16_v1_causal_shapes(N):
    out, ref = v1_case(2, N, N, 3, 64, 128, torch.bfloat16, 200 + N, causal=True, epilogue=True,
                       li=0.7779)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("N", [1, 33, 128, 257])
def test_bf16_v1_noncausal_noepi(N):
    out, ref = v1_case(2, N, N, 2, 64, 128, torch.bfloat16, 300 + N, causal=False, epilogue=False)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("Nq,Nk,causal", [(17, 100, True), (64, 200, True), (130, 131, False),
                                          (5, 300, False)])
def test_bf16_v1_rect(Nq, Nk, causal):
    out, ref = v1_case(1, Nq, Nk, 2, 64, 128, torch.bfloat16, 400 + Nq, causal=causal, epilogue=True)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("Nq,Nk,causal", [(50, 4500, True), (50, 4500, False), (300, 4133, True)])
def test_bf16_v1_rect_long_keys(Nq, Nk, causal):
    # from 4096 keys the launches take the kernels built under the max-ilp schedule; a few query
    # tiles against a ragged key range
    out, ref = v1_case(1, Nq, Nk, 2, 64, 128, torch.bfloat16, 450 + Nq, causal=causal, epilogue=True)
    assert maxerr(out, ref) <= TOL_BF16


def test_bf16_v1_options():
    out, ref = v1_case(2, 150, 150, 2, 64, 128, torch.bfloat16, 500, causal=True, epilogue=True,
                       norm=True, scale=0.2, li=0.6, eps=1e-3, lam=[-0.4, 1.3])
    assert maxerr(out, ref) <= TOL_BF16


def test_bf16_v1_packed_strided_inputs():
    # Q1/Q2 (and K1/K2) as the two halves of one packed [B, N, H, 2, d] projection output
    B, N, H, d, dv = 2, 100, 3, 64, 128
    qp = rand((B, N, H, 2, d), 11, torch.bfloat16)
    kp = rand((B, N, H, 2, d), 12, torch.bfloat16)
    v = rand((B, N, H, dv), 13, torch.bfloat16)
    lam = torch.tensor([0.5, 0.7, 0.9])
    q1, q2, k1, k2 = qp[:, :, :, 0], qp[:, :, :, 1], kp[:, :, :, 0], kp[:, :, :, 1]
    assert not q1.is_contiguous()
    note("packed strided V1")
    out = da.diffattn_fwd(q1, q2, k1, k2, v, lam.to(DEV), causal=True, epilogue=True)
    torch.cuda.synchronize()
    ref = oracle.v1_forward(f64(q1), f64(q2), f64(k1), f64(k2), f64(v), lam.numpy(), causal=True,
                            epilogue=True)
    assert maxerr(f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("top", [38.8, 318.0])
def test_bf16_v1_large_logits(top):
    # logit magnitudes of the size the pages report for trained models (top-1 38.8 and 318):
    # the running maximum must absorb them without overflow.
    B, N, H = 1, 200, 2
    qscale = top / 8.0 / 4.0       # q.k over 64 channels has std 8; scaled by 1/8 -> std 1
    out, ref = v1_case(B, N, N, H, 64, 128, torch.bfloat16, 600, causal=True, epilogue=True,
                       qscale=qscale)
    assert np.all(np.isfinite(out))
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_v1_dense_large_logits(causal):
    # every logit large: std 12 in natural units (17 in base 2), so each row's weights hinge on
    # small logit differences between many competing keys
    out, ref = v1_case(1, 900, 900, 2, 64, 128, torch.bfloat16, 650, causal=causal, epilogue=False,
                       qscale=12.0)
    assert maxerr(out, ref) <= TOL_BF16


def test_bf16_generic_fallback_shape():
    out, ref = v1_case(2, 70, 70, 2, 32, 64, torch.bfloat16, 700, causal=True, epilogue=True)
    assert maxerr(out, ref) <= TOL_BF16


def test_common_mode_cancels_exactly():
    B, N, H = 1, 160, 2
    q = rand((B, N, H, 64), 21, torch.bfloat16)
    k = rand((B, N, H, 64), 22, torch.bfloat16)
    v = rand((B, N, H, 128), 23, torch.bfloat16)
    out = da.diffattn_fwd(q, q, k, k, v, torch.ones(H, device=DEV), causal=True, epilogue=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_deterministic_repeat():
    B, N, H = 2, 300, 2
    args = [rand((B, N, H, 64), 30 + i, torch.bfloat16) for i in range(4)] + \
           [rand((B, N, H, 128), 34, torch.bfloat16)]
    lam = torch.tensor([0.3, 0.6], device=DEV)
    a = da.diffattn_fwd(*args, lam, causal=True, epilogue=True)
    b = da.diffattn_fwd(*args, lam, causal=True, epilogue=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------------
# lambda
# ------------------------------------------------------------------------------------------------

def test_lambda_kernel():
    cfg = W.V1_PREFILL_2K
    x = W.v1_inputs(cfg, device="cpu", B=1, N=1)
    vec = [x[k] for k in ("lq1", "lk1", "lq2", "lk2")]
    got = da.diffattn_lambda(*(t.to(DEV) for t in vec), cfg.layer)
    torch.cuda.synchronize()
    ref = oracle.lam(*(t.double().numpy() for t in vec), cfg.layer)
    assert np.max(np.abs(got.cpu().double().numpy() - ref)) <= 1e-6
    one = da.diffattn_lambda(*(t[0].contiguous().to(DEV) for t in vec), 3)
    assert one.shape == (1,)


# ------------------------------------------------------------------------------------------------
# decode
# ------------------------------------------------------------------------------------------------

def decode_case(B, H, L, d, dv, seed, lens=None, epilogue=True, dtype=torch.bfloat16):
    q1 = rand((B, H, d), seed, dtype)
    q2 = rand((B, H, d), seed + 1, dtype)
    k1 = rand((B, L, H, d), seed + 2, dtype)
    k2 = rand((B, L, H, d), seed + 3, dtype)
    v = rand((B, L, H, dv), seed + 4, dtype)
    lam = torch.linspace(0.2, 0.8, H)
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    note(f"decode case B={B} H={H} L={L} d={d} dv={dv} lens={lens}")
    out = da.diffattn_decode(q1, q2, k1, k2, v, lam.to(DEV), cache_lens=lens_t, epilogue=epilogue)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q1), f64(q2), f64(k1), f64(k2), f64(v), lam.numpy(), cache_lens=lens,
                        epilogue=epilogue)
    return f64(out), ref


@pytest.mark.parametrize("L", [1, 7, 128, 1000, 5000])
def test_decode_shapes(L):
    out, ref = decode_case(3, 4, L, 64, 128, 800 + L)
    assert maxerr(out, ref) <= TOL_BF16


def test_decode_ragged_lengths_and_noepi():
    out, ref = decode_case(4, 2, 3000, 64, 128, 900, lens=[3000, 1, 129, 2047], epilogue=False)
    assert maxerr(out, ref) <= TOL_BF16


def test_decode_generic_fallback():
    out, ref = decode_case(2, 3, 300, 32, 48, 950, dtype=torch.float32)
    assert maxerr(out, ref) <= TOL_F32


def test_decode_equals_last_prefill_row():
    B, N, H = 2, 777, 3
    q1, q2, k1, k2 = (rand((B, N, H, 64), 40 + i, torch.bfloat16) for i in range(4))
    v = rand((B, N, H, 128), 44, torch.bfloat16)
    lam = torch.tensor([0.2, 0.5, 0.8], device=DEV)
    fwd = da.diffattn_fwd(q1, q2, k1, k2, v, lam, causal=True, epilogue=True)
    dec = da.diffattn_decode(q1[:, -1], q2[:, -1], k1, k2, v, lam, epilogue=True)
    torch.cuda.synchronize()
    assert maxerr(f64(dec), f64(fwd[:, -1])) <= TOL_BF16


# ------------------------------------------------------------------------------------------------
# V2
# ------------------------------------------------------------------------------------------------

def v2_case(B, N, hq, hkv, d, seed, causal=True, dtype=torch.bfloat16):
    q = rand((B, N, hq, d), seed, dtype)
    k = rand((B, N, hkv, d), seed + 1, dtype)
    v = rand((B, N, hkv, d), seed + 2, dtype)
    g = torch.Generator().manual_seed(seed + 3)
    lam = torch.rand((B, N, hq // 2), generator=g)
    note(f"v2 case B={B} N={N} hq={hq} hkv={hkv} d={d} causal={causal}")
    out = da.diffattn_v2_fwd(q, k, v, lam.to(DEV), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.v2_forward(f64(q), f64(k), f64(v), lam.numpy(), causal=causal)
    return f64(out), ref


@pytest.mark.parametrize("N", [1, 31, 33, 100, 257])
def test_v2_shapes(N):
    out, ref = v2_case(2, N, 16, 2, 128, 1000 + N)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 4), (32, 2), (8, 1)])
def test_v2_groupings(hq, hkv):
    out, ref = v2_case(1, 70, hq, hkv, 128, 1100 + hq, causal=(hq != 8))
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("N,causal", [(4200, True), (4133, False)])
def test_v2_long_keys(N, causal):
    # the V2 kernel built under the max-ilp schedule (4096 keys and more), ragged last tile
    out, ref = v2_case(1, N, 4, 2, 128, 1300 + N, causal=causal)
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_generic_fallback():
    out, ref = v2_case(1, 50, 6, 1, 64, 1200)
    assert maxerr(out, ref) <= TOL_BF16
    out, ref = v2_case(1, 40, 4, 2, 16, 1201, dtype=torch.float32)
    assert maxerr(out, ref) <= TOL_F32


# ------------------------------------------------------------------------------------------------
# V2 decode
# ------------------------------------------------------------------------------------------------

def v2_decode_case(B, L, hq, hkv, d, seed, lens=None, dtype=torch.bfloat16, qscale=1.0, kramp=None):
    q = rand((B, hq, d), seed, dtype, scale=qscale)
    k = rand((B, L, hkv, d), seed + 1, dtype)
    if kramp is not None:
        # key norms growing along the cache by the factor kramp
        ramp = torch.linspace(1.0, kramp, L, device=k.device).view(1, L, 1, 1)
        k = (k.float() * ramp).to(dtype)
    v = rand((B, L, hkv, d), seed + 2, dtype)
    g = torch.Generator().manual_seed(seed + 3)
    lam = torch.rand((B, hq // 2), generator=g)
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    note(f"v2 decode case B={B} L={L} hq={hq} hkv={hkv} d={d} lens={lens} qscale={qscale}")
    out = da.diffattn_v2_decode(q, k, v, lam.to(DEV), cache_lens=lens_t)
    torch.cuda.synchronize()
    ref = oracle.v2_decode(f64(q), f64(k), f64(v), lam.numpy(), cache_lens=lens)
    return f64(out), ref


@pytest.mark.parametrize("L", [1, 7, 32, 33, 300, 5000])
def test_v2_decode_shapes(L):
    out, ref = v2_decode_case(3, L, 16, 2, 128, 1300 + L)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (12, 2), (32, 2), (48, 2), (32, 1), (64, 8), (64, 2)])
def test_v2_decode_groupings(hq, hkv):
    out, ref = v2_decode_case(2, 700, hq, hkv, 128, 1400 + hq + hkv)
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_decode_ragged_lengths():
    out, ref = v2_decode_case(4, 3000, 16, 4, 128, 1500, lens=[3000, 1, 129, 2047])
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_decode_large_logits():
    # logits far outside +-60 (base 2) put the waves in shifted mode
    out, ref = v2_decode_case(2, 900, 8, 2, 128, 1550, qscale=12.0)
    assert maxerr(out, ref) <= TOL_BF16


@pytest.mark.parametrize("hq,hkv", [(16, 2), (48, 2)])
def test_v2_decode_logits_grow_along_the_cache(hq, hkv):
    # the first tiles' maxima lie within +-60 (base 2), later keys push the weights past the
    # unshifted bound, so the shifts move in the middle of a slice
    out, ref = v2_decode_case(2, 4000, hq, hkv, 128, 1570 + hq, kramp=40.0)
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_decode_many_slices_ragged_tail():
    # one (batch, KV head) unit per group and a cache that is no multiple of 32: the slice count
    # rule gives many slices, the last of them ending in a partial tile; a second batch row with a
    # short length leaves most of its slices empty
    out, ref = v2_decode_case(2, 40001, 16, 2, 128, 1580, lens=[40001, 700])
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_decode_large_logits_wide_group():
    out, ref = v2_decode_case(2, 900, 48, 2, 128, 1560, qscale=12.0)
    assert maxerr(out, ref) <= TOL_BF16


def test_v2_decode_generic_fallback():
    out, ref = v2_decode_case(2, 300, 8, 2, 64, 1600)                  # d = 64
    assert maxerr(out, ref) <= TOL_BF16
    out, ref = v2_decode_case(1, 200, 48, 1, 128, 1601)                # a group of 48 heads
    assert maxerr(out, ref) <= TOL_BF16
    out, ref = v2_decode_case(2, 100, 8, 4, 16, 1602, dtype=torch.float32)
    assert maxerr(out, ref) <= TOL_F32


def test_v2_decode_equals_last_prefill_row():
    B, N, hq, hkv = 2, 333, 16, 4
    q = rand((B, N, hq, 128), 1700, torch.bfloat16)
    k = rand((B, N, hkv, 128), 1701, torch.bfloat16)
    v = rand((B, N, hkv, 128), 1702, torch.bfloat16)
    lam = torch.rand((B, N, hq // 2), generator=torch.Generator().manual_seed(1703)).to(DEV)
    fwd = da.diffattn_v2_fwd(q, k, v, lam, causal=True)
    dec = da.diffattn_v2_decode(q[:, -1], k, v, lam[:, -1].contiguous())
    torch.cuda.synchronize()
    assert maxerr(f64(dec), f64(fwd[:, -1])) <= TOL_BF16


def test_v1_decode_deterministic():
    # split partials are merged in a fixed order: repeated calls agree bit for bit
    q1, q2 = rand((2, 4, 64), 1900, torch.bfloat16), rand((2, 4, 64), 1901, torch.bfloat16)
    k1, k2 = rand((2, 5000, 4, 64), 1902, torch.bfloat16), rand((2, 5000, 4, 64), 1903, torch.bfloat16)
    v = rand((2, 5000, 4, 128), 1904, torch.bfloat16)
    lam = torch.tensor([0.2, 0.4, 0.6, 0.8], device=DEV)
    a = da.diffattn_decode(q1, q2, k1, k2, v, lam)
    b = da.diffattn_decode(q1, q2, k1, k2, v, lam)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_v2_forward_deterministic():
    q = rand((1, 300, 8, 128), 1950, torch.bfloat16)
    k = rand((1, 300, 2, 128), 1951, torch.bfloat16)
    v = rand((1, 300, 2, 128), 1952, torch.bfloat16)
    lam = torch.rand((1, 300, 4), generator=torch.Generator().manual_seed(1953)).to(DEV)
    a = da.diffattn_v2_fwd(q, k, v, lam, causal=True)
    b = da.diffattn_v2_fwd(q, k, v, lam, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_v2_decode_deterministic():
    q = rand((2, 16, 128), 1800, torch.bfloat16)
    k = rand((2, 4000, 2, 128), 1801, torch.bfloat16)
    v = rand((2, 4000, 2, 128), 1802, torch.bfloat16)
    lam = torch.rand((2, 8), generator=torch.Generator().manual_seed(1803)).to(DEV)
    a = da.diffattn_v2_decode(q, k, v, lam)
    b = da.diffattn_v2_decode(q, k, v, lam)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------------
# full-size workloads, sampled rows (same launch configuration as the benchmark)
# ------------------------------------------------------------------------------------------------

def sample_rows(rng, B, H, N, extra_rows, n_random):
    rows = []
    for b in range(B):
        for h in range(H):
            picks = set(extra_rows) | set(rng.integers(0, N, n_random).tolist())
            rows += [(b, h, i) for i in sorted(picks) if 0 <= i < N]
    return np.array(rows)


def _boundary_rows(N):
    return [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2 - 1, N // 2, N - 2, N - 1]


def test_full_v1_prefill_2k():
    cfg = W.V1_PREFILL_2K
    x = W.v1_inputs(cfg, device=DEV)
    lam = da.diffattn_lambda(*(x[k].to(DEV) for k in ("lq1", "lk1", "lq2", "lk2")), cfg.layer)
    li = da.lambda_init(cfg.layer)
    note(f"full {cfg.name}")
    out = da.diffattn_fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, causal=True, epilogue=True,
                          lambda_init_value=li)
    torch.cuda.synchronize()
    rows = sample_rows(np.random.default_rng(0), cfg.B, cfg.H, cfg.N, _boundary_rows(cfg.N), 12)
    lam_ref = oracle.lam(*(x[k].double().numpy() for k in ("lq1", "lk1", "lq2", "lk2")), cfg.layer)
    ref = oracle.v1_forward(*(x[k].float().cpu().numpy() for k in ("q1", "q2", "k1", "k2", "v")),
                            lam_ref, causal=True, epilogue=True,
                            lambda_init_value=oracle.lambda_init(cfg.layer), rows=rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert maxerr(got, ref) <= TOL_BF16


def test_full_v1_prefill_32k_needle():
    cfg = W.V1_PREFILL_32K
    x = W.v1_inputs(cfg, device=DEV)
    lam = da.diffattn_lambda(*(x[k].to(DEV) for k in ("lq1", "lk1", "lq2", "lk2")), cfg.layer)
    li = da.lambda_init(cfg.layer)
    note(f"full {cfg.name}")
    out = da.diffattn_fwd(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, causal=True, epilogue=True,
                          lambda_init_value=li)
    torch.cuda.synchronize()
    rows = sample_rows(np.random.default_rng(1), cfg.B, cfg.H, cfg.N, _boundary_rows(cfg.N), 4)
    host = {k: x[k].float().cpu().numpy() for k in ("q1", "q2", "k1", "k2", "v")}
    ref = oracle.v1_forward(host["q1"], host["q2"], host["k1"], host["k2"], host["v"],
                            np.full(cfg.H, oracle.lambda_init(cfg.layer)), causal=True, epilogue=True,
                            lambda_init_value=oracle.lambda_init(cfg.layer), rows=rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert maxerr(got, ref) <= TOL_BF16
    # the planted needle gives the probe row a logit gap near 8 in map 1
    d = cfg.d
    for h in range(cfg.H):
        p = int(x["needle_pos"][0, h])
        gap = float(host["q1"][0, -1, h] @ host["k1"][0, p, h]) / math.sqrt(d)
        assert abs(gap - cfg.needle_gap) < 0.1


def test_full_v1_decode_64k():
    cfg = W.V1_DECODE_64K
    note(f"full {cfg.name}: generating the 17.2 GB cache on the device")
    x = W.decode_inputs(cfg, device=DEV)
    lam = x["lam"].to(DEV)
    out = da.diffattn_decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], lam, epilogue=True,
                             lambda_init_value=cfg.lambda_init)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    pairs = [(0, 0), (cfg.B - 1, cfg.H - 1)] + [(int(b), int(h)) for b, h in
                                                 zip(rng.integers(0, cfg.B, 6), rng.integers(0, cfg.H, 6))]
    got = out.float().cpu().numpy()
    for b, h in pairs:
        ref = oracle.decode(x["q1"][b:b + 1, h:h + 1].float().cpu().numpy(),
                            x["q2"][b:b + 1, h:h + 1].float().cpu().numpy(),
                            x["k1"][b:b + 1, :, h:h + 1].float().cpu().numpy(),
                            x["k2"][b:b + 1, :, h:h + 1].float().cpu().numpy(),
                            x["v"][b:b + 1, :, h:h + 1].float().cpu().numpy(),
                            lam[h:h + 1].cpu().numpy(), epilogue=True,
                            lambda_init_value=cfg.lambda_init)
        assert maxerr(got[b, h], ref[0, 0]) <= TOL_BF16, (b, h)
    del x
    torch.cuda.empty_cache()


def test_full_v2_8k():
    cfg = W.V2_GQA_8K
    x = W.v2_inputs(cfg, device=DEV)
    note(f"full {cfg.name}")
    out = da.diffattn_v2_fwd(x["q"], x["k"], x["v"], x["lam"], causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(np.random.default_rng(3), cfg.B, cfg.hq // 2, cfg.N, _boundary_rows(cfg.N), 2)
    ref = oracle.v2_forward(*(x[k].float().cpu().numpy() for k in ("q", "k", "v")),
                            x["lam"].cpu().numpy(), causal=True, rows=rows)
    got = out.float().cpu().numpy()[rows[:, 0], rows[:, 2], rows[:, 1]]
    assert maxerr(got, ref) <= TOL_BF16


def test_full_v2_decode_64k():
    cfg = W.V2_DECODE_64K
    note(f"full {cfg.name}: generating the 8.6 GB cache on the device")
    x = W.v2_decode_inputs(cfg, device=DEV)
    lam = x["lam"].to(DEV)
    out = da.diffattn_v2_decode(x["q"], x["k"], x["v"], lam)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    h = cfg.hq // 2
    pairs = [(0, 0), (cfg.B - 1, h - 1)] + [(int(b), int(p)) for b, p in
                                             zip(rng.integers(0, cfg.B, 6), rng.integers(0, h, 6))]
    got = out.float().cpu().numpy()
    group = cfg.hq // cfg.hkv
    for b, p in pairs:
        g = (2 * p) // group
        # the pair's KV head only: query heads 2p, 2p+1 of one group read KV head g
        ref = oracle.v2_decode(x["q"][b:b + 1, 2 * p:2 * p + 2].float().cpu().numpy(),
                               x["k"][b:b + 1, :, g:g + 1].float().cpu().numpy(),
                               x["v"][b:b + 1, :, g:g + 1].float().cpu().numpy(),
                               lam[b:b + 1, p:p + 1].cpu().numpy())
        assert maxerr(got[b, p], ref[0, 0]) <= TOL_BF16, (b, p)
    del x
    torch.cuda.empty_cache()
