"""fp8 attention logits on the GPU: the library's dynamic absmax e4m3 quantisation must give the
oracle's codes and scales bit for bit (the codes are integer results), and the fp8 forward must
match the oracle's forward over the oracle's own dequantised operands (bf16 tolerance 2e-2)."""
import sys

import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def rand(shape, seed, scale=1.0):
    return (torch.randn(shape, generator=torch.Generator().manual_seed(seed)) * scale).to(torch.bfloat16).to(DEV)


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def gpu_codes(x):
    codes, s, amax = da.diffattn_quantize_fp8(x)
    torch.cuda.synchronize()
    return codes.view(torch.uint8).cpu().numpy(), s.cpu().numpy(), amax.cpu().numpy()


@pytest.mark.parametrize("B,N,H,dim,seed", [(1, 1, 1, 2, 1), (2, 100, 3, 64, 2), (1, 333, 2, 128, 3),
                                             (1, 5000, 2, 128, 4),    # long slices: the multi-block path
                                             (4, 40, 64, 64, 5)])     # 256 slices: one block per slice
def test_quantize_codes_bit_exact(B, N, H, dim, seed):
    note(f"fp8 quantise B={B} N={N} H={H} dim={dim}")
    # slices of very different magnitudes, so small values fall into the subnormal codes
    mag = torch.logspace(-3, 2, H)
    x = (torch.randn((B, N, H, dim), generator=torch.Generator().manual_seed(seed)) * mag[None, None, :, None])
    x = x.to(torch.bfloat16)
    codes, s, amax = gpu_codes(x.to(DEV))
    rc, rs = oracle.quantize_fp8(x.float().numpy())
    assert np.array_equal(s, rs)
    assert np.array_equal(amax, np.max(np.abs(x.float().numpy()), axis=(1, 3)))
    assert np.array_equal(codes, rc)


def test_quantize_ties_zero_slice_and_extremes():
    # exact ties of e4m3 after the scaling (amax 448 gives scale 1), an all-zero slice, negative
    # zero and the largest magnitude
    vals = torch.tensor([448.0, -448.0, 1.0625, 1.1875, 2 ** -10, 3 * 2 ** -10, -0.0, 0.0, 2.5, -2.5, 7 * 2 ** -9,
                         1 / 3, 100.0, 255.0, 0.01, -0.3])
    x = torch.zeros((1, 4, 2, 8))
    x[0, :2, 0, :] = vals.reshape(2, 8)
    x = x.to(torch.bfloat16)
    codes, s, _ = gpu_codes(x.to(DEV))
    rc, rs = oracle.quantize_fp8(x.float().numpy())
    assert np.array_equal(s, rs) and s[0, 1] == 1.0
    assert np.array_equal(codes, rc)


def fp8_case(B, Nq, Nk, H, seed, causal, epilogue, qscale=1.0):
    q1, q2 = rand((B, Nq, H, 64), seed, qscale), rand((B, Nq, H, 64), seed + 1, qscale)
    k1, k2 = rand((B, Nk, H, 64), seed + 2), rand((B, Nk, H, 64), seed + 3)
    v = rand((B, Nk, H, 128), seed + 4)
    lam = torch.linspace(0.2, 0.9, H)
    note(f"fp8 forward B={B} Nq={Nq} Nk={Nk} H={H} causal={causal} epi={epilogue} qscale={qscale}")
    qs = [da.diffattn_quantize_fp8(t) for t in (q1, q2, k1, k2)]
    out = da.diffattn_fwd_fp8(qs[0][0], qs[1][0], qs[2][0], qs[3][0], qs[0][1], qs[1][1], qs[2][1], qs[3][1], v,
                              lam.to(DEV), causal=causal, epilogue=epilogue)
    torch.cuda.synchronize()
    # the oracle quantises the same bf16 inputs itself and runs the fp64 forward on the values
    deq = [oracle.dequantize_fp8(*oracle.quantize_fp8(t.float().cpu().numpy())) for t in (q1, q2, k1, k2)]
    ref = oracle.v1_forward(*deq, f64(v), lam.numpy(), causal=causal, epilogue=epilogue)
    return f64(out), ref


@pytest.mark.parametrize("N,causal,epilogue", [(1, True, True), (31, True, True), (100, False, True),
                                               (257, True, False), (300, True, True)])
def test_fp8_forward(N, causal, epilogue):
    out, ref = fp8_case(2, N, N, 2, 7000 + N, causal, epilogue)
    assert maxerr(out, ref) <= TOL_BF16


def test_fp8_forward_long_keys():
    # 4096 keys and more run the kernels' max-ilp build
    out, ref = fp8_case(1, 4100, 4100, 1, 7300, True, True)
    assert maxerr(out, ref) <= TOL_BF16


def test_fp8_forward_rectangular_and_large_logits():
    out, ref = fp8_case(1, 70, 200, 3, 7100, True, True)
    assert maxerr(out, ref) <= TOL_BF16
    out, ref = fp8_case(1, 150, 150, 2, 7200, True, True, qscale=8.0)
    assert maxerr(out, ref) <= TOL_BF16


def test_full_fp8_prefill_2k():
    # the V1 prefill workload (B=4, H=16, N=2048) with fp8 score operands, in the launch
    # configuration the benchmark times; sampled rows against the oracle
    cfg = W.V1_PREFILL_2K
    x = W.v1_inputs(cfg, device=DEV)
    lam = da.diffattn_lambda(*(x[k].to(DEV) for k in ("lq1", "lk1", "lq2", "lk2")), cfg.layer)
    li = da.lambda_init(cfg.layer)
    note(f"full fp8 {cfg.name}")
    qs = [da.diffattn_quantize_fp8(x[k]) for k in ("q1", "q2", "k1", "k2")]
    out = da.diffattn_fwd_fp8(qs[0][0], qs[1][0], qs[2][0], qs[3][0], qs[0][1], qs[1][1], qs[2][1], qs[3][1], x["v"],
                              lam, causal=True, epilogue=True, lambda_init_value=li)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    got = out.float().cpu().numpy()
    lam_np = lam.cpu().numpy()
    for b, h in ((0, 0), (cfg.B - 1, cfg.H - 1), (int(rng.integers(cfg.B)), int(rng.integers(cfg.H)))):
        sl = lambda t: t[b:b + 1, :, h:h + 1].float().cpu().numpy()
        deq = [oracle.dequantize_fp8(*oracle.quantize_fp8(sl(x[k]))) for k in ("q1", "q2", "k1", "k2")]
        rows = [0, 1, 31, 32, 1000, cfg.N - 1] + [int(r) for r in rng.integers(0, cfg.N, 4)]
        ref = oracle.v1_forward(*deq, sl(x["v"]).astype(np.float64), lam_np[h:h + 1], causal=True, epilogue=True,
                                lambda_init_value=li, rows=np.array([(0, 0, r) for r in rows]))
        assert maxerr(got[b, rows, h], ref) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("B,Nq,Nk,H", [(2, 100, 100, 3), (1, 40, 300, 2), (4, 2048, 2048, 16), (1, 5000, 5000, 2)])
def test_quantize_qk_equals_per_operand(B, Nq, Nk, H):
    # one call for the four operands (one launch when the slices fit in registers: the 2K
    # workload's shape; operand by operand otherwise) against diffattn_quantize_fp8 and the oracle
    g = torch.Generator(device=DEV).manual_seed(7000 + Nq + Nk)
    xs = [torch.randn((B, n, H, 64), generator=g, device=DEV).mul_(s).to(torch.bfloat16)
          for n, s in ((Nq, 1.0), (Nq, 3.0), (Nk, 0.5), (Nk, 20.0))]
    xs[1][0, :, 0] = 0.0                                       # an all-zero slice
    codes, scales, amax = da.diffattn_quantize_fp8_qk(*xs)
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        c1, s1, a1 = da.diffattn_quantize_fp8(x)
        torch.cuda.synchronize()
        assert torch.equal(codes[i].view(torch.uint8), c1.view(torch.uint8)), i
        assert torch.equal(scales[i], s1) and torch.equal(amax[i], a1), i
        if B * x.shape[1] <= 4 * 2048:
            rc, rs = oracle.quantize_fp8(x.float().cpu().numpy())
            assert np.array_equal(codes[i].view(torch.uint8).cpu().numpy(), rc), i
            assert np.array_equal(scales[i].cpu().numpy(), rs), i
