"""Seeded synthetic inputs for the differential-attention workloads.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and lays them out; it holds none of the method's
arithmetic (no softmax, no lambda, no norm), so the oracle and the HIP path
each compute everything from these inputs on their own.

Recipe (all draws are torch fp32 normals or uniforms from a seeded
``torch.Generator``; bf16 inputs are those draws rounded to nearest-even by
``Tensor.to(torch.bfloat16)``):

  fp32 single head   N=64, d=8, dv=16, lambda 0.8, non-causal, no norm.
  V1 prefill 2K      B=4, H=16, N=2048, d=64, dv=128, causal. Lambda vectors
                     4 x [16, 64] ~ N(0, 0.1^2), layer 12. RMSNorm epilogue.
  V1 prefill 32K     B=1, H=16, N=32768, d=64, dv=128, causal, lambda vectors
                     all zero at layer 24 (so lambda = lambda_init(24)), and
                     one planted needle key per head: for a seeded position p
                     and the probe row r = N - 1,
                     K1[p] = D * sqrt(d) * Q1[r] / |Q1[r]|^2 with D = 8, which
                     gives the probe a logit gap of D over N(0,1) background
                     logits (the needle construction of "softmax can't say
                     zero, so it subtracts", section "Why softmax can't say
                     zero").
  V1 decode 64K      B=32, H=16, cache length 65536, d=64, dv=128; lambda per
                     head ~ U[0.2, 0.8]; lambda_init 0.8 for the rescale.
  V2 GQA 8K          B=2, N=8192, 64 query heads, 8 KV heads, d=128, causal,
                     lambda per token and pair ~ U[0, 1).

Large tensors are drawn on the device they are used on (``device=``), in
slices, so the decode cache (17.2 GB in bf16) never exists in fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class V1Config:
    name: str
    B: int
    H: int
    N: int
    d: int
    dv: int
    causal: bool
    epilogue: bool
    dtype: str            # "f32" or "bf16"
    seed: int
    layer: int = 0        # >0: lambda from the four vectors at this layer
    lam_fixed: float | None = None
    lam_vec_std: float = 0.1
    lam_vec_zero: bool = False
    needle_gap: float | None = None


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    L: int
    d: int
    dv: int
    seed: int
    lam_lo: float = 0.2
    lam_hi: float = 0.8
    lambda_init: float = 0.8


@dataclass(frozen=True)
class V2Config:
    name: str
    B: int
    N: int
    hq: int               # query heads (2h)
    hkv: int
    d: int
    causal: bool
    seed: int


@dataclass(frozen=True)
class V2DecodeConfig:
    name: str
    B: int
    L: int
    hq: int               # query heads (2h)
    hkv: int
    d: int
    seed: int


FP32_SINGLE_HEAD = V1Config("fp32 single head N=64 d=8 dv=16", B=1, H=1, N=64, d=8, dv=16,
                            causal=False, epilogue=False, dtype="f32", seed=1, lam_fixed=0.8)
V1_PREFILL_2K = V1Config("V1 prefill B=4 H=16 N=2048 d=64 dv=128 causal", B=4, H=16, N=2048, d=64,
                         dv=128, causal=True, epilogue=True, dtype="bf16", seed=2, layer=12)
V1_PREFILL_32K = V1Config("V1 prefill B=1 H=16 N=32768 d=64 dv=128 causal needle D=8", B=1, H=16,
                          N=32768, d=64, dv=128, causal=True, epilogue=True, dtype="bf16", seed=3,
                          layer=24, lam_vec_zero=True, needle_gap=8.0)
V1_DECODE_64K = DecodeConfig("V1 decode B=32 H=16 L=65536 d=64 dv=128", B=32, H=16, L=65536, d=64,
                             dv=128, seed=4)
V2_GQA_8K = V2Config("V2 GQA prefill B=2 N=8192 64q/8kv heads d=128 causal", B=2, N=8192, hq=64,
                     hkv=8, d=128, causal=True, seed=5)
# V2 decode: the V2 prefill's head layout against a 64K cache per sequence (as the V1 decode)
V2_DECODE_64K = V2DecodeConfig("V2 decode B=32 L=65536 64q/8kv heads d=128", B=32, L=65536, hq=64,
                               hkv=8, d=128, seed=6)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, dtype, chunk_dim0=False):
    if not chunk_dim0:
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
    out = torch.empty(shape, device=device, dtype=dtype)
    for i in range(shape[0]):
        out[i] = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32).to(dtype)
    return out


def v1_inputs(cfg: V1Config, device="cpu", B=None, N=None) -> dict:
    """Q1, Q2, K1, K2: [B, N, H, d]; V: [B, N, H, dv]; lambda vectors [H, d] x 4 (or a fixed lambda)."""
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    g = _gen(cfg.seed, device)
    q1 = _normal((B, N, cfg.H, cfg.d), g, device, dt)
    q2 = _normal((B, N, cfg.H, cfg.d), g, device, dt)
    k1 = _normal((B, N, cfg.H, cfg.d), g, device, dt)
    k2 = _normal((B, N, cfg.H, cfg.d), g, device, dt)
    v = _normal((B, N, cfg.H, cfg.dv), g, device, dt)
    out = dict(q1=q1, q2=q2, k1=k1, k2=k2, v=v)
    if cfg.lam_fixed is not None:
        out["lam_fixed"] = torch.full((cfg.H,), float(cfg.lam_fixed), dtype=torch.float32)
    else:
        shp = (cfg.H, cfg.d)
        if cfg.lam_vec_zero:
            lv = [torch.zeros(shp, dtype=torch.float32) for _ in range(4)]
        else:
            gl = _gen(cfg.seed + 1000, "cpu")
            lv = [torch.randn(shp, generator=gl, dtype=torch.float32) * cfg.lam_vec_std
                  for _ in range(4)]
        out.update(lq1=lv[0], lk1=lv[1], lq2=lv[2], lk2=lv[3], layer=cfg.layer)
    if cfg.needle_gap is not None:
        out["needle_pos"] = plant_needles(q1, k1, cfg.needle_gap, seed=cfg.seed + 2000)
    return out


def plant_needles(q1: torch.Tensor, k1: torch.Tensor, gap: float, seed: int) -> torch.Tensor:
    """Per (b, h): overwrite one key of map 1 so the last query sees it with logit gap ``gap``.

    K1[b, p, h] = gap * sqrt(d) * Q1[b, r, h] / |Q1[b, r, h]|^2, r = N - 1, p seeded in [0, N - 1).
    Computed in fp64 on the host and rounded to the tensor's dtype. Returns p as [B, H].
    """
    B, N, H, d = q1.shape
    gp = _gen(seed, "cpu")
    pos = torch.randint(0, N - 1, (B, H), generator=gp)
    qr = q1[:, N - 1].to("cpu", torch.float64)                    # [B, H, d]
    key = gap * math.sqrt(d) * qr / (qr * qr).sum(-1, keepdim=True)
    for b in range(B):
        for h in range(H):
            k1[b, int(pos[b, h]), h] = key[b, h].to(k1.dtype).to(k1.device)
    return pos


def decode_inputs(cfg: DecodeConfig, device="cpu", B=None, L=None) -> dict:
    """q1, q2: [B, H, d]; K1, K2 caches [B, L, H, d]; V cache [B, L, H, dv]; lambda [H]."""
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    dt = torch.bfloat16
    g = _gen(cfg.seed, device)
    q1 = _normal((B, cfg.H, cfg.d), g, device, dt)
    q2 = _normal((B, cfg.H, cfg.d), g, device, dt)
    k1 = _normal((B, L, cfg.H, cfg.d), g, device, dt, chunk_dim0=True)
    k2 = _normal((B, L, cfg.H, cfg.d), g, device, dt, chunk_dim0=True)
    v = _normal((B, L, cfg.H, cfg.dv), g, device, dt, chunk_dim0=True)
    gl = _gen(cfg.seed + 1000, "cpu")
    lam = cfg.lam_lo + (cfg.lam_hi - cfg.lam_lo) * torch.rand((cfg.H,), generator=gl,
                                                               dtype=torch.float32)
    return dict(q1=q1, q2=q2, k1=k1, k2=k2, v=v, lam=lam, lambda_init=cfg.lambda_init)


def v2_inputs(cfg: V2Config, device="cpu", B=None, N=None) -> dict:
    """q: [B, N, 2h, d]; k, v: [B, N, h_kv, d]; lambda [B, N, h] ~ U[0, 1)."""
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    dt = torch.bfloat16
    g = _gen(cfg.seed, device)
    q = _normal((B, N, cfg.hq, cfg.d), g, device, dt)
    k = _normal((B, N, cfg.hkv, cfg.d), g, device, dt)
    v = _normal((B, N, cfg.hkv, cfg.d), g, device, dt)
    lam = torch.rand((B, N, cfg.hq // 2), generator=g, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, lam=lam)


def v2_decode_inputs(cfg: V2DecodeConfig, device="cpu", B=None, L=None) -> dict:
    """q: [B, 2h, d]; K, V caches [B, L, h_kv, d]; lambda [B, h] ~ U[0, 1)."""
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    dt = torch.bfloat16
    g = _gen(cfg.seed, device)
    q = _normal((B, cfg.hq, cfg.d), g, device, dt)
    k = _normal((B, L, cfg.hkv, cfg.d), g, device, dt, chunk_dim0=True)
    v = _normal((B, L, cfg.hkv, cfg.d), g, device, dt, chunk_dim0=True)
    gl = _gen(cfg.seed + 1000, "cpu")
    lam = torch.rand((B, cfg.hq // 2), generator=gl, dtype=torch.float32)
    return dict(q=q, k=k, v=v, lam=lam)


def scatter_to_pages(caches, page_size: int, seed: int, spare_pages: int = 3):
    """Lay contiguous caches [B, L, H, D] out as a shared page pool and a block table.

    Every sequence's pages take distinct pool slots in a seeded random order, plus a few spare
    slots that no table entry names, the layout a serving system's allocator leaves behind. Pool
    rows that hold no token (spare pages, the tail of a sequence's last page) are filled with
    seeded noise. ``caches`` is one tensor or a tuple of tensors that share the table; pools are
    built on the caches' device.
    Returns (pools [P, page_size, H, D] in the order given, block_table int32 [B, ceil(L / page_size)]).
    """
    single = isinstance(caches, torch.Tensor)
    caches = (caches,) if single else tuple(caches)
    B, L = caches[0].shape[:2]
    dev = caches[0].device
    per_seq = (L + page_size - 1) // page_size
    P = B * per_seq + spare_pages
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(P, generator=g)[:B * per_seq].to(torch.int32)
    gd = _gen(seed + 1, dev)
    pools = []
    for c in caches:
        tail = per_seq * page_size - L
        if tail:
            pad = torch.randn((B, tail) + tuple(c.shape[2:]), generator=gd, device=dev).to(c.dtype)
            c = torch.cat([c, pad], dim=1)
        pool = torch.empty((P, page_size) + tuple(c.shape[2:]), dtype=c.dtype, device=dev)
        pool.index_copy_(0, perm.to(dev).long(), c.reshape((B * per_seq, page_size) + tuple(c.shape[2:])))
        if spare_pages:
            used = torch.zeros(P, dtype=torch.bool)
            used[perm.long()] = True
            spare = torch.nonzero(~used).flatten().to(dev)
            pool[spare] = torch.randn((spare.numel(), page_size) + tuple(c.shape[2:]), generator=gd,
                                      device=dev).to(c.dtype)
        pools.append(pool)
    table = perm.reshape(B, per_seq).to(dev)
    return (pools[0] if single else tuple(pools)), table


def lambda_logits(shape, seed: int, device="cpu", std: float = 2.0) -> torch.Tensor:
    """DIFF V2 lambda logits (the projection W_lambda x before its sigmoid), fp32 ~ N(0, std^2):
    wide enough that some sigmoids saturate near 0 and 1."""
    return torch.randn(shape, generator=_gen(seed, "cpu"), dtype=torch.float32).mul_(std).to(device)
