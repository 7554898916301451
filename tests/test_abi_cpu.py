"""The C ABI without a GPU: the library loads, exports every declared symbol, and every invalid
argument is rejected with its status code before any HIP call (so these run on a CPU-only host)."""
import ctypes
import math
import os
import re

import pytest

import differential_softmax_attention_amd as da
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T = da.Tensor
FAKE = 0x10000          # never dereferenced: each call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(da.LIB_PATH):
        from differential_softmax_attention_amd import build
        build.build()
    return da.lib()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "diffattn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(da.EXPORTED), declared
    for name in declared:
        assert hasattr(L, name), name
    assert L.diffattn_version() >= 100


def test_lambda_init_matches_schedule(L):
    for layer in (1, 2, 4, 8, 12, 16, 24, 28):
        assert da.lambda_init(layer) == pytest.approx(oracle.lambda_init(layer), abs=1e-15)
    assert math.isnan(da.lambda_init(0))


def _t(ptr=FAKE, sb=0, ss=0, sh=0):
    return T(ptr, sb, ss, sh)


def _fwd(L, dtype=1, tensors=None, B=1, H=1, Nq=4, Nk=4, d=64, dv=128, lam=FAKE, li=0.8, causal=1,
         epi=1, w=None, eps=1e-5, scale=0.0):
    ts = tensors or [_t(FAKE, 4096, 512, 64) for _ in range(6)]
    return L.diffattn_fwd(dtype, ts[0], ts[1], ts[2], ts[3], ts[4], B, H, Nq, Nk, d, dv, lam, li, causal,
                          epi, w, eps, scale, ts[5], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), da.DIFFATTN_ERR_ARG),
    (dict(lam=None), da.DIFFATTN_ERR_ARG),
    (dict(B=0), da.DIFFATTN_ERR_ARG),
    (dict(Nq=0), da.DIFFATTN_ERR_ARG),
    (dict(d=0), da.DIFFATTN_ERR_ARG),
    (dict(dv=-1), da.DIFFATTN_ERR_ARG),
    (dict(Nq=8, Nk=4, causal=1), da.DIFFATTN_ERR_ARG),
    (dict(epi=5), da.DIFFATTN_ERR_ARG),
    (dict(eps=float("nan")), da.DIFFATTN_ERR_ARG),
    (dict(eps=-1.0), da.DIFFATTN_ERR_ARG),
    (dict(li=float("inf")), da.DIFFATTN_ERR_ARG),
    (dict(scale=float("nan")), da.DIFFATTN_ERR_ARG),
    (dict(d=300), da.DIFFATTN_ERR_UNSUPPORTED),
    (dict(dv=1024), da.DIFFATTN_ERR_UNSUPPORTED),
    (dict(H=70000), da.DIFFATTN_ERR_ARG),
])
def test_fwd_rejects(L, kw, status):
    assert _fwd(L, **kw) == status
    assert L.diffattn_last_error().decode() != ""


def test_fwd_rejects_bad_tensors(L):
    good = [_t(FAKE, 4096, 512, 64) for _ in range(6)]
    for i in range(6):
        ts = list(good)
        ts[i] = _t(0, 4096, 512, 64)                       # null
        assert _fwd(L, tensors=ts) == da.DIFFATTN_ERR_ARG
        ts[i] = _t(FAKE + 1, 4096, 512, 64)                # bf16 element misaligned
        assert _fwd(L, tensors=ts) == da.DIFFATTN_ERR_ARG
        ts[i] = _t(FAKE + 2, 4096, 512, 64)                # fp32 element misaligned
        assert _fwd(L, dtype=0, tensors=ts) == da.DIFFATTN_ERR_ARG
        ts[i] = _t(FAKE, 4096, -512, 64)                   # negative stride
        assert _fwd(L, tensors=ts) == da.DIFFATTN_ERR_ARG
    assert "q1" in (_fwd(L, tensors=[_t(0)] + good[1:]) and L.diffattn_last_error().decode())


def _decode(L, B=2, H=2, Lc=100, d=64, dv=128, ws=FAKE, ws_bytes=1 << 30, epi=1, lens=None, lam=FAKE):
    ts = [_t(FAKE, 4096, 512, 64) for _ in range(6)]
    return L.diffattn_decode(1, ts[0], ts[1], ts[2], ts[3], ts[4], lens, B, H, Lc, d, dv, lam, 0.8, epi,
                             None, 1e-5, 0.0, ts[5], ws, ws_bytes, None)


def test_decode_rejects(L):
    assert _decode(L, Lc=0) == da.DIFFATTN_ERR_ARG
    assert _decode(L, B=0) == da.DIFFATTN_ERR_ARG
    assert _decode(L, lam=None) == da.DIFFATTN_ERR_ARG
    assert _decode(L, epi=3) == da.DIFFATTN_ERR_ARG
    need = L.diffattn_decode_workspace_size(2, 2, 100, 128)
    assert need > 0
    assert _decode(L, ws_bytes=need - 1) == da.DIFFATTN_ERR_WORKSPACE
    assert _decode(L, ws=None) == da.DIFFATTN_ERR_ARG
    assert _decode(L, ws=FAKE + 16) == da.DIFFATTN_ERR_ARG     # not 256-byte aligned
    assert _decode(L, d=512) == da.DIFFATTN_ERR_UNSUPPORTED


def test_decode_workspace_size(L):
    assert L.diffattn_decode_workspace_size(0, 16, 100, 128) == 0
    assert L.diffattn_decode_workspace_size(32, 16, 0, 128) == 0
    small = L.diffattn_decode_workspace_size(1, 1, 1, 128)
    big = L.diffattn_decode_workspace_size(32, 16, 65536, 128)
    assert 0 < small < big < 64 << 20      # partials only: a few MB even for a 17 GB cache


def _decode_noalloc(L, B=2, H=2, Lc=100, d=64, dv=128, epi=1, lens=None, lam=FAKE, dtype=1):
    ts = [_t(FAKE, 4096, 512, 64) for _ in range(6)]
    return L.diffattn_decode_noalloc(dtype, ts[0], ts[1], ts[2], ts[3], ts[4], lens, B, H, Lc, d, dv, lam, 0.8, epi,
                                     None, 1e-5, 0.0, ts[5], None)


def test_decode_noalloc_rejects_before_any_hip_call(L):
    assert _decode_noalloc(L, Lc=0) == da.DIFFATTN_ERR_ARG
    assert _decode_noalloc(L, lam=None) == da.DIFFATTN_ERR_ARG
    assert _decode_noalloc(L, dtype=9) == da.DIFFATTN_ERR_ARG
    assert _decode_noalloc(L, d=512) == da.DIFFATTN_ERR_UNSUPPORTED
    # beyond the library's scratch: a clear ERR_WORKSPACE that names the limit
    assert _decode_noalloc(L, B=64, H=512, Lc=4096) == da.DIFFATTN_ERR_WORKSPACE
    msg = L.diffattn_last_error().decode()
    assert "diffattn_decode_noalloc" in msg and str(da.DECODE_NOALLOC_MAX_BYTES) in msg


def test_decode_noalloc_limit_covers_what_the_header_states(L):
    # every batch * heads up to 31,775 fits at any cache length; one more does not (at one split)
    lim = da.DECODE_NOALLOC_MAX_BYTES
    for bh in (1, 7, 100, 4095, 4097, 5000, 8000, 8191, 8192, 8193, 16384, 31775):
        for lc in (1, 255, 256, 257, 4096, 65536, 1 << 20):
            assert L.diffattn_decode_workspace_size(1, bh, lc, 128) <= lim, (bh, lc)
    assert L.diffattn_decode_workspace_size(1, 31776, 1 << 20, 128) > lim
    assert L.diffattn_decode_workspace_size(32, 16, 65536, 128) <= lim     # the 64K decode workload


def _v2(L, B=1, N=8, h=4, hkv=2, d=128, lam=FAKE, causal=1, dtype=1, scale=0.0, mode=0):
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(4)]
    return L.diffattn_v2_fwd(dtype, ts[0], ts[1], ts[2], lam, mode, B, N, h, hkv, d, causal, scale, ts[3], None)


def test_v2_rejects(L):
    assert _v2(L, hkv=3) == da.DIFFATTN_ERR_ARG          # 8 query heads into 3 groups
    assert _v2(L, h=3, hkv=2) == da.DIFFATTN_ERR_ARG     # groups of 3: a pair would straddle groups
    assert _v2(L, lam=None) == da.DIFFATTN_ERR_ARG
    assert _v2(L, N=0) == da.DIFFATTN_ERR_ARG
    assert _v2(L, d=512) == da.DIFFATTN_ERR_UNSUPPORTED
    assert _v2(L, dtype=9) == da.DIFFATTN_ERR_ARG
    assert _v2(L, mode=2) == da.DIFFATTN_ERR_ARG         # unknown lambda mode
    assert _v2(L, mode=-1) == da.DIFFATTN_ERR_ARG


def _v2dec(L, B=2, h=8, hkv=2, Lc=300, d=128, lam=FAKE, ws=FAKE, ws_bytes=1 << 30, dtype=1, lens=None, mode=1):
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(4)]
    return L.diffattn_v2_decode(dtype, ts[0], ts[1], ts[2], lens, lam, mode, B, h, hkv, Lc, d, 0.0, ts[3], ws,
                                ws_bytes, None)


def test_v2_decode_rejects(L):
    assert _v2dec(L, hkv=3) == da.DIFFATTN_ERR_ARG         # 16 query heads into 3 groups
    assert _v2dec(L, h=3, hkv=2) == da.DIFFATTN_ERR_ARG    # groups of 3 heads
    assert _v2dec(L, lam=None) == da.DIFFATTN_ERR_ARG
    assert _v2dec(L, Lc=0) == da.DIFFATTN_ERR_ARG
    assert _v2dec(L, B=0) == da.DIFFATTN_ERR_ARG
    assert _v2dec(L, dtype=9) == da.DIFFATTN_ERR_ARG
    need = L.diffattn_v2_decode_workspace_size(2, 8, 2, 300)
    assert need > 0
    assert _v2dec(L, ws_bytes=need - 1) == da.DIFFATTN_ERR_WORKSPACE
    assert _v2dec(L, ws=None) == da.DIFFATTN_ERR_ARG
    assert _v2dec(L, ws=FAKE + 64) == da.DIFFATTN_ERR_ARG      # not 256-byte aligned
    assert _v2dec(L, d=512) == da.DIFFATTN_ERR_UNSUPPORTED
    assert _v2dec(L, mode=5) == da.DIFFATTN_ERR_ARG


def test_v2_decode_workspace_size(L):
    assert L.diffattn_v2_decode_workspace_size(0, 32, 8, 100) == 0
    assert L.diffattn_v2_decode_workspace_size(1, 32, 8, 0) == 0
    assert L.diffattn_v2_decode_workspace_size(1, 3, 4, 100) == 0      # 6 heads do not split into 4
    small = L.diffattn_v2_decode_workspace_size(1, 1, 1, 1)
    big = L.diffattn_v2_decode_workspace_size(32, 32, 8, 65536)
    assert 0 < small < big < 64 << 20      # slice partials only


def _v2_slices(L, B, h, h_kv, Lc):
    """Cache slices per (batch, KV head) of the V2 decode, read back from its workspace size: one
    partial of 132 floats (shift, sum, two pad words, 128 channels) per slice and query head."""
    G = 2 * h // h_kv
    ws = L.diffattn_v2_decode_workspace_size(B, h, h_kv, Lc)
    per = B * h_kv * G * 132 * 4
    assert ws % per == 0, (ws, per)
    return ws // per


def test_v2_decode_slices_fill_whole_rounds(L):
    # 768 blocks resident at once (three per CU on a 256-CU device; the size query falls back to
    # that without a device): the slice count fills whole rounds of them with long slices
    assert _v2_slices(L, 32, 32, 8, 65536) == 3        # the 64K workload: 768 blocks, one round
    assert _v2_slices(L, 1, 4, 1, 65536) == 256        # one (batch, KV head): 256 slices of 8 tiles
    assert _v2_slices(L, 2, 32, 8, 65536) == 48        # 16 units x 48 = 768 blocks
    for B, h, h_kv, Lc in ((3, 8, 2, 300), (4, 8, 4, 3000), (1, 16, 1, 1), (32, 32, 8, 1000)):
        n = _v2_slices(L, B, h, h_kv, Lc)
        assert 1 <= n <= max(1, (Lc + 255) // 256), (B, h, h_kv, Lc, n)   # at least 8 tiles a slice


def _bwd(L, B=1, H=2, N=64, d=64, dv=128, dtype=1, lse=FAKE, maps=FAKE, lam=FAKE, ws=FAKE, ws_bytes=1 << 30, epi=1,
         causal=1, Nk=None):
    Nk = N if Nk is None else Nk
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(11)]
    return L.diffattn_bwd(dtype, *ts[:6], B, H, N, Nk, d, dv, lam, 0.8, causal, epi, None, 1e-5, 0.0, lse, maps,
                          *ts[6:], FAKE, FAKE, ws, ws_bytes, None)


def test_bwd_rejects(L):
    assert _bwd(L, lse=None) == da.DIFFATTN_ERR_ARG
    assert _bwd(L, maps=None) == da.DIFFATTN_ERR_ARG
    assert _bwd(L, maps=FAKE + 4) == da.DIFFATTN_ERR_ARG                 # maps not 16-byte aligned
    assert _bwd(L, lam=None) == da.DIFFATTN_ERR_ARG
    assert _bwd(L, N=0) == da.DIFFATTN_ERR_ARG
    assert _bwd(L, N=65, Nk=64) == da.DIFFATTN_ERR_ARG                   # causal with seq_q > seq_k
    assert _bwd(L, epi=7) == da.DIFFATTN_ERR_ARG
    need = L.diffattn_bwd_workspace_size(1, 2, 64)
    assert need > 0
    assert _bwd(L, ws_bytes=need - 1) == da.DIFFATTN_ERR_WORKSPACE
    assert _bwd(L, ws=FAKE + 32) == da.DIFFATTN_ERR_ARG
    assert _bwd(L, d=32) == da.DIFFATTN_ERR_UNSUPPORTED
    assert _bwd(L, dtype=0) == da.DIFFATTN_ERR_UNSUPPORTED               # fp32: no backward kernel
    assert L.diffattn_bwd_workspace_size(0, 2, 64) == 0


def _v2_bwd(L, lse=FAKE, maps=FAKE, lam=FAKE, dlam=FAKE, h=4, h_kv=2, d=128, seq=64, ws_bytes=1 << 30, ws=FAKE):
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(7)]
    return L.diffattn_v2_bwd(1, *ts[:4], lam, 0, 1, seq, h, h_kv, d, 1, 0.0, lse, maps, *ts[4:], dlam, ws, ws_bytes,
                             None)


def test_v2_bwd_rejects(L):
    for kw in ({"lse": None}, {"maps": None}, {"lam": None}, {"dlam": None}, {"seq": 0}, {"h_kv": 3},
               {"maps": FAKE + 4}, {"ws": FAKE + 32}):
        assert _v2_bwd(L, **kw) == da.DIFFATTN_ERR_ARG, kw
    need = L.diffattn_v2_bwd_workspace_size(1, 4, 64)
    assert need > 0
    assert _v2_bwd(L, ws_bytes=need - 1) == da.DIFFATTN_ERR_WORKSPACE
    assert _v2_bwd(L, d=64) == da.DIFFATTN_ERR_UNSUPPORTED


def test_fwd_train_rejects(L):
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(6)]
    call = lambda lse, maps, d=64, dtype=1: L.diffattn_fwd_train(dtype, *ts[:5], 1, 2, 64, 64, d, 128, FAKE, 0.8, 1,
                                                                 1, None, 1e-5, 0.0, ts[5], lse, maps, None)
    assert call(None, FAKE) == da.DIFFATTN_ERR_ARG
    assert call(FAKE, None) == da.DIFFATTN_ERR_ARG
    assert call(FAKE, FAKE + 4) == da.DIFFATTN_ERR_ARG                   # maps not 16-byte aligned
    assert call(FAKE, FAKE, d=32) == da.DIFFATTN_ERR_UNSUPPORTED
    assert call(FAKE, FAKE, dtype=0) == da.DIFFATTN_ERR_UNSUPPORTED


def _paged(L, v2=False, table=FAKE, bt_stride=4, num_pages=16, page=64, max_len=256, d=None, dtype=1, ws_bytes=1 << 30,
           ws=FAKE):
    if v2:
        d = 128 if d is None else d
        ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(4)]
        return L.diffattn_v2_decode_paged(dtype, ts[0], ts[1], ts[2], table, bt_stride, num_pages, page, None, FAKE, 0,
                                          2, 8, 2, max_len, d, 0.0, ts[3], ws, ws_bytes, None)
    d = 64 if d is None else d
    ts = [_t(FAKE, 1 << 20, 1024, 128) for _ in range(6)]
    return L.diffattn_decode_paged(dtype, *ts[:5], table, bt_stride, num_pages, page, None, 2, 4, max_len, d, 128,
                                   FAKE, 0.8, 1, None, 1e-5, 0.0, ts[5], ws, ws_bytes, None)


@pytest.mark.parametrize("v2", [False, True])
def test_paged_decode_rejects(L, v2):
    assert _paged(L, v2, table=None) == da.DIFFATTN_ERR_ARG
    assert _paged(L, v2, page=48) == da.DIFFATTN_ERR_ARG                 # not a multiple of 32
    assert _paged(L, v2, page=0) == da.DIFFATTN_ERR_ARG
    assert _paged(L, v2, num_pages=0) == da.DIFFATTN_ERR_ARG
    assert _paged(L, v2, bt_stride=3) == da.DIFFATTN_ERR_ARG             # 256 tokens need 4 pages of 64
    assert _paged(L, v2, max_len=0) == da.DIFFATTN_ERR_ARG
    assert _paged(L, v2, ws_bytes=16) == da.DIFFATTN_ERR_WORKSPACE
    assert _paged(L, v2, ws=FAKE + 32) == da.DIFFATTN_ERR_ARG
    assert _paged(L, v2, d=32) == da.DIFFATTN_ERR_UNSUPPORTED            # no paged generic kernel
    assert _paged(L, v2, dtype=0) == da.DIFFATTN_ERR_UNSUPPORTED


def test_lambda_bwd_rejects(L):
    assert L.diffattn_lambda_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, None) == da.DIFFATTN_ERR_ARG
    assert L.diffattn_lambda_bwd(FAKE, FAKE, FAKE, FAKE, None, 16, 64, FAKE, FAKE, FAKE, FAKE, None) == da.DIFFATTN_ERR_ARG


def test_lambda_rejects(L):
    assert L.diffattn_lambda(FAKE, FAKE, FAKE, FAKE, 0, 64, 12, FAKE, None) == da.DIFFATTN_ERR_ARG
    assert L.diffattn_lambda(FAKE, FAKE, FAKE, FAKE, 16, 0, 12, FAKE, None) == da.DIFFATTN_ERR_ARG
    assert L.diffattn_lambda(FAKE, FAKE, FAKE, FAKE, 16, 64, 0, FAKE, None) == da.DIFFATTN_ERR_ARG
    assert L.diffattn_lambda(None, FAKE, FAKE, FAKE, 16, 64, 12, FAKE, None) == da.DIFFATTN_ERR_ARG
    assert L.diffattn_lambda(FAKE, FAKE, FAKE, FAKE, 16, 64, 12, None, None) == da.DIFFATTN_ERR_ARG


def test_product_does_not_import_oracle():
    pkg = os.path.join(ROOT, "differential_softmax_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    src = f.read()
                assert "oracle" not in src, fn


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # the Python layer has no fallback: without the built library every call must raise
    monkeypatch.setattr(da, "LIB_PATH", str(tmp_path / "libdiffattn.so"))
    monkeypatch.setattr(da, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        da.lib()
    with pytest.raises(RuntimeError, match="not built"):
        da.diffattn_bwd_workspace_size(1, 1, 1)


def test_host_tensors_refused():
    import torch
    # every pointer the library receives is dereferenced on the GPU: a host tensor must be
    # refused by the binding before any launch
    q = torch.zeros((1, 8, 4, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    lam = torch.zeros((1, 8, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="on the GPU"):
        da.diffattn_v2_fwd(q, k, k.clone(), lam, causal=True)
    with pytest.raises(ValueError, match="on the GPU"):
        da._dp(lam)
