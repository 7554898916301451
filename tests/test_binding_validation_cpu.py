"""The Python binding checks every operand's shape, dtype and device against the others before it
takes a pointer or touches the library: the C ABI receives pointers and sizes only, so a short
operand would become out-of-bounds device reads and a short output out-of-bounds writes. Runs on
the CPU: the library is replaced by a function that fails the test if it is reached."""
import pytest
import torch

import differential_softmax_attention_amd as da

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


class Reached(Exception):
    """Raised in place of loading the library: the call got past argument validation."""


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def stand_in():
        raise Reached()
    monkeypatch.setattr(da, "lib", stand_in)


def passes_validation(fn):
    """A well-formed call gets past validation: it reaches the library or the GPU-pointer check."""
    try:
        fn()
    except Reached:
        return True
    except ValueError as e:
        return "expected a tensor on the GPU" in str(e)
    return False


def v1(B=2, N=40, Nk=None, H=3, d=64, dv=128, dt=bf):
    Nk = N if Nk is None else Nk
    z = lambda *s: torch.zeros(s, dtype=dt)
    return dict(q1=z(B, N, H, d), q2=z(B, N, H, d), k1=z(B, Nk, H, d), k2=z(B, Nk, H, d), v=z(B, Nk, H, dv),
                lam=torch.zeros(H, dtype=f32))


def call_fwd(**over):
    a = v1()
    a.update(over)
    return da.diffattn_fwd(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], a["lam"], out=a.get("out"),
                           norm_w=a.get("norm_w"))


def test_well_formed_call_passes_validation():
    assert passes_validation(call_fwd)


@pytest.mark.parametrize("over,match", [
    (dict(k2=torch.zeros(2, 39, 3, 64, dtype=bf)), "k2: expected shape"),
    (dict(q2=torch.zeros(2, 40, 2, 64, dtype=bf)), "q2: expected shape"),
    (dict(v=torch.zeros(2, 41, 3, 128, dtype=bf)), "v: expected shape"),
    (dict(k1=torch.zeros(2, 40, 3, 64, dtype=f32)), "k1: expected dtype"),
    (dict(v=torch.zeros(2, 40, 3, 128, dtype=f32)), "v: expected dtype"),
    (dict(lam=torch.zeros(2, dtype=f32)), "lam: expected a contiguous"),
    (dict(lam=torch.zeros(3, dtype=torch.float64)), "lam: expected a contiguous"),
    (dict(out=torch.zeros(2, 40, 3, 64, dtype=bf)), "out: expected shape"),
    (dict(out=torch.zeros(2, 40, 3, 128, dtype=f32)), "out: expected dtype"),
    (dict(norm_w=torch.zeros(64, dtype=f32)), "norm_w: expected a contiguous"),
    (dict(q1=torch.zeros(2, 40, 3, 64, dtype=torch.float16), q2=torch.zeros(2, 40, 3, 64, dtype=torch.float16)),
     "unsupported dtype"),
])
def test_fwd_rejects(over, match):
    with pytest.raises(ValueError, match=match):
        call_fwd(**over)


def test_fwd_train_and_lambda_variants():
    a = v1()
    with pytest.raises(ValueError, match="lam: expected"):
        da.diffattn_fwd_train(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], torch.zeros(4, dtype=f32))
    vec = torch.zeros(3, 64, dtype=f32)
    with pytest.raises(ValueError, match="lk2: expected float32"):
        da.diffattn_fwd_lambda(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], vec, vec, vec, torch.zeros(3, 32), 12)
    with pytest.raises(ValueError, match="lam_out"):
        da.diffattn_fwd_lambda(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], vec, vec, vec, vec, 12,
                               lam_out=torch.zeros(2, dtype=f32))
    with pytest.raises(ValueError, match="lk1: expected"):
        da.diffattn_lambda(vec, torch.zeros(3, 32, dtype=f32), vec, vec, 12)


def test_bwd_rejects():
    a = v1()
    dy = torch.zeros(2, 40, 3, 128, dtype=bf)
    lse = torch.zeros(2, 3, 40, 2, dtype=f32)
    maps = torch.zeros(2, 40, 3, 2, 128, dtype=f32)
    args = (a["q1"], a["q2"], a["k1"], a["k2"], a["v"])
    with pytest.raises(ValueError, match="dout: expected shape"):
        da.diffattn_bwd(*args, dy[:, :39], a["lam"], lse, maps)
    with pytest.raises(ValueError, match="lse: expected"):
        da.diffattn_bwd(*args, dy, a["lam"], lse[:, :2], maps)
    with pytest.raises(ValueError, match="maps: expected"):
        da.diffattn_bwd(*args, dy, a["lam"], lse, maps[..., :64])
    assert passes_validation(lambda: da.diffattn_bwd(*args, dy, a["lam"], lse, maps))
    with pytest.raises(ValueError, match="dlam: expected"):
        vec = torch.zeros(3, 64, dtype=f32)
        da.diffattn_lambda_bwd(vec, vec, vec, vec, torch.zeros(2, dtype=f32))


def test_decode_rejects():
    B, L, H = 2, 100, 3
    q = torch.zeros(B, H, 64, dtype=bf)
    k = torch.zeros(B, L, H, 64, dtype=bf)
    vc = torch.zeros(B, L, H, 128, dtype=bf)
    lam = torch.zeros(H, dtype=f32)
    with pytest.raises(ValueError, match="cache_lens: expected"):
        da.diffattn_decode(q, q, k, k, vc, lam, cache_lens=torch.zeros(B + 1, dtype=i32))
    with pytest.raises(ValueError, match="cache_lens: expected"):
        da.diffattn_decode(q, q, k, k, vc, lam, cache_lens=torch.zeros(B, dtype=torch.int64))
    with pytest.raises(ValueError, match="vc: expected shape"):
        da.diffattn_decode(q, q, k, k, vc[:, :, :2], lam)
    with pytest.raises(ValueError, match="k2c: expected shape"):
        da.diffattn_decode(q, q, k, k[:, :50], vc, lam)
    with pytest.raises(ValueError, match="out: expected shape"):
        da.diffattn_decode(q, q, k, k, vc, lam, out=torch.zeros(B, H, 64, dtype=bf))
    # paged: the table must cover every sequence
    pool = torch.zeros(10, 32, H, 64, dtype=bf)
    vpool = torch.zeros(10, 32, H, 128, dtype=bf)
    table = torch.zeros(B, 3, dtype=i32)
    with pytest.raises(ValueError, match="does not cover"):
        da.diffattn_decode_paged(q, q, pool, pool, vpool, table, lam, max_len=100)
    with pytest.raises(ValueError, match="does not cover"):
        da.diffattn_decode_paged(q, q, pool, pool, vpool, table[:1], lam, max_len=96)
    with pytest.raises(ValueError, match="v_pages: expected shape"):
        da.diffattn_decode_paged(q, q, pool, pool, vpool[:9], table, lam, max_len=96)


def test_v2_rejects():
    B, N, hq, hkv, d = 2, 50, 8, 2, 128
    q = torch.zeros(B, N, hq, d, dtype=bf)
    k = torch.zeros(B, N, hkv, d, dtype=bf)
    lam = torch.zeros(B, N, hq // 2, dtype=f32)
    with pytest.raises(ValueError, match="lam: expected"):
        da.diffattn_v2_fwd(q, k, k, lam[:, :, :3].contiguous())
    with pytest.raises(ValueError, match="k: expected shape"):
        da.diffattn_v2_fwd(q, k[:, :49], k[:, :49], lam)
    with pytest.raises(ValueError, match="v: expected shape"):
        da.diffattn_v2_fwd(q, k, k[:, :, :1], lam)
    with pytest.raises(ValueError, match="out: expected shape"):
        da.diffattn_v2_fwd(q, k, k, lam, out=torch.zeros(B, N, hq, d, dtype=bf))
    dy = torch.zeros(B, N, hq // 2, d, dtype=bf)
    lse = torch.zeros(B, hq // 2, N, 2, dtype=f32)
    maps = torch.zeros(B, N, hq // 2, 2, d, dtype=f32)
    with pytest.raises(ValueError, match="maps: expected"):
        da.diffattn_v2_bwd(q, k, k, dy, lam, lse, maps[:1])
    qd = torch.zeros(B, hq, d, dtype=bf)
    kc = torch.zeros(B, 70, hkv, d, dtype=bf)
    with pytest.raises(ValueError, match="lam: expected"):
        da.diffattn_v2_decode(qd, kc, kc, torch.zeros(B, hq, dtype=f32))
    assert passes_validation(lambda: da.diffattn_v2_decode(qd, kc, kc, torch.zeros(B, hq // 2, dtype=f32)))


def test_fp8_rejects():
    x = torch.zeros(2, 40, 3, 64, dtype=bf)
    with pytest.raises(ValueError, match="x: expected dtype"):
        da.diffattn_quantize_fp8(x.float())
    with pytest.raises(ValueError, match="out: expected shape"):
        da.diffattn_quantize_fp8(x, out=torch.zeros(2, 40, 3, 32, dtype=torch.float8_e4m3fn))
    c = torch.zeros(2, 40, 3, 64, dtype=torch.float8_e4m3fn)
    s = torch.zeros(2, 3, dtype=f32)
    v = torch.zeros(2, 40, 3, 128, dtype=bf)
    lam = torch.zeros(3, dtype=f32)
    with pytest.raises(ValueError, match="sk2: expected"):
        da.diffattn_fwd_fp8(c, c, c, c, s, s, s, s[:1], v, lam)
    with pytest.raises(ValueError, match="v: expected dtype"):
        da.diffattn_fwd_fp8(c, c, c, c, s, s, s, s, v.float(), lam)
