"""diffattn_decode_noalloc, the decode entry point that allocates nothing (its split partials go to
the library's own per-GPU scratch array), against diffattn_decode with a caller's workspace: the
same kernels, so the outputs must be bit-identical, and both within the bf16 bound of the fp64
oracle. Two calls in a row, the second on smaller inputs, so the scratch holds the first call's
partials when the second runs."""
import numpy as np
import pytest
import torch

import differential_softmax_attention_amd as da
import oracle
from tolerances import FWD_BF16_ABS

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def note(msg):
    print(f"[case] {msg}", flush=True)


def inputs(B, H, L, seed, lens=None):
    g = torch.Generator(device=DEV).manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=g, device=DEV).to(torch.bfloat16)
    x = dict(q1=r(B, H, 64), q2=r(B, H, 64), k1=r(B, L, H, 64), k2=r(B, L, H, 64), v=r(B, L, H, 128))
    x["lam"] = torch.linspace(0.2, 0.8, H, device=DEV)
    x["lens"] = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    return x


def both(x, epilogue):
    ref = da.diffattn_decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], cache_lens=x["lens"],
                             epilogue=epilogue)
    out = torch.empty_like(ref)
    got = da.diffattn_decode_noalloc(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lam"], out, cache_lens=x["lens"],
                                     epilogue=epilogue)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return got, ref


def oracle_rows(x, pairs, epilogue):
    f = lambda t: t.double().cpu().numpy()
    lens = None if x["lens"] is None else x["lens"].cpu().numpy()
    return oracle.decode(f(x["q1"]), f(x["q2"]), f(x["k1"]), f(x["k2"]), f(x["v"]), x["lam"].cpu().numpy(),
                         cache_lens=lens, epilogue=epilogue, pairs=np.array(pairs))


def test_noalloc_equals_decode_two_calls_shrinking():
    cases = [(4, 16, 5000, None, True, 11), (2, 8, 1500, [1500, 733], False, 12)]
    for B, H, L, lens, epi, seed in cases:
        note(f"noalloc decode B={B} H={H} L={L} lens={lens} epilogue={epi}")
        x = inputs(B, H, L, seed, lens)
        got, ref = both(x, epi)
        assert torch.equal(got, ref)
        pairs = [(0, 0), (B - 1, H - 1), (B // 2, H // 3)]
        want = oracle_rows(x, pairs, epi)
        for n, (b, h) in enumerate(pairs):
            assert np.max(np.abs(got[b, h].double().cpu().numpy() - want[n])) <= FWD_BF16_ABS, (b, h)


def test_noalloc_at_the_64k_workloads_split_shape():
    # batch 32 x 16 heads: the 64K decode workload's grid (16 splits of each (batch, head), 8.65 MB
    # of partials), on a shorter cache
    note("noalloc decode B=32 H=16 L=8192")
    x = inputs(32, 16, 8192, 13)
    got, ref = both(x, True)
    assert torch.equal(got, ref)
    # and again after a smaller call, so the scratch starts from another call's partials
    y = inputs(3, 5, 700, 14, lens=[700, 1, 333])
    g2, r2 = both(y, True)
    assert torch.equal(g2, r2)
    got, ref = both(x, True)
    assert torch.equal(got, ref)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    x = inputs(1, 1, 1, 15)     # one cached token, expanded (stride 0) to the large shape
    big = dict(q1=x["q1"].expand(64, 512, 64), q2=x["q2"].expand(64, 512, 64),
               k1=x["k1"].expand(64, 4096, 512, 64), k2=x["k2"].expand(64, 4096, 512, 64),
               v=x["v"].expand(64, 4096, 512, 128))
    out = torch.empty((64, 512, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(da.DiffAttnError, match="ERR_WORKSPACE"):
        da.diffattn_decode_noalloc(big["q1"], big["q2"], big["k1"], big["k2"], big["v"],
                                   torch.zeros(512, device=DEV), out)
