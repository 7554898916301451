"""The inline asm of the product meets the CDNA wait-state rules it relies on (tests/asm_hazards.py),
checked on the gfx950 assembly of every source that contains inline asm, built with the library's
own flags and again under a different instruction schedule (`-amdgpu-sched-strategy=max-ilp`, or
max-memory-clause for a source the library already builds under max-ilp):
the guards must hold wherever the compiler places the surrounding instructions, not only in
today's schedule. Runs on the CPU (hipcc cross-compiles for gfx950)."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

import asm_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_softmax_attention_amd", "csrc")


def _build_module():
    import importlib
    return importlib.import_module("differential_softmax_attention_amd.build")


def _asm_sources():
    """Sources whose text or included local headers hold inline asm."""
    b = _build_module()
    has_asm = {h for h in b.HEADERS if re.search(r"\basm\b", open(os.path.join(CSRC, h)).read())}
    out = []
    for src in b.SOURCES:
        if not src.endswith(".hip"):
            continue
        text = open(os.path.join(CSRC, src)).read()
        incs = set(re.findall(r'#include "([^"]+)"', text))
        # headers pull in headers: follow one level (mfma_tile.hpp via bwd_tile.hpp)
        for h in list(incs):
            if h in b.HEADERS:
                incs |= set(re.findall(r'#include "([^"]+)"', open(os.path.join(CSRC, h)).read()))
        if re.search(r"\basm\b", text) or (incs & has_asm):
            out.append(src)
    return out


SCHEDULES = {"default": [], "other": None}


def _schedule_flags(src, sched):
    """The build's own schedule, or another one: max-ilp, or max-memory-clause for a source that the
    build already compiles under max-ilp."""
    if sched == "default":
        return []
    own = " ".join(_build_module().SOURCE_FLAGS.get(src, []))
    strategy = "max-memory-clause" if "sched-strategy=max-ilp" in own else "max-ilp"
    return ["-mllvm", f"-amdgpu-sched-strategy={strategy}"]


def _assemble(src, sched, outdir):
    b = _build_module()
    out = os.path.join(outdir, f"{src}.{sched}.s")
    own = b.SOURCE_FLAGS.get(src, [])
    if sched != "default" and any("sched-strategy" in f for f in own):
        own = [f for f in own if f != "-mllvm" and "sched-strategy" not in f]
        own = [x for f in own for x in ("-mllvm", f)]
    cmd = [b.HIPCC, *b.CFLAGS, *own, *_schedule_flags(src, sched), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src} ({sched}):\n{r.stderr[-3000:]}")
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc is not installed")
    outdir = str(tmp_path_factory.mktemp("asm"))
    jobs = [(s, k) for s in _asm_sources() for k in SCHEDULES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        texts = list(ex.map(lambda j: _assemble(j[0], j[1], outdir), jobs))
    return dict(zip(jobs, texts))


def test_sources_with_inline_asm_are_found():
    srcs = _asm_sources()
    for s in ("fwd_mfma.hip", "fwd_mfma_long.hip", "bwd.hip", "bwd_v2.hip", "decode_v2.hip"):
        assert s in srcs


def test_product_inline_asm_meets_the_wait_states(assembly):
    total = 0
    problems = []
    for (src, sched), text in assembly.items():
        found, sites = H.check(text)
        total += sites
        problems += [f"[{src}, {sched}] {m}" for m in found]
    assert total > 1000, total          # every DMA and asm MFMA site of every instantiation was seen
    assert not problems, "\n".join(problems[:20])


# ---- the checker itself, on hand-written snippets --------------------------------------------

def _fn(body):
    return "k:\n" + "\n".join(body) + "\n.Lfunc_end0:\n"


def _dma(prefix=()):
    return [";;#ASMSTART", *prefix, "global_load_lds_dwordx4 v1, s[10:11]", ";;#ASMEND"]


def test_checker_dma_base_written_by_valu():
    bad = _fn(["v_readfirstlane_b32 s10, v4", "v_add_f32_e32 v2, v3, v2", *_dma()])
    assert len(H.check(bad)[0]) == 1
    ok = _fn(["v_readfirstlane_b32 s10, v4", *_dma(["s_nop 4"])])
    assert H.check(ok) == ([], 1)
    short = _fn(["v_readfirstlane_b32 s11, v4", *_dma(["s_nop 3"])])
    assert len(H.check(short)[0]) == 1
    far = _fn(["v_readfirstlane_b32 s10, v4", "s_nop 2", "v_mov_b32 v5, 0", "v_mov_b32 v6, 0", *_dma()])
    assert H.check(far)[0] == []


def test_checker_m0_and_branches():
    assert len(H.check(_fn(["s_mov_b32 m0, s3", *_dma()]))[0]) == 1
    assert H.check(_fn(["s_mov_b32 m0, s3", *_dma(["s_nop 0"])]))[0] == []
    # the write reaches the load through a branch: found on the path through the label
    looped = _fn(["v_readfirstlane_b32 s10, v4", "s_branch .LBB0_2", "s_nop 7", "s_nop 7",
                  ".LBB0_2:", *_dma()])
    assert len(H.check(looped)[0]) == 1
    # a loop back edge: the write at the loop's end precedes the load at its start
    back = _fn([".LBB0_1:", *_dma(), "s_nop 7", "v_readfirstlane_b32 s10, v4", "s_cbranch_scc1 .LBB0_1"])
    assert len(H.check(back)[0]) == 1


def test_checker_mfma_rules():
    asm_mfma = [";;#ASMSTART", "s_nop 1", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND"]
    assert H.check(_fn(["v_mov_b32 v3, 0", *asm_mfma, "s_nop 7", "s_nop 7", "s_nop 7"]))[0] == []
    no_nop = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]", ";;#ASMEND"]
    assert len(H.check(_fn(["v_mov_b32 v3, 0", *no_nop, "s_nop 7", "s_nop 7", "s_nop 7"]))[0]) == 1
    # reading the accumulator too soon, and after enough wait states
    assert len(H.check(_fn([*asm_mfma, "s_nop 7", "v_accvgpr_read_b32 v0, a3"]))[0]) == 1
    assert H.check(_fn([*asm_mfma, "s_nop 7", "s_nop 7", "s_nop 1", "v_accvgpr_read_b32 v0, a3"]))[0] == []
    # back-to-back accumulation into the same registers needs no wait
    assert H.check(_fn([*asm_mfma, *asm_mfma, "s_nop 7", "s_nop 7", "s_nop 7"]))[0] == []


def test_no_inline_float_constant_in_bf16_dot_operands(assembly):
    """v_dot2c_f32_bf16 reads an inline float constant as that float's 32-bit pattern (1.0 gives the
    bf16 pair {0, 1}), while the compiler folds the pair {1, 0} into the inline operand 1.0: the
    selector then picks the other weight of the pair. Packed bf16 operands stay in registers or
    literals."""
    bad = []
    for (src, sched), text in assembly.items():
        for line in text.splitlines():
            t = line.strip()
            if t.startswith(("v_dot2c_f32_bf16", "v_dot2_f32_bf16")):
                ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
                if any(re.fullmatch(r"-?\d+\.\d+", o) for o in ops[1:3]):
                    bad.append(f"[{src}, {sched}] {t}")
    assert not bad, "\n".join(bad[:10])
