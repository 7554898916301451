"""Build libdiffattn.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Each source is compiled to an object under ``_build/`` (in parallel), then linked into
``differential_softmax_attention_amd/libdiffattn.so``.
"""
import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdiffattn.so")

SOURCES = ["diffattn_api.cpp", "generic_kernel.hip", "fwd_mfma.hip", "fwd_mfma_long.hip", "decode.hip", "decode_v2.hip", "bwd.hip", "bwd_v2.hip", "quant_fp8.hip", "lambda_kernel.hip", "probe.hip"]
HEADERS = ["common.hpp", "kernels.hpp", "mfma_tile.hpp", "bwd_tile.hpp", "fwd_mfma_kernel.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]
# Per-source additions. The dK/dV backward kernel runs one wave per SIMD with ~320 live
# registers; left to itself the compiler gives its MFMA accumulators the AGPR form and then
# copies them to VGPRs around every element-wise step. The VGPR form keeps them in place. The V2
# decode's output accumulators are scaled by VALU on its rare shift path, which in the AGPR form
# costs 64 AGPR-to-VGPR copies on every tile.
SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form=1"] for src in ("bwd.hip", "bwd_v2.hip", "decode_v2.hip")}
# The forward kernels a second time under the max-ilp schedule, which the launches use from 4096 keys.
SOURCE_FLAGS["fwd_mfma_long.hip"] = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = CFLAGS + SOURCE_FLAGS.get(src, [])
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdiffattn.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
