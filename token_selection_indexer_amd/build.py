"""Build the HIP library token_selection_indexer_amd/liblsa.so for gfx950 (in-tree).

Every translation unit under csrc/ is compiled by hipcc in parallel and linked into one shared
object that exports only the C ABI of include/lsa.h.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblsa.so")
SOURCES = ["api.hip", "score.hip", "topk.hip", "pages.hip", "attn.hip", "attn_bwd.hip",
           "index_bwd.hip"]
ARCH = os.environ.get("LSA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         # packed fp32 VALU ops are kept out of the device code on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]


# per-file extras: the scoring kernels keep their MFMA accumulators in VGPRs (their epilogue
# reads every accumulator with VALU instructions; AGPR-resident results would each need a copy)
# the page keys are defined with separately rounded multiplies and adds: no FMA contraction
# the backward kernels add their gradients with the hardware's fp32 atomics (device memory)
EXTRA = {"score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "pages.hip": ["-ffp-contract=off"],
         "attn_bwd.hip": ["-munsafe-fp-atomics"], "index_bwd.hip": ["-munsafe-fp-atomics"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in x)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
