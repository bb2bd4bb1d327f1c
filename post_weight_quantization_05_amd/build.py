"""Build libgptq_mi355x.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m post_weight_quantization_05_amd.build   (or __graft_entry__.build())
Every .hip file under csrc/ is compiled to an object in _build/, then linked into
post_weight_quantization_05_amd/libgptq_mi355x.so. A build always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgptq_mi355x.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 VALU forms stay off (the compiler would otherwise form them from float2 code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# A test build of the same library in which every fp64 product takes the chunked-ring GEMM (the small-K and
# large-product kernels switched off) and the factorization forms L^-1 by the level-wise doubling at every size
# (the step-carried route's cutoff set to 0), so that parity tests cover those routes at small sizes too.
# Only these sources differ; the tests load it beside the main library.
VARIANT_LIB = os.path.join(PKG, "libgptq_mi355x_ringonly.so")
VARIANT_DEFS = {"dgemm.hip": ["-DGPTQ_DGEMM_SMALLK_TILES=0", "-DGPTQ_DGEMM_BIG=0"], "factor.hip": ["-DGPTQ_FACTOR_FILL_MAX=0"]}


def _compile(src: str, defs=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    cmd = [HIPCC, *CFLAGS, *defs, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    # hipcc's host pass does not know the packed-fp32 feature flag and says so; keep other warnings
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found; set HIPCC")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(VARIANT_DEFS))) as ex:
        objs_f = ex.map(_compile, srcs)
        var_f = {name: ex.submit(_compile, os.path.join(CSRC, name), defs, ".ringonly")
                 for name, defs in VARIANT_DEFS.items()}
        objs = list(objs_f)
        var_objs = {name: f.result() for name, f in var_f.items()}
    _link(objs, LIB)
    _link([var_objs.get(os.path.basename(o)[:-len(".o")], o) for o in objs], VARIANT_LIB)
    if verbose:
        print(f"built {LIB} (and the test build {os.path.basename(VARIANT_LIB)})")
    return LIB


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    # -Bsymbolic: calls between the library's own functions bind inside it, so the test build can be loaded
    # beside the main library in one process
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out)


if __name__ == "__main__":
    build()
