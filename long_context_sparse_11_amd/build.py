"""Build the HIP library ``libcsa.so`` in-tree for gfx950.

Every source under csrc/ is compiled to an object in parallel (objects in
_build/ at the repository root), then linked into
long_context_sparse_11_amd/libcsa.so.  Run ``python -m
long_context_sparse_11_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
SOURCES = ["abi.hip", "compress.hip", "indexer.hip", "topk.hip", "attn.hip", "mxfp4.hip",
           "kvfp8.hip", "oproj.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed fp32 ops stay disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# attention keeps its output accumulators in ordinary VGPRs (MFMA VGPR form):
# the online-softmax rescale touches them with VALU ops, and the AGPR form
# made the allocator shuttle them between register files on every tile
SOURCE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = True, extra_flags: list[str] | None = None) -> str:
    os.makedirs(OBJ, exist_ok=True)
    flags = FLAGS + list(extra_flags or [])
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "csa.h")]

    def compile_one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        rc, out = _run([HIPCC, *flags, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                        "-o", obj])
        return src, obj, rc, out

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    failed = [r for r in results if r[2] != 0]
    for src, _, rc, out in results:
        if verbose and out.strip():
            print(f"[{src}]\n{out}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP compile failed: " + ", ".join(r[0] for r in failed))
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
                    *[r[1] for r in results]])
    if rc != 0:
        raise RuntimeError("link failed:\n" + out)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(deps)} inputs", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
