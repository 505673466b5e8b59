"""Build libmla.so (HIP for gfx950) in-tree with hipcc.

    python -m paged_mla_decode_02_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libmla.so")
SYNC_LIB_PATH = os.path.join(HERE, "libmla_sync.so")
SOURCES = ["api.cpp", "pager.cpp", "sched.hip", "decode.hip", "decode_wide.hip", "decode_qkpv.hip", "combine.hip", "absorb.hip", "kv_append.hip", "sparse.hip",
           "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla.so)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the online-softmax rescale and the
            # epilogue scale them with VALU ops, and the AGPR form duplicates them
            "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile(src: str, build_dir: str, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + [f"-D{d}" for d in defines] + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib_path: str) -> str:
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> str:
    """libmla.so, and libmla_sync.so: the same library with every page transfer
    synchronous (MLA_SYNC_DEBUG), the reference the race test compares with."""
    variants = [(LIB_PATH, BUILD_DIR, ()), (SYNC_LIB_PATH, BUILD_DIR + "_sync", ("MLA_SYNC_DEBUG=1",))]
    jobs = []
    for _, bdir, defs in variants:
        os.makedirs(bdir, exist_ok=True)
        jobs += [(src, bdir, defs) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    for k, (lib_path, _, _) in enumerate(variants):
        _link(objs[k * n:(k + 1) * n], lib_path)
        if verbose:
            print(f"built {lib_path}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
