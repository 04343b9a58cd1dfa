"""Builds libemb.so (HIP kernels + C-ABI host layer) for gfx950, in-tree.

    python -m dlrm_sparse_embedding_amd.build [-j JOBS]

Every translation unit is compiled by hipcc into an object under
``dlrm_sparse_embedding_amd/_build`` and linked into
``dlrm_sparse_embedding_amd/libemb.so``. The library's DT_NEEDED
``libamdhip64.so.7`` is resolved through an rpath to torch's bundled ROCm
runtime, so a process that also uses PyTorch holds exactly one HIP runtime.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libemb.so")

SOURCES = ["emb_api.cpp", "emb_plan.cpp", "k_init.hip", "k_forward.hip", "k_keys_sort.hip", "k_rle.hip",
           "k_reduce.hip", "k_atomic.hip", "k_pack.hip", "k_hash.hip", "k_probe.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          # never emit packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _torch_lib_dir() -> str | None:
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            d = os.path.join(os.path.dirname(spec.origin), "lib")
            if os.path.exists(os.path.join(d, "libamdhip64.so")):
                return d
    except Exception:
        pass
    return None


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall",
               "-x", "hip", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int = 8, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", LIB + ".tmp"]
    tl = _torch_lib_dir()
    if tl:
        link += [f"-Wl,-rpath,{tl}"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args()
    build(a.jobs)


if __name__ == "__main__":
    main()
