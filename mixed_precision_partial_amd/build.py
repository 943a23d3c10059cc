"""Build the gfx950 shared library ``libmpp_ar.so`` in-tree with hipcc.

Every source compiles to an object of its own (in parallel: the kernel tables
are spread over several files), then one hipcc line links the library.

Usage:  python -m mixed_precision_partial_amd.build   (or build_library())
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmpp_ar.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# reference streaming kernels of the benchmark's ceilings (not part of the reduce)
CEILING_SRC = os.path.join(CSRC, "bench_ceiling.hip")
CEILING_LIB = os.path.join(HERE, "libmpp_ceiling.so")

OBJ_DIR = os.path.join(HERE, "_build")


def sources() -> list[str]:
    """Sources of the reduce library (the ceiling kernels build on their own)."""
    hip = [s for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if s != CEILING_SRC]
    return [os.path.join(CSRC, "ar_api.cpp")] + hip


HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # binary32 subnormals are results of the method, never flushed
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off",
    "-Wall",
]


# The non-residual streaming kernels' eight leading scalar parameters are
# preloaded into SGPRs at dispatch.  The residual and single-shot kernels read
# their arguments from the argument block (the leading parameters stay unused
# there), so their tables are built without preloading.
PRELOAD_FLAGS = ["-mllvm", "-amdgpu-kernarg-preload-count=8"]


def preload_flags(src: str) -> list[str]:
    name = os.path.basename(src)
    if name.startswith("ar_k_") and "_res" not in name and name != "ar_k_single.hip":
        return PRELOAD_FLAGS
    if src == CEILING_SRC:
        return PRELOAD_FLAGS
    return []


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


# hipcc's host pass does not know the packed-fp32 feature and says so; that is expected
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd: list[str]) -> tuple[int, list[str]]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l and l.strip()]
    return res.returncode, msgs


def build_library(out: str = LIB_PATH, verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources() + [CEILING_SRC]
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in srcs]
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    cmds = [[hipcc(), *HIPCC_FLAGS, *preload_flags(s), *inc, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(_run, cmds))
    failed = [(c, m) for c, (rc, m) in zip(cmds, results) if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join("\n".join(m) for _, m in failed))
    tmp = out + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs[:-1], "-o", tmp]
    ceil_link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", objs[-1], "-o", CEILING_LIB + ".tmp"]
    for cmd in (link, ceil_link):
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msgs = _run(cmd)
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    if verbose:
        for _, m in results:
            if m:
                print("\n".join(m), file=sys.stderr)
    os.replace(tmp, out)
    build_fast_call(verbose=verbose)
    return out


def build_fast_call(verbose: bool = False) -> str:
    """Compile csrc/ar_pycall.c (a CPython type holding one pre-converted call of the
    C ABI; no GPU code) with the host C compiler into _ar_fast<EXT_SUFFIX>."""
    import sysconfig

    src = os.path.join(CSRC, "ar_pycall.c")
    out = os.path.join(HERE, "_ar_fast" + sysconfig.get_config_var("EXT_SUFFIX"))
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-O2", "-shared", "-fPIC", "-Wall", "-Werror", f"-I{sysconfig.get_paths()['include']}", src,
           "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    rc, msgs = _run(cmd)
    if rc != 0:
        raise RuntimeError("building the fast-call module failed:\n" + "\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
