"""Build libqmatmul.so (the C-ABI library of HIP kernels for gfx950) in-tree.

Each source compiles to its own object in parallel (hipcc -c), then one link
step makes the shared library.  Every call compiles every source.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmatmul.so")
SOURCES = ["qmm_capi.cpp", "qmm_quant.hip", "qmm_gemv.hip", "qmm_gemv_row.hip", "qmm_gemm.hip", "qmm_gemm_q.hip",
           "qmm_dequant.hip", "qmm_ext.hip", "qmm_noalloc.hip", "qmm_gemv_b.hip", "qmm_gemv_emit.hip", "qmm_gemv_reg.hip",
           "qmm_gemm_s.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# rocBLAS: the plain f32 GEMM of the dequantize-all form
LIBS = ["-L/opt/rocm/lib", "-lrocblas", "-Wl,-rpath,/opt/rocm/lib"]


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "is not a recognized feature" not in l)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode, _filter(r.stdout)


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    for (rc, out), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, *LIBS, "-o", LIB + ".tmp"], verbose)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
