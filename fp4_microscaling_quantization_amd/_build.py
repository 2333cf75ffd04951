"""Build the gfx950 HIP library ``libfp4.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfp4.so")
SOURCES = ["api.cpp", "quantize.hip", "dequant.hip", "gemm.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fno-gpu-rdc",
    "-fno-fast-math",
    "-ffp-contract=fast-honor-pragmas",  # fp contract(off) regions stay unfused
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libfp4.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="fp4build") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def run(cmd):
            return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)

        with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
            results = list(ex.map(run, [[hipcc(), *compile_flags, *inc, "-c", "-o", o, s]
                                        for s, o in zip(srcs, objs)]))
        tmp = LIB + ".tmp%d" % os.getpid()
        results.append(run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
                       if all(r.returncode == 0 for r in results) else results[0])
        out = "\n".join(l for r in results for l in r.stdout.splitlines()
                        if "packed-fp32-ops" not in l)
        if any(r.returncode != 0 for r in results):
            raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB
