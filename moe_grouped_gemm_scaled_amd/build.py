"""Build libdg.so (the HIP library) in-tree with hipcc for gfx950.

    python -m moe_grouped_gemm_scaled_amd.build

Every source is compiled ahead of time (no JIT); the object files go to
_build/ next to this file and the shared library to libdg.so beside it.
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdg.so")
SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "decode.hip", "pipelined.hip", "persistent.hip", "mqa.hip", "noalloc.hip", "stream.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 from the compiler.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(HERE, "..", "include")]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    t0 = time.time()
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + COMMON + lang + ["-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature: harmless noise
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and
                         "is not a recognized feature for this target" not in l)
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and text.strip():
            print(text, file=sys.stderr)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
