"""Build libqb.so (HIP for gfx950) in-tree with hipcc.

Every source is compiled with round-to-nearest binary32 arithmetic kept exact:
no contraction of a*b+c into FMA (-ffp-contract=off; the kernels call fmaf
explicitly where a fused operation is meant), IEEE division and square root,
denormals kept, and packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqb.so")
# the two optimizer sources first: they take longest, and compile in parallel
SOURCES = ["qb_optim.hip", "qb_optim_uv.hip", "qb_tables.cpp", "qb_api.cpp", "qb_runtime.hip", "qb_quant.hip",
           "qb_dequant.hip", "qb_codes.hip", "qb_matmul.hip"]
ARCH = os.environ.get("QB_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _compile(src, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, src + ".o")
    cmd = [_hipcc(), *COMMON, *extra]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


STREAM_SRC = os.path.join(CSRC, "stream", "qb_stream.hip")
STREAM_LIB = os.path.join(HERE, "libqb_stream.so")


def build_stream(out=STREAM_LIB):
    """The benchmark's HBM reference streams (libqb_stream.so: copy, read,
    write), a library of their own: not part of libqb."""
    tmp = out + ".tmp"
    cmd = [_hipcc(), *COMMON, "-x", "hip", *DEVICE, "-shared", STREAM_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(jobs=None, out=LIB, extra=()):
    """Compile every source (always) and link the library (libqb.so by
    default; `extra` adds compiler flags); returns its path."""
    build_dir = BUILD if out == LIB else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, tuple(extra)), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    print(build_stream())
