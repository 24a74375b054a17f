"""Builds libmce.so in-tree from csrc/ with hipcc for gfx950 only.

Every HIP translation unit is compiled with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The per-kernel
register/LDS/scratch report of the compiler is kept in
_build/resource_usage.txt.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libmce.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unknown-warning-option",
          f"-I{os.path.join(HERE, '..', 'include')}"]


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-Rpass-analysis=kernel-resource-usage",
           "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for _, log in results:
            f.write("\n".join(l for l in log.splitlines() if "remark" in l))
            f.write("\n")
    tmp = LIB_PATH + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel whose host-side launch
    # stub the compiler did not emit) fails the build instead of the load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(LIB_PATH, flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
