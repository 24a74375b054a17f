"""Builds libmce.so in-tree from csrc/ with hipcc for gfx950 only.

Every HIP translation unit is compiled with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).  The compiler's
per-kernel register/LDS/scratch remarks are kept in _build/resource_usage.txt
and summarised, one line per kernel, in profiles/kernel_resources.txt.
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
          "-Wall", "-Wshadow-all", "-Wno-unused-function", "-Wno-unknown-warning-option",
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


RESOURCE_TABLE = os.path.join(HERE, "..", "profiles", "kernel_resources.txt")


def resource_table(remarks):
    """Per-kernel registers, scratch, LDS and occupancy from the compiler's
    kernel-resource-usage remarks, one line per kernel (demangled)."""
    import re
    rows, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\S+) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    names = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows),
                           capture_output=True, text=True).stdout.splitlines()
    out = ["# Per-kernel resources of libmce.so, from the compiler's kernel-resource-usage",
           "# remarks (hipcc -O3 --offload-arch=gfx950 -Rpass-analysis=kernel-resource-usage).",
           "# Made by: python -c 'import __graft_entry__ as g; g.build()'",
           "# VGPR/AGPR per lane; scratch in bytes per lane (0 = no spill); LDS bytes per",
           "# workgroup; occupancy in waves per SIMD.",
           f"{'VGPR':>5} {'AGPR':>5} {'spillV':>6} {'scratch':>7} {'LDS':>7} {'occ':>3}  kernel"]
    for r, n in sorted(zip(rows, names), key=lambda t: t[1]):
        n = n.replace("mce::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        n = n.replace("mce::", "").split("(")[0] if "(" in n and "<" not in n.split("(")[0] else n.split("(mce::GemmArgs")[0]
        out.append(f"{r.get('VGPRs', '?'):>5} {r.get('AGPRs', '?'):>5} {r.get('VGPRs Spill', '?'):>6} "
                   f"{r.get('ScratchSize [bytes/lane]', '?'):>7} {r.get('LDS Size [bytes/block]', '?'):>7} "
                   f"{r.get('Occupancy [waves/SIMD]', '?'):>3}  {n}")
    return "\n".join(out) + "\n"


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    remarks = "\n".join(l for _, log in results for l in log.splitlines() if "remark" in l)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(remarks + "\n")
    os.makedirs(os.path.dirname(RESOURCE_TABLE), exist_ok=True)
    with open(RESOURCE_TABLE, "w") as f:
        f.write(resource_table(remarks))
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
