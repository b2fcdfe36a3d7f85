"""Build the HIP library libmoe_mi355x.so in-tree for gfx950.

Every source under csrc/ is compiled by hipcc to an object under _build/ (in
parallel), then linked into mixture_experts_layer_39_amd/libmoe_mi355x.so.
Usage:  python -m mixture_experts_layer_39_amd.build  [--jobs N]
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
ARCH = "gfx950"

# -packed-fp32-ops off: no packed fp32 VALU instructions are generated.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Kernels that must not use scratch memory.  decode_kernel separates its
# phases with grid barriers, so every workgroup must be resident at once, and
# scratch allocation can limit how many are; a variant of it that spilled to
# scratch also computed its second Linear wrongly (with every barrier met).
# The large-tile GEMM keeps its tile state in registers; scratch there means
# part of it went to memory, which costs that kernel a large part of its speed.
NO_SCRATCH = {"decode.hip": ("decode_kernel",), "grouped_gemm.hip": ("gemm_bf16_big_kernel",)}


def _scratch_sizes(remarks):
    """Kernel name -> ScratchSize from hipcc's kernel-resource-usage remarks."""
    sizes, name = {}, None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].split()[0]
        elif name and "ScratchSize [bytes/lane]:" in line:
            sizes[name] = int(line.split("ScratchSize [bytes/lane]:", 1)[1].split()[0])
    return sizes


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    guarded = NO_SCRATCH.get(os.path.basename(src), ())
    extra = ["-Rpass-analysis=kernel-resource-usage"] if guarded else []
    cmd = [hipcc()] + FLAGS + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    msgs = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l
                     and not l.lstrip().startswith(("|", "^")) and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    for kern, size in _scratch_sizes(out).items():
        if any(g in kern for g in guarded) and size > 0:
            raise RuntimeError(f"{kern} in {src} uses {size} bytes of scratch per lane; it must use none")
    return obj, msgs


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, msgs in ex.map(_compile, srcs):
            objs.append(obj)
            if verbose and msgs.strip():
                print(msgs)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
