"""Compile the HIP extension (libmk.so) for gfx950, in-tree.

hipcc builds the device runtime (runtime.hip) and the host planner
(plan.cpp) into one shared library exporting the C ABI of include/mk.h.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")

# (source, extra defines): the device kernels are compiled once per
# (weight type, batch tile) so the instantiations build in parallel
UNITS = [("runtime.hip", []), ("plan.cpp", [])] + \
    [("kernels.hip", ["-DMK_WT_BF16", "-DMK_NB=%d" % nb]) for nb in (1, 2, 4, 8, 16)] + \
    [("kernels.hip", ["-DMK_WT_F32", "-DMK_NB=%d" % nb]) for nb in (1, 2, 4)] + \
    [("kernels.hip", ["-DMK_WT_BF16", "-DMK_NB=1", "-DMK_LDS_STREAM"])] + \
    [("kernels.hip", ["-DMK_WT_BF16", "-DMK_NB=%d" % nb, "-DMK_W4_KERNELS"]) for nb in (4, 8, 16)]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
# packed-FP32 instructions stay off on the device (plain float code only)
DEVICE = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Always recompiles (the build check must compile every time). At most
    `jobs` compiles run at once (0: one per CPU, at most 16)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = _hipcc()
    jobs = jobs if jobs > 0 else max(1, min(16, os.cpu_count() or 1))
    cmds = []
    objs = []
    for src, defs in UNITS:
        tag = "".join(d.replace("-D", "_").replace("=", "") for d in defs)
        obj = os.path.join(objdir, src + tag + ".o")
        objs.append(obj)
        if src.endswith(".hip"):
            cmd = [hipcc, "-c", os.path.join(CSRC, src), "-o", obj, "--offload-arch=" + ARCH] + COMMON + DEVICE + defs
        else:
            cmd = [hipcc, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
        cmds.append((src + tag, cmd))
    failed = []

    def finish(src, p):
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature flag
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))

    running = []
    for src, cmd in cmds:
        if len(running) >= jobs:
            finish(*running.pop(0))
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for src, p in running:
        finish(src, p)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
