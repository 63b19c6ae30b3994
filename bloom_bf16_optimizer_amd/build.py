"""Builds the gfx950 shared libraries in-tree with hipcc.

* ``bloom_bf16_optimizer_amd/libbloomkern.so`` -- the kernels and their C ABI
  (``include/bloom_kernels.h``), from ``bloom_bf16_optimizer_amd/csrc``.
* ``synth/libbloomsynth.so`` -- the device side of the seeded input generator,
  and a plain streaming copy that ``bench.py`` times as the bandwidth ceiling.

Run ``python -m bloom_bf16_optimizer_amd.build`` (or ``__graft_entry__.build()``).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bloom_bf16_optimizer_amd")
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

LIB_KERNELS = os.path.join(PKG, "libbloomkern.so")
LIB_SYNTH = os.path.join(ROOT, "synth", "libbloomsynth.so")

# Packed FP32 instructions are kept out of every device build.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build")
    return exe


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *extra, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    kern_srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = []
    for s in kern_srcs:
        jobs.append((s, os.path.join(BUILD, "k_" + os.path.basename(s) + ".o"), []))
    synth_srcs = sorted(glob.glob(os.path.join(ROOT, "synth", "csrc", "*.hip")))
    for s in synth_srcs:
        jobs.append((s, os.path.join(BUILD, "s_" + os.path.basename(s) + ".o"), ["-ffp-contract=off"]))
    workers = min(8, os.cpu_count() or 4, len(jobs))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(_compile, s, o, e) for s, o, e in jobs]
        for f in futs:
            f.result()
    _link([o for s, o, _ in jobs if s not in synth_srcs], LIB_KERNELS)
    _link([o for s, o, _ in jobs if s in synth_srcs], LIB_SYNTH)
    if verbose:
        print(f"built {LIB_KERNELS}\nbuilt {LIB_SYNTH}")
    return [LIB_KERNELS, LIB_SYNTH]


if __name__ == "__main__":
    build()
    sys.exit(0)
