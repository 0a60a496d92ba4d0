"""Build libjetlong.so in-tree with hipcc for gfx950.

    python -m rope_context_extension_amd.build      (or build() from Python)

Every .hip file under csrc/ is compiled to an object in csrc/_build/ (in
parallel) and linked into rope_context_extension_amd/libjetlong.so.  Only the
jl_* entry points are exported (-fvisibility=hidden elsewhere).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libjetlong.so")
ARCH = os.environ.get("JL_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Per-source flags.  The decode kernels take their leading arguments in
# scalar registers at wave launch (kernel-argument preloading, at most 14
# dwords on gfx950): a decode step's first loads then wait for no load of a
# kernel argument.  The prefill kernels are scheduled with the compiler's
# ILP strategy, which orders the softmax phase's instructions (the matrix
# phases are pinned by scheduling barriers): results are bitwise the same,
# and a prefill call was about 0.4% faster on two boxes with the earlier
# two-launch kernels and 0.7% faster with the three-pass kernel (same-box
# A/B, 116.1 against 117.0 ms).  On the decode kernels it was slower
# at 128K keys, so they keep the default.
EXTRA = {
    "jl_decode.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=10"],
    "jl_prefill_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


# Every kernel keeps its state in registers and LDS: a kernel that spills
# VGPRs or puts arrays on the stack (scratch) runs many times slower (a
# restructured prefill kernel once took 704 bytes of stack per lane and ran
# at half speed), so the build reads the compiler's resource report and
# stops on either.
RESOURCE_REPORT = "-Rpass-analysis=kernel-resource-usage"


def _check_resources(src: str, report: str) -> None:
    kernel, bad = None, []
    for ln in report.splitlines():
        if "remark:" not in ln:
            continue
        msg = ln.split("remark:", 1)[1].split(" [-R", 1)[0].strip()
        if msg.startswith("Function Name:"):
            kernel = msg.split(":", 1)[1].strip()
        elif msg.startswith("ScratchSize") or msg.startswith("VGPRs Spill") or msg.startswith("SGPRs Spill"):
            key, val = msg.split(":", 1)
            n = int(val.split()[0])
            if n and not key.startswith("SGPRs"):
                bad.append(f"{kernel}: {key.strip()} {n}")
    if bad:
        raise RuntimeError(f"{src}: kernels use stack or spill VGPRs:\n  " + "\n  ".join(bad))


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), RESOURCE_REPORT, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    _check_resources(src, r.stderr)
    # (the report's remarks quote their source lines: "  42 | code" and "     | ^")
    noisy = [ln for ln in r.stderr.splitlines()
             if "packed-fp32-ops" not in ln and "remark:" not in ln and ln.strip()
             and not re.match(r"\s*\d*\s*\|", ln)]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")


def build(verbose: bool = True) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    bdir = os.path.join(CSRC, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(*so), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
