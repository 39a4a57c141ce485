"""Build the gfx950 HIP library ``linear_amd/liblinear_amd.so`` with hipcc.

Run ``python -m linear_amd.build``.  Always recompiles (the build check must
really compile); object files go to ``_build/`` at the repository root.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblinear_amd.so")
# measurement kernels for bench.py's ceilings, kept out of the layer's library
PROBE_OUT = os.path.join(HERE, "liblinear_probe.so")
PROBE_SOURCES = ["probe.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["gemm_f16.hip", "gemm_bf16.hip", "skinny.hip", "epilogue.hip", "indexed.hip", "linear_abi.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-fno-gpu-flush-denormals-to-zero",   # binary16 subnormals are kept (IEEE gradual underflow)
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
    "-Rpass-analysis=kernel-resource-usage",   # per-kernel registers, spills, scratch (checked below)
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _resources(text: str) -> dict:
    """Kernel name -> {field: value} from hipcc's kernel-resource-usage remarks."""
    res, name = {}, None
    for line in text.splitlines():
        if "[-Rpass-analysis=kernel-resource-usage]" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass", 1)[0].strip()
        key, _, val = body.partition(": ")
        if key == "Function Name":
            name = val
            res[name] = {}
        elif name is not None:
            res[name][key] = val
    return res


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    noise = ("is not a recognized feature for this target", "kernel-resource-usage")
    msg = "\n".join(l for l in out.splitlines()
                    if not any(n in l for n in noise) and not l.lstrip().startswith(("|", "^", "In file included from"))
                    and not (l[:6].strip().isdigit() and " | " in l))
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
    if msg.strip():
        print(msg, file=sys.stderr)
    # every kernel must run from registers and LDS: scratch memory (spills, or an
    # argument copy indexed at run time) costs a memory round trip per access
    res = _resources(out)
    bad = {k: v for k, v in res.items()
           if v.get("ScratchSize [bytes/lane]", "0") != "0" or v.get("VGPRs Spill", "0") != "0"}
    with open(os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".resources.txt"), "w") as f:
        for k, v in sorted(res.items()):
            f.write("%s %s\n" % (k, " ".join("%s=%s" % (a.replace(" ", "_"), b) for a, b in v.items())))
    if bad:
        raise RuntimeError("kernels in %s use scratch memory: %s" % (src, ", ".join(sorted(bad))))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    # a failed build must not leave the previous library behind for tests and
    # benchmarks to load
    for out in (OUT, PROBE_OUT):
        if os.path.exists(out):
            os.remove(out)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    for out, part in ((OUT, objs[:len(SOURCES)]), (PROBE_OUT, objs[len(SOURCES):])):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *part, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
        if verbose:
            print("built", out)
    return OUT


if __name__ == "__main__":
    build()
