"""Build the HIP engine library for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
OUT = os.path.join(OUT_DIR, "libpdm.so")
SOURCES = ["engine.hip", "batch.hip", "batch_step.hip", "dsa.hip", "api.cpp", "planner.cpp"]

# Packed FP32 VALU forms stay off: plain float code only. The atomic
# optimizer (which turns a few lanes' LDS or global atomics into a lane loop
# plus one atomic) is off: the engine's atomics come from one to four lanes.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


USAGE = os.path.join(OUT_DIR, "resource_usage.json")


def parse_resource_usage(text: str) -> dict:
    """Per-kernel register, spill, scratch and LDS figures from hipcc's
    kernel-resource-usage remarks."""
    usage, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = usage.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(-?\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return usage


def build_library(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"),
           "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    msgs = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l
                     and not l.lstrip().startswith(("|", "^")) and not re.match(r"^\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    with open(USAGE, "w") as f:
        json.dump(parse_resource_usage(text), f, indent=1, sort_keys=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build_library(verbose=True))
