"""Builds libmxq.so (every HIP source under csrc/, gfx950 only) in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import json
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmxq.so")
OBJ_DIR = os.path.join(ROOT, "_build", "mxq")
# Per-kernel register use of the last build (the compiler's resource remarks).
RESOURCES = os.path.join(OBJ_DIR, "resource_usage.json")

ARCH = "gfx950"
# Packed fp32 arithmetic is switched off (the device pass honours the flag; the
# host pass prints a harmless "not a recognized feature" warning).
HIPFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|"
                     r"Occupancy \[waves/SIMD\]): (\S+)")
_KEYS = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch", "VGPRs Spill": "vgpr_spill",
         "SGPRs Spill": "sgpr_spill", "Occupancy [waves/SIMD]": "occupancy"}


def _resources(remarks: str) -> dict:
    """kernel -> {vgpr, agpr, scratch, vgpr_spill, sgpr_spill, occupancy} from the resource remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(remarks):
        if m.group(1) == "Function Name":
            cur = m.group(2)
            out[cur] = {}
        elif cur is not None:
            out[cur][_KEYS[m.group(1)]] = int(m.group(2))
    return out


def _compile(src: str):
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPFLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj, _resources(r.stderr)


def build(jobs: int = 8) -> str:
    """Compile every csrc/*.hip for gfx950 and link libmxq.so (always rebuilds).
    The compiler's per-kernel register use goes to RESOURCES."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(_compile, sources()))
    objs = [o for o, _ in done]
    usage = {}
    for src, (_, res) in zip(sources(), done):
        for kern, r in res.items():
            usage[kern] = dict(r, source=os.path.basename(src))
    with open(RESOURCES, "w") as f:
        json.dump(usage, f, indent=0, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
