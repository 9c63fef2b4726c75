"""Build libmk.so (the C-ABI library) with hipcc for gfx950, in-tree.

The compiler's per-kernel resource report (VGPRs, SGPRs, scratch bytes per
lane, occupancy) is saved beside the library as libmk.resources.json, keyed
by a hash of the sources it was built from; tests/test_kernel_resources.py
checks it (no kernel may spill to scratch).
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")  # the public C ABI header
LIB = os.path.join(HERE, "libmk.so")
RESOURCES = os.path.join(HERE, "libmk.resources.json")
SOURCES = ["mk_api.hip", "mk_kernel.hip", "mk_prelayout.hip", "mk_prefill.hip"]
HEADERS = [os.path.join(CSRC, "mk_internal.h"), os.path.join(INCLUDE, "mk.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions stay off (they are emitted only by the compiler)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # per-kernel register / scratch report on stderr (parsed below)
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark: ([^:]*(?:\.hip|\.h)):\d+:\d+: *(?:remark: )?\s*([A-Za-z][A-Za-z /\[\]]*?)\s*:\s*(\S+)")


def sources_hash() -> str:
    h = hashlib.sha256()
    for p in [os.path.join(CSRC, s) for s in SOURCES] + HEADERS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_resources(text: str) -> list:
    """Kernel records from the compiler's kernel-resource-usage remarks."""
    kernels, cur = [], None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        if cur is None:
            continue
        for key, pat in (("sgprs", r"TotalSGPRs: (\d+)"), ("vgprs", r"\bVGPRs: (\d+)"), ("agprs", r"AGPRs: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)"), ("lds", r"LDS Size \[bytes/block\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                cur[key] = int(m.group(1))
    return kernels


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    os.replace(tmp, LIB)
    kernels = parse_resources(res.stderr)
    with open(RESOURCES, "w") as f:
        json.dump({"sources_hash": sources_hash(), "flags": FLAGS, "kernels": kernels}, f, indent=1)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
