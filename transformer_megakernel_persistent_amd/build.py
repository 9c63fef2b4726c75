"""Build libmk.so (the C-ABI library) with hipcc for gfx950, in-tree.

Every source compiles to an object in _build/ (in parallel), then one link.
mk_kernel.hip compiles several times: once per (dtype, query-group) part of
the decode kernel's instantiations, and once for the host launch code.

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
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")  # the public C ABI header
LIB = os.path.join(HERE, "libmk.so")
RESOURCES = os.path.join(HERE, "libmk.resources.json")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["mk_api.hip", "mk_kernel.hip", "mk_prelayout.hip", "mk_prefill.hip"]
HEADERS = [os.path.join(CSRC, "mk_internal.h"), os.path.join(INCLUDE, "mk.h")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# (dtype, query heads per KV head) parts of the decode kernel's instantiations
# (dtype 0 float32, 1 bfloat16, 2 weight-only INT8)
KERNEL_PARTS = [(dt, gq) for dt in (0, 1, 2) for gq in (1, 2, 4, 8)]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 instructions stay off (they are emitted only by the compiler)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# per-kernel register / scratch report on stderr (parsed below)
REMARKS = "-Rpass-analysis=kernel-resource-usage"


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


# per-source options: the prefill kernels keep their matrix-core
# accumulators in ordinary VGPRs (the online-softmax rescaling and the GEMM
# epilogues then need no moves between accumulation and vector registers)
SOURCE_FLAGS = {"mk_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _jobs():
    jobs = []
    for s in SOURCES:
        jobs.append((s, SOURCE_FLAGS.get(s, []), os.path.join(OBJDIR, s.replace(".hip", ".o"))))
    for dt, gq in KERNEL_PARTS:
        jobs.append(("mk_kernel.hip", ["-DMK_KERNEL_PART", f"-DMK_PART_DT={dt}", f"-DMK_PART_GQ={gq}"],
                     os.path.join(OBJDIR, f"mk_kernel_part_{dt}_{gq}.o")))
    return jobs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(job):
        src, defs, obj = job
        cmd = [HIPCC, *FLAGS, REMARKS, *defs, "-I", INCLUDE, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, capture_output=True, text=True), src, defs

    jobs = _jobs()
    with ThreadPoolExecutor(max_workers=min(len(jobs), max(1, os.cpu_count() or 1))) as ex:
        results = list(ex.map(compile_one, jobs))
    remarks = []
    for res, src, defs in results:
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {src} {' '.join(defs)}")
        remarks.append(res.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[j[2] for j in jobs]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libmk.so failed")
    os.replace(tmp, LIB)
    kernels = parse_resources("\n".join(remarks))
    with open(RESOURCES, "w") as f:
        json.dump({"sources_hash": sources_hash(), "flags": FLAGS, "kernels": kernels}, f, indent=1)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
