"""Builds libpa.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: ``python -m paged_kv_cache_195_amd.build`` (or ``__graft_entry__.build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so the Python binding finds it.  The per-kernel
register and LDS report of the compiler goes to ``_build/resource_usage.txt``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "pa_api.cpp",
    "attn_valu_f32.hip",
    "attn_mfma_f16.hip",
    "attn_mfma_bf16.hip",
    "attn_mfma_q_f16.hip",
    "attn_mfma_q_bf16.hip",
    "combine.hip",
    "page_check.hip",
    "pa_noalloc.hip",
]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj, res.stderr


_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr",
           "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "waves/simd",
           "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}


def resource_table(logs) -> str:
    """One line per kernel from the compiler's kernel-resource-usage remarks."""
    rows, cur = [], None
    for log in logs:
        for ln in log.splitlines():
            if "remark:" not in ln:
                continue
            body = ln.split("remark:", 1)[1].split("[-Rpass")[0].strip()
            key, _, val = body.partition(":")
            key, val = key.strip(), val.strip()
            if key == "Function Name":
                cur = {"name": val}
                rows.append(cur)
            elif cur is not None and key in _FIELDS:
                cur[_FIELDS[key]] = val
    cols = list(_FIELDS.values())
    out = ["kernel " + " ".join(cols)]
    for r in rows:
        out.append(r["name"] + " " + " ".join(r.get(c, "?") for c in cols))
    return "\n".join(out) + "\n"


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(_compile, SOURCES))
    objs = [r[0] for r in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(resource_table([r[1] for r in results]))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
