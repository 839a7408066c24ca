"""Build the gfx950 HIP library ``libdsa.so`` in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, then linked into one
shared library exporting the C ABI declared in include/dsa.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["dsa_api.cpp", "indexer_decode.hip", "indexer_prefill.hip", "sfa.hip", "noalloc.hip", "prolog.hip"]

# Kernels that issue LDS reads through inline assembly and wait for them later
# with an explicit lgkmcnt: the compiler takes an asm result as ready at once,
# so a spill or copy of such a register before the wait would read stale data.
# Their build must report no scratch and no spills.
NO_SPILL = {"sfa.hip": ("sfa_bf16_kernel",)}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
          "-I" + INCLUDE, "-I" + CSRC]


def check_no_spills(remarks: str, names) -> list:
    """Kernels among `names` whose resource-usage remarks report scratch or
    spills; raises if none of them was reported at all."""
    cur, bad, seen = None, [], 0
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        if text.startswith("Function Name:"):
            fn = text.split(":", 1)[1].strip()
            cur = fn if any(n in fn for n in names) else None
            seen += cur is not None
            continue
        if cur is None or ":" not in text:
            continue
        key, val = (x.strip() for x in text.rsplit(":", 1))
        if key in ("ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill") and val != "0":
            bad.append(f"{cur}: {key} = {val}")
    if seen == 0:
        raise RuntimeError(f"no resource-usage remarks found for {names}")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    extra = ["-Rpass-analysis=kernel-resource-usage"] if src in NO_SPILL else []
    cmd = [hipcc()] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if src in NO_SPILL:
        bad = check_no_spills(r.stderr, NO_SPILL[src])
        if bad:
            os.remove(obj)
            raise RuntimeError("kernels with deferred-wait inline-asm LDS reads spilled:\n" + "\n".join(bad))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
