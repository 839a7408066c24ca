"""Build the gfx950 HIP library ``libdsa.so`` in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only, then linked into one
shared library exporting the C ABI declared in include/dsa.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["dsa_api.cpp", "indexer_decode.hip", "indexer_prefill.hip", "sfa.hip", "noalloc.hip", "prolog.hip",
           "checks.hip", "fused_decode.hip"]

# Kernels that issue LDS reads through inline assembly and wait for them later
# with an explicit lgkmcnt: the compiler takes an asm result as ready at once,
# so a spill or copy of such a register before the wait would read stale data.
# Their build must report no scratch and no spills, and their device assembly
# must not touch such a register before a wait that covers its read.
NO_SPILL = {"sfa.hip": ("sfa_bf16_kernel",), "fused_decode.hip": ("fused_decode_kernel",)}


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
        # SGPR spills go to lanes of reserved VGPRs (no scratch, no copy of a
        # pending LDS result), so only scratch and VGPR spills are refused
        if key in ("ScratchSize [bytes/lane]", "VGPRs Spill") and val != "0":
            bad.append(f"{cur}: {key} = {val}")
    if seen == 0:
        raise RuntimeError(f"no resource-usage remarks found for {names}")
    return bad


_REG = re.compile(r"\b([vas])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_STORES = ("ds_write", "ds_store", "global_store", "buffer_store", "scratch_store", "flat_store")
_NO_DEST = ("s_cbranch", "s_branch", "s_barrier", "s_nop", "s_setprio", "s_sleep", "s_waitcnt", "s_endpgm")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def check_deferred_lds_waits(asm: str, names) -> list:
    """Instructions in the functions named by `names` that read or write a
    register loaded by an inline-asm LDS read (between ;;#ASMSTART and
    ;;#ASMEND) before an s_waitcnt lgkmcnt that covers that read.  LDS
    operations complete in order; every lgkm operation (compiler-issued too)
    counts, and while a scalar memory load is outstanding only lgkmcnt(0)
    retires anything.  The scan is linear: each function's code is taken in
    the order it is laid out."""
    bad, seen = [], 0
    for part in re.split(r"\n(?=[A-Za-z_.$][\w.$]*:[ \t]*(?:;.*)?\n)", asm):
        name = part.split(":", 1)[0].strip()
        if not any(n in name for n in names):
            continue
        seen += 1
        pending, in_asm = [], False     # [dest regs, from asm, is scalar load, text]
        for raw in part.split("\n"):
            line = raw.strip()
            if line.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if line.startswith(";;#ASMEND"):
                in_asm = False
                continue
            ins = line.split(";")[0].strip()
            if not ins or ins.endswith(":") or ins.startswith("."):
                continue
            op, _, args = ins.partition(" ")
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", args)
                if m is not None or args.strip() == "0":
                    keep = int(m.group(1)) if m else 0
                    if keep == 0:
                        pending = []
                    elif not any(p[2] for p in pending):
                        pending = pending[len(pending) - keep:] if len(pending) > keep else pending
                continue
            ops = [a.strip() for a in args.split(",")] if args.strip() else []
            first_is_dest = not op.startswith(_STORES) and not op.startswith(_NO_DEST)
            rd, wr = set(), set()
            for i, a in enumerate(ops):
                (wr if (i == 0 and first_is_dest) else rd).update(_regs(a))
            for dest, from_asm, _, text in pending:
                if from_asm and dest and (dest & (rd | wr)):
                    bad.append(f"{name}: '{ins}' uses a register of '{text}' before its wait")
            if op.startswith(("ds_", "s_load", "s_buffer_load", "s_sendmsg")):
                loads = op.startswith(("ds_read", "ds_bpermute", "ds_permute", "ds_swizzle", "s_load", "s_buffer_load"))
                pending.append([_regs(ops[0]) if (loads and ops) else None,
                                in_asm and op.startswith("ds_read"), op.startswith(("s_load", "s_buffer_load")), ins])
    if seen == 0:
        raise RuntimeError(f"no device code found for {names}")
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
        if not bad:
            asm_path = os.path.splitext(obj)[0] + ".s"
            cmd = [hipcc()] + COMMON + ["-S", "--offload-device-only", os.path.join(CSRC, src), "-o", asm_path]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"assembly listing failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            with open(asm_path) as f:
                bad = check_deferred_lds_waits(f.read(), NO_SPILL[src])
        if bad:
            os.remove(obj)
            raise RuntimeError("kernels with deferred-wait inline-asm LDS reads are unsafe:\n" + "\n".join(bad[:20]))
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
