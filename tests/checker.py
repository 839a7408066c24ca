"""Comparison rules between the HIP path and the oracle.

Top-K: the GPU row holds n = min(k, t+1) distinct positions in [0, t] (any
order) followed by -1; every position in the symmetric difference with the
oracle's set must score within 1e-3 * max(|I_(n)|, rms(I)) of the oracle's n-th
largest score I_(n); otherwise the sets are equal.

SFA: max-abs error within the dtype's bar (bf16 2e-2, fp8 KV 6e-2, f32 2e-2 with
the achieved error reported) and, for bf16, relative L2 error <= 1e-2 so that an
all-zero output cannot pass on inputs whose outputs are small.  The output is
stored in the query dtype, so each element may also differ by that dtype's
rounding of the oracle's value (half an ulp: 2^-8 |x| for bf16): with 20-sigma
outliers in the latent rows an output near 20 has a bf16 spacing of 0.125,
which no bf16 result can meet within 2e-2 alone.
"""
from __future__ import annotations

import numpy as np

TOPK_REL = 1e-3
SFA_ABS = {"bf16": 2e-2, "fp8": 6e-2, "f32": 2e-2}
SFA_REL_L2 = {"bf16": 1e-2, "fp8": 3e-2, "f32": 1e-4}
OUT_ROUND = {"bf16": 2.0 ** -8, "fp8": 2.0 ** -8, "f32": 0.0}   # storage rounding of the output


class Mismatch(AssertionError):
    pass


def check_topk_row(gpu_row, ref, k: int) -> int:
    """Raise Mismatch on failure; return the size of the tolerated difference."""
    t = int(ref["t"])
    n = min(k, t + 1)
    row = np.asarray(gpu_row).astype(np.int64)
    if row.shape != (k,):
        raise Mismatch(f"row shape {row.shape} != ({k},)")
    if not np.all(row[n:] == -1):
        raise Mismatch(f"slots >= n={n} must hold -1: {row[n:][row[n:] != -1][:8]}")
    g = row[:n]
    if np.any(g < 0) or np.any(g > t):
        raise Mismatch(f"positions outside [0, {t}]: {g[(g < 0) | (g > t)][:8]}")
    gs = set(g.tolist())
    if len(gs) != n:
        raise Mismatch(f"duplicate positions: {n - len(gs)} duplicates")
    rs = set(np.asarray(ref["idx"]).tolist())
    diff = gs ^ rs
    if diff:
        scores = np.asarray(ref["scores"])
        kth = float(ref["kth"])
        band = TOPK_REL * max(abs(kth), float(np.sqrt(np.mean(scores ** 2))))
        bad = [p for p in diff if abs(scores[p] - kth) > band]
        if bad:
            raise Mismatch(f"{len(bad)} positions differ outside the 1e-3 band "
                           f"(kth={kth:.6g}, band={band:.3g}), e.g. pos {bad[0]} score {scores[bad[0]]:.6g}")
    return len(diff)


def check_sfa(gpu_out, ref_out, dtype: str):
    """Raise Mismatch on failure; return (max_abs, rel_l2)."""
    g = np.asarray(gpu_out, np.float64)
    r = np.asarray(ref_out, np.float64)
    if g.shape != r.shape:
        raise Mismatch(f"shape {g.shape} != {r.shape}")
    if not np.isfinite(g).all():
        raise Mismatch("non-finite output")
    err = np.abs(g - r)
    excess = err - OUT_ROUND[dtype] * np.abs(r)
    mx = float(excess.max()) if err.size else 0.0
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
    if mx > SFA_ABS[dtype]:
        raise Mismatch(f"max abs error beyond output rounding {mx:.3g} > {SFA_ABS[dtype]}")
    if rel > SFA_REL_L2[dtype]:
        raise Mismatch(f"relative L2 error {rel:.3g} > {SFA_REL_L2[dtype]}")
    return mx, rel
