"""CPU oracle for the DSA hot path: Lightning Indexer + Top-K + Sparse Flash Attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module; only the test-suite, the package smoke check and the benchmark's
``cpu_baseline`` leg do.  It is plain NumPy in float64, deliberately slow and
written so that each step can be read against the pages:

  Pages (each cited by its title and section):
    [P1] "Day0 Inference Optimization on Ascend CANN: A Deep Dive into Hybrid
         Architecture Acceleration"
    [P2] "Adapting and Optimizing Inference for a New Model Architecture on Ascend"
    [P3] "Day0 Inference Optimization for New LLM Architectures on Heterogeneous
         Computing Platforms"
    [P4] "Inference Acceleration for Next-Gen Attention Architectures: From
         Operator Reuse to Parallel Orchestration"

What is computed (the method as the pages state it):
  * the indexer scores every visible historical position with per-head relevance
    scores q_h . k_s, weights the heads and keeps the Top-K positions
    ([P1] sec. 1 "DSA mechanism" and sec. 2 "Deep Fusion of LI and SFA";
    [P2] sec. 2.2 and 3.1; [P4] sec. 1 and 3.1);
  * causal index computation: a query at position t only sees positions <= t
    ([P1] sec. 4 "Zigzag Layout"; [P2] sec. 5.2);
  * Sparse Flash Attention reads the latent KV rows at the selected positions and
    runs softmax attention over only those rows ([P2] sec. 3.1; [P4] sec. 3.2),
    on top of multi-head latent attention ([P1] sec. 1; [P3] sec. 1);
  * paged caches are read through a block table ([P4] sec. 3.2 "efficient paged
    addressing"; [P1] sec. 2 "directly reads paged KV cache");
  * MXFP8: every 32 elements share one scale ([P1] sec. 3; [P2] sec. 4.2);
  * the SFA KV cache may be stored in FP8 with one scale per token, head and
    tile of 128 elements ([P1] sec. 3, "FP8 Block Quantization for SFA KV
    Cache"; [P2] sec. 4.3 and its table; [P3] quantisation item 2; [P4] sec. 4
    and its table).
  * before the indexer, the prolog projects each new token's hidden row to
    the indexer query, its key (normalised) and the head weights, quantises
    the query and key dynamically and appends the key to the paged cache
    ([P1] sec. 2 "Three-Stream Coordination for Indexer Prolog"; [P2] sec. 3.2
    and 4.2; [P4] sec. 3.3); the readings it takes are listed with its
    functions at the end of this module.

Readings where the pages are silent (each is listed in the design notes):
  * no activation on per-head scores; the weighted combination is a sum over
    heads giving one score per (query, position);
  * Top-K keeps n = min(k, t + 1) positions, larger score first, ties broken
    toward the smaller position; the boundary is inclusive (s <= t);
  * query i of a sequence with T_b new tokens and L_b cached keys sits at
    t = L_b - T_b + i;
  * SFA uses the absorbed (MQA) MLA form: one latent row per position shared by
    every head; logits over all qk dims, V = the first d_v dims of the row;
  * in that form the latent row is the one "head" of the FP8 KV cache: a row of
    576 = 512 latent + 64 rope elements is 5 tiles, the last one 64 long (a row
    shorter than 128 is one tile); each scale is an fp32 that multiplies the
    decoded e4m3 values of its tile.

Every function here is pinned by tests that do not retype its formula
(brute-force loops, library routines, closed forms and invariants).
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------- O1: decoding ---

def decode_bf16_bits(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16) -> float64, exactly: a bf16 value is
    the upper half of the float32 with the same bits."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 ('fn') byte: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); the
    pattern S.1111.111 is NaN; there are no infinities (max 448)."""
    t = np.empty(256, np.float64)
    for byte in range(256):
        sign = -1.0 if byte & 0x80 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 0x7
        if e == 0xF and m == 0x7:
            t[byte] = np.nan
        elif e == 0:
            t[byte] = sign * m * 2.0 ** -9
        else:
            t[byte] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = e4m3fn_table()


def decode_e4m3(bits) -> np.ndarray:
    return _E4M3[np.asarray(bits, dtype=np.uint8)]


def decode_e8m0(bits) -> np.ndarray:
    """OCP E8M0 scale byte -> 2^(E - 127); 0xFF is NaN."""
    e = np.asarray(bits, dtype=np.uint8).astype(np.float64)
    v = np.ldexp(1.0, (e - 127).astype(np.int64))
    return np.where(e == 255, np.nan, v)


KV_TILE = 128   # elements per scale tile of an FP8 SFA KV row


def decode_values(raw, dtype: str, scale=None, group: int = 32) -> np.ndarray:
    """Storage -> float64 for one tensor slice whose last axis is the element axis.

    dtype 'f32'  : raw float32
    dtype 'bf16' : raw bf16 bit patterns
    dtype 'fp8'  : raw e4m3 bytes; ``scale`` has the shape of raw[..., 0]
                   (one fp32 scale per row: per token for keys, per token and
                   head for queries)
    dtype 'mxfp8': raw e4m3 bytes; ``scale`` holds one e8m0 byte per group of
                   ``group`` consecutive elements ([P1] sec. 3, [P2] sec. 4.2)
    dtype 'fp8_t128': raw e4m3 bytes; ``scale`` [..., ceil(D / 128)] holds one
                   fp32 per tile of KV_TILE consecutive elements, the last tile
                   possibly shorter ([P1] sec. 3, [P2] sec. 4.3: the SFA KV
                   cache is quantised per token, head and tile of 128)
    """
    if dtype == "f32":
        return np.asarray(raw, np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16_bits(raw)
    if dtype == "fp8":
        v = decode_e4m3(raw)
        return v * np.asarray(scale, np.float64)[..., None]
    if dtype == "mxfp8":
        v = decode_e4m3(raw)
        sc = decode_e8m0(scale)
        shp = v.shape
        v = v.reshape(*shp[:-1], shp[-1] // group, group) * sc[..., None]
        return v.reshape(shp)
    if dtype == "fp8_t128":
        v = decode_e4m3(raw)
        sc = np.asarray(scale, np.float64)
        tile_of = np.arange(v.shape[-1]) // KV_TILE     # element c -> its tile
        assert sc.shape[-1] == -(-v.shape[-1] // KV_TILE)
        return v * sc[..., tile_of]
    raise ValueError(dtype)


# ---------------------------------------------------------- O2: locate/read ---

def query_position(seq_len: int, q_len: int, i: int) -> int:
    """Position of query i among the T_b newest tokens of a context of L_b keys."""
    return int(seq_len) - int(q_len) + int(i)


def paged_rows(pool_raw, block_table_row, page_size: int, positions) -> np.ndarray:
    """Rows of a paged pool [num_pages][P][...] for logical ``positions``: logical
    page s // P is looked up in the block table, the row is s % P of that page."""
    positions = np.asarray(positions, np.int64)
    pages = np.asarray(block_table_row, np.int64)[positions // page_size]
    return np.asarray(pool_raw)[pages, positions % page_size]


# ------------------------------------------------- O3: indexer (a3 and a4) ---

def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """One score per key: for every head h the relevance q_h . k_s, then the
    head-weighted sum over heads.  q [H][D], w [H], keys [n][D] -> I [n]."""
    per_head = keys @ q.T          # [n][H]: per-head relevance scores
    return per_head @ w            # weighted sum over the heads


# ---------------------------------------------------------- O4: Top-K (a6) ---

def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """Positions of the n = min(k, len(scores)) largest scores; a tie goes to the
    smaller position.  Returned in ascending position order."""
    n = min(int(k), len(scores))
    pos = np.arange(len(scores))
    order = np.lexsort((pos, -np.asarray(scores, np.float64)))  # primary: -score
    return np.sort(order[:n])


# ------------------------------------------------------ O5: SFA (a8 - a11) ---

def sparse_attention(q: np.ndarray, rows: np.ndarray, d_v: int, scale: float):
    """Softmax attention of every head over the gathered latent rows only.
    q [H][Dqk], rows [n][Dqk] -> (O [H][d_v], lse [H]); V = rows[:, :d_v]."""
    z = scale * (q @ rows.T)                      # [H][n] logits
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ rows[:, :d_v]) / l
    return o, (m + np.log(l))[:, 0]


# ------------------------------------------------------ zigzag (a13) ---

def zigzag_units(n_blocks: int):
    """Pair query blocks from the two ends of the sequence: unit u holds blocks
    u and n_blocks-1-u (an odd count leaves the middle block alone), so that a
    short-history block shares a unit with a long-history one ([P1] sec. 4;
    [P2] sec. 5.2; [P3] sec. 4.2; [P4] sec. 5.2)."""
    units = [[u, n_blocks - 1 - u] for u in range(n_blocks // 2)]
    if n_blocks % 2:
        units.append([n_blocks // 2])
    return units


# ------------------------------------------------ per-query driver (O6) ---

class QueryResult(dict):
    """idx (ascending), scores I[0..t], kth (the n-th largest score), out, lse."""


def indexer_query(case, b: int, i: int):
    """Indexer + Top-K for query i of sequence b of a case (see the input module
    for layouts).  Reads every key through the block table."""
    P = case.page_size
    L, T = int(case.seq_lens_host[b]), int(case.q_lens_host[b])
    t = query_position(L, T, i)
    tok = case.token(b, i)
    bt = _np(case.block_table[b])
    pos = np.arange(t + 1)
    q = decode_values(_np(case.q_i[tok]), case.idx_dtype,
                      None if case.q_i_scale is None else _np(case.q_i_scale[tok]))
    k_raw = paged_rows(_np(case.k_pool), bt, P, pos)
    k_sc = None if case.k_scale is None else paged_rows(_np(case.k_scale), bt, P, pos)
    keys = decode_values(k_raw, case.idx_dtype, k_sc)
    w = _np(case.w[tok]).astype(np.float64)
    scores = indexer_scores(q, w, keys)
    idx = topk_select(scores, case.topk)
    kth = np.sort(scores)[::-1][len(idx) - 1]
    return t, scores, idx, kth


def sfa_query(case, b: int, i: int, idx) -> tuple:
    """SFA for query i of sequence b over logical positions ``idx``."""
    tok = case.token(b, i)
    bt = _np(case.block_table[b])
    kv_dtype = getattr(case, "kv_dtype", None) or case.sfa_dtype
    kv_scale = getattr(case, "kv_scale", None)
    rows = decode_values(paged_rows(_np(case.kv_pool), bt, case.page_size, np.asarray(idx)),
                         kv_dtype,
                         None if kv_scale is None
                         else paged_rows(_np(kv_scale), bt, case.page_size, np.asarray(idx)))
    q = decode_values(_np(case.q_s[tok]), case.sfa_dtype)
    return sparse_attention(q, rows, case.d_v, case.softmax_scale)


def run_query(case, b: int, i: int) -> QueryResult:
    t, scores, idx, kth = indexer_query(case, b, i)
    out, lse = sfa_query(case, b, i, idx)
    return QueryResult(t=t, scores=scores, idx=idx, kth=kth, out=out, lse=lse)


# Host copies of large device/CPU tensors, kept (with a reference to the tensor,
# so that its storage cannot be reused while cached) for repeated per-query calls.
_HOST_CACHE: dict = {}
_HOST_CACHE_MAX = 6


def _np(x) -> np.ndarray:
    """Accept numpy arrays or torch tensors (CPU or device); bf16 tensors come
    back as their uint16 bit patterns, fp8 bytes as uint8."""
    if isinstance(x, np.ndarray):
        return x
    try:
        import torch
    except ImportError:  # pragma: no cover
        return np.asarray(x)
    if not isinstance(x, torch.Tensor):
        return np.asarray(x)
    big = x.numel() > (1 << 20)
    if big and id(x) in _HOST_CACHE and _HOST_CACHE[id(x)][0] is x:
        return _HOST_CACHE[id(x)][1]
    t = x.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    a = t.cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if big:
        if len(_HOST_CACHE) >= _HOST_CACHE_MAX:
            _HOST_CACHE.pop(next(iter(_HOST_CACHE)))
        _HOST_CACHE[id(x)] = (x, a)
    return a


# ===================================================== indexer prolog (NEXT) ===
# The steps the pages place before the fused indexer ([P1] sec. 2 "Three-Stream
# Coordination for Indexer Prolog"; [P2] sec. 3.2 and 4.2; [P4] sec. 3.3):
# Q projection, K normalisation, dynamic Q quantisation and the head-weight
# projection, plus writing the new tokens' keys into the paged K cache.
# Readings (the pages name the steps, not their formulas):
#   * one bf16 hidden row x[t] of width d_model per new token feeds all three
#     projections; weights are bf16 in the linear-layer layout [out][in];
#   * q = bf16(x W_q^T) reshaped [H][D]; the projections stay bf16 ([P2] sec. 4:
#     projection is precision-sensitive);
#   * k = bf16(LayerNorm(x W_k^T)) over the D elements, biased variance,
#     eps = 1e-6, then gamma and beta;
#   * w = x W_w^T in float (one weight per head);
#   * quantisation as for the quantised indexer inputs: FP8 with scale
#     amax / 448 (1 if amax = 0) in float32, elements x / scale rounded to
#     nearest-even and saturated (per token and head for q, per token for k);
#     MXFP8 with E = floor(log2 amax) - 8 clamped to [-127, 127] per group of
#     32, elements x * 2^-E rounded and saturated (OCP MX v1.0 rule for e4m3);
#   * the new key of token i of sequence b goes to position t = L_b - T_b + i:
#     row t % P of page block_table[b][t // P], with its scale(s).

def round_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit pattern (uint16) rounding the exact value to nearest,
    ties to an even significand: a bf16 number has 8 significant bits (7
    stored), the float32 exponent range and subnormals below 2^-126."""
    x = np.asarray(x, np.float64)
    out = np.zeros(x.shape, np.uint16)
    flat, res = x.reshape(-1), out.reshape(-1)
    for n, v in enumerate(flat):
        if v != v:
            res[n] = 0x7FC0
            continue
        sign = 0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0
        a = abs(float(v))
        if a == 0.0:
            res[n] = sign
            continue
        e = max(int(np.floor(np.log2(a))), -126)
        if 2.0 ** e > a:            # guard log2 rounding
            e -= 1
        elif 2.0 ** (e + 1) <= a:
            e += 1
        e = max(e, -126)
        q = a / 2.0 ** (e - 7)      # significand in units of the last place
        m = np.floor(q)
        frac = q - m
        if frac > 0.5 or (frac == 0.5 and int(m) % 2 == 1):
            m += 1
        val = m * 2.0 ** (e - 7)
        if val >= 2.0 ** 128:
            res[n] = sign | 0x7F80          # overflow: infinity
            continue
        b = np.float32(val).view(np.uint32) >> 16
        res[n] = sign | int(b)
    return out


def e4m3_encode(y) -> np.ndarray:
    """float -> OCP e4m3fn byte: the nearest value of the e4m3 table (ties to
    the even code), saturating to +-448; the sign of zero is kept."""
    y = np.asarray(y, np.float64)
    t = _E4M3[:0x7F]                 # codes 0x00..0x7E: 0 .. 448, increasing
    a = np.minimum(np.abs(y), 448.0)
    hi = np.clip(np.searchsorted(t, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - t[lo], t[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def fp8_quantise(v):
    """One row of float values (float32-exact) -> (e4m3 bytes, float32 scale):
    scale = amax / 448 in float32 (1 for an all-zero row), elements v / scale
    in float32, then rounded to e4m3."""
    v = np.asarray(v, np.float32)
    amax = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = (v / s).astype(np.float32)
    return e4m3_encode(y), s


def mx_quantise(v, group: int = 32):
    """One row (float32-exact values) -> (e4m3 bytes, e8m0 bytes per group):
    E = floor(log2 amax) - 8 (amax = 0 -> -127), clamped to [-127, 127];
    elements v * 2^-E, rounded to e4m3 with saturation."""
    v = np.asarray(v, np.float32).reshape(-1, group)
    codes, scales = [], []
    for g in v:
        amax = float(np.max(np.abs(g)))
        if amax > 0:
            m, ex = np.frexp(amax)            # amax = m 2^ex, m in [0.5, 1)
            E = int(ex) - 1 - 8
        else:
            E = -127
        E = min(max(E, -127), 127)
        codes.append(e4m3_encode(np.ldexp(g.astype(np.float64), -E)))
        scales.append(E + 127)
    return np.concatenate(codes), np.asarray(scales, np.uint8)


def layer_norm(v, gamma, beta, eps: float = 1e-6):
    """(v - mean) / sqrt(var + eps) * gamma + beta over the last axis, biased var."""
    v = np.asarray(v, np.float64)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def prolog_token(x_bits, wq_bits, wk_bits, ww_bits, gamma, beta, n_heads: int, head_dim: int,
                 eps: float = 1e-6):
    """The projections of one new token: x [d_model] bf16 bits, weights bf16 bits
    [out][in].  Returns (q bf16 bits [H][D], k bf16 bits [D], w float64 [H])."""
    x = decode_bf16_bits(x_bits)
    q = decode_bf16_bits(wq_bits) @ x
    k = layer_norm(decode_bf16_bits(wk_bits) @ x, gamma, beta, eps)
    w = decode_bf16_bits(ww_bits) @ x
    return round_bf16_bits(q).reshape(n_heads, head_dim), round_bf16_bits(k), w


def quantise_query(q_bits, dtype: str):
    """q bf16 bits [H][D] -> (stored q, its scales) for the indexer dtype."""
    q = decode_bf16_bits(q_bits)
    if dtype == "bf16":
        return np.asarray(q_bits, np.uint16), None
    parts = [fp8_quantise(r) if dtype == "fp8" else mx_quantise(r) for r in q]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def quantise_key(k_bits, dtype: str):
    """k bf16 bits [D] -> (stored key row, its scale(s))."""
    if dtype == "bf16":
        return np.asarray(k_bits, np.uint16), None
    k = decode_bf16_bits(k_bits)
    return fp8_quantise(k) if dtype == "fp8" else mx_quantise(k)


def append_position(seq_len: int, q_len: int, i: int, block_table_row, page_size: int):
    """(page, row) where the key of new token i goes: position t = L - T + i."""
    t = query_position(seq_len, q_len, i)
    return int(np.asarray(block_table_row)[t // page_size]), t % page_size
