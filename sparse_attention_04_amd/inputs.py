"""Seeded synthetic inputs for the DSA hot path (indexer + Top-K + SFA).

This module only *prepares inputs*: it draws random values, rounds them to the
storage dtype, encodes the FP8 / MXFP8 variants and lays the rows out in paged
pools addressed through a block table.  It holds none of the method's own
arithmetic (no scores, no selection, no attention), so both the CPU oracle and
the HIP path consume its output without sharing any computation.

Workload shapes follow the problem statement of the Lightning Indexer and Sparse
Flash Attention on the pages ("Deep Fusion of LI and SFA", Day0 Inference
Optimization on Ascend CANN, section 2): a query, a paged K cache read through a
block table, per-head weights, a Top-K size and per-sequence lengths.  The
quantised storage formats follow the layered-quantisation sections of the same
pages (MXFP8 with groups of 32 elements sharing one scale; FP8 with one fp32
scale per token for keys and per token and head for queries; the SFA KV cache
optionally in FP8 with one fp32 scale per tile of 128 elements of each row,
"Adapting and Optimizing Inference for a New Model Architecture on Ascend",
section 4.3).

Recipe (fixed, documented):
  * every tensor has its own torch generator seeded from
    SeedSequence([seed, tensor_id]) so any tensor can be regenerated alone;
  * on device="cuda" the same draws are made by torch's CUDA generator
    (a different stream of numbers, still seeded and deterministic);
  * values are drawn in float32 and rounded to bf16 with round-to-nearest-even;
  * FP8 scale = amax / 448 (amax == 0 -> 1), elements x / scale rounded to
    nearest-even and saturated to +-448 (OCP e4m3fn); amax is taken per row,
    or per tile of 128 elements (the last tile of a row may be shorter) for the
    tiled KV format;
  * MX scale exponent E = floor(log2 amax) - 8 clamped to e8m0's range, elements
    x * 2^-E saturated to +-448 (OCP MX v1.0 rule for e4m3 elements);
  * the tail of every sequence's last page, and one spare page that all unused
    block-table entries point at, are filled with NaN (0x7F for e4m3), so a read
    past a sequence's length shows up as a non-finite result.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Storage dtype names used across the package.
F32, BF16, FP8, MXFP8 = "f32", "bf16", "fp8", "mxfp8"
FP8T = "fp8_t128"    # SFA KV rows: e4m3 bytes + one fp32 scale per 128-element tile

E4M3_MAX = 448.0
MX_GROUP = 32
KV_TILE = 128

# Tensor ids for per-tensor seeding (fixed: changing them changes every case).
_TID = dict(seq_lens=1, pages=2, q_i=3, k_i=4, w=5, q_s=6, kv=7,
            out_q_i=8, out_k_i=9, out_q_s=10, out_kv=11,
            pro_x=12, pro_wq=13, pro_wk=14, pro_ww=15, pro_ln=16)


def _gen(seed: int, tid: str, device: str) -> torch.Generator:
    s = int(np.random.SeedSequence([seed, _TID[tid]]).generate_state(1, np.uint64)[0] & ((1 << 63) - 1))
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


@dataclasses.dataclass
class Case:
    """One seeded workload.  All tensors live on ``device``.

    Layouts (row-major):
      seq_lens  int32 [B]            keys already in the caches for sequence b
      q_lens    int32 [B]            new query tokens T_b (the last T_b positions)
      cu_q      int32 [B+1]          query-token offsets
      block_table int32 [B][max_pages_per_seq]  logical page -> physical page
      q_i       [sum T][H_I][D_I]    f32 / bf16 / uint8 (e4m3 bits)
      q_i_scale None | f32 [sum T][H_I] (fp8) | uint8 [sum T][H_I][D_I/32] (e8m0)
      w         f32 [sum T][H_I]     head weights
      k_pool    [num_pages][P][D_I]  f32 / bf16 / uint8 (e4m3 bits)
      k_scale   None | f32 [num_pages][P] | uint8 [num_pages][P][D_I/32]
      q_s       [sum T][H_S][D_qk]   f32 / bf16
      kv_pool   [num_pages][P][D_qk] f32 / bf16, or uint8 (e4m3 bits) when
                kv_dtype is fp8_t128 (V = the first D_v columns)
      kv_scale  None | f32 [num_pages][P][ceil(D_qk / 128)] (fp8_t128)
    """
    name: str
    seed: int
    device: str
    batch: int
    seq_lens: torch.Tensor
    q_lens: torch.Tensor
    cu_q: torch.Tensor
    page_size: int
    num_pages: int
    max_pages_per_seq: int
    block_table: torch.Tensor
    h_i: int
    d_i: int
    topk: int
    idx_dtype: str
    q_i: torch.Tensor
    q_i_scale: Optional[torch.Tensor]
    w: torch.Tensor
    k_pool: torch.Tensor
    k_scale: Optional[torch.Tensor]
    h_s: int
    d_qk: int
    d_v: int
    softmax_scale: float
    sfa_dtype: str
    q_s: torch.Tensor
    kv_pool: torch.Tensor
    # host copies of the small integer metadata (always on the CPU)
    seq_lens_host: np.ndarray = None
    q_lens_host: np.ndarray = None
    # storage of the latent KV rows: sfa_dtype (None), or fp8_t128 with kv_scale
    kv_dtype: Optional[str] = None
    kv_scale: Optional[torch.Tensor] = None

    def __post_init__(self):
        if self.kv_dtype is None:
            self.kv_dtype = self.sfa_dtype

    @property
    def total_q(self) -> int:
        return int(self.q_lens_host.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens_host.max())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens_host.max())

    def token(self, b: int, i: int) -> int:
        """Row of query i of sequence b in the [sum T] arrays."""
        return int(self.q_lens_host[:b].sum()) + i

    def position(self, b: int, i: int) -> int:
        """Causal position t of query i of sequence b (the new tokens are the
        last T_b positions of a context of seq_lens[b] keys)."""
        return int(self.seq_lens_host[b]) - int(self.q_lens_host[b]) + i


# ---------------------------------------------------------------- encoders ---

def round_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def encode_e4m3(x: torch.Tensor) -> torch.Tensor:
    """float -> e4m3fn bits (uint8), RNE, saturated to +-448."""
    return x.float().clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def quant_fp8_rows(x: torch.Tensor):
    """Per-row FP8: x [..., D] -> (bits uint8 [..., D], scale f32 [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()
    return encode_e4m3(x / scale.unsqueeze(-1)), scale


def quant_fp8_tiles(x: torch.Tensor, tile: int = KV_TILE):
    """FP8 with one scale per tile of ``tile`` consecutive elements along the
    last dim (the last tile may be shorter):
    x [..., D] -> (bits uint8 [..., D], scale f32 [..., ceil(D / tile)])."""
    x = x.float()
    D = x.shape[-1]
    nt = -(-D // tile)
    xp = torch.nn.functional.pad(x, (0, nt * tile - D))
    g = xp.reshape(*x.shape[:-1], nt, tile)
    amax = g.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).float()
    bits = encode_e4m3(g / scale.unsqueeze(-1)).reshape(*x.shape[:-1], nt * tile)[..., :D]
    return bits.contiguous(), scale


def quant_mx_rows(x: torch.Tensor):
    """MXFP8 along the last dim in groups of 32:
    x [..., D] -> (bits uint8 [..., D], e8m0 uint8 [..., D/32])."""
    x = x.float()
    shp = x.shape
    g = x.reshape(*shp[:-1], shp[-1] // MX_GROUP, MX_GROUP)
    amax = g.abs().amax(dim=-1)
    # floor(log2(amax)) via frexp: amax = m * 2^e, m in [0.5, 1)
    _, e = torch.frexp(amax)
    ex = (e.to(torch.int32) - 1) - 8
    ex = torch.where(amax > 0, ex, torch.full_like(ex, -127))
    ex = ex.clamp(-127, 127)
    scale = torch.ldexp(torch.ones_like(amax), ex.float())
    bits = encode_e4m3(g / scale.unsqueeze(-1)).reshape(shp)
    return bits, (ex + 127).to(torch.uint8)


# ------------------------------------------------------------------ presets ---

PRESETS = {
    # Tiny decode, fp32.
    "c1_tiny_f32": dict(batch=1, seq_len_range=(256, 256), q_len=1, page_size=16,
                        h_i=4, d_i=32, topk=64, idx_dtype=F32, w_div=1.0,
                        h_s=8, d_qk=80, d_v=64, scale_dim=80, sfa_dtype=F32, sfa_mult=1.0),
    # Decode, bf16, contexts U[4096, 32768].
    "c2_decode_bf16": dict(batch=32, seq_len_range=(4096, 32768), q_len=1, page_size=64,
                           h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                           h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=0.1),
    # The same decode with every context at 32768 tokens.
    "c2_decode_bf16_32k": dict(batch=32, seq_len_range=(32768, 32768), q_len=1, page_size=64,
                               h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                               h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=0.1),
    # Causal prefill, one sequence of 32768 tokens.
    "c3_prefill_bf16": dict(batch=1, seq_len_range=(32768, 32768), q_len=32768, page_size=64,
                            h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                            h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0),
    # Quantised indexer decode, FP8 (per-token K scale, per-token-head Q scale).
    "c4_decode_fp8": dict(batch=64, seq_len_range=(16384, 65536), q_len=1, page_size=64,
                          h_i=64, d_i=128, topk=2048, idx_dtype=FP8, w_div=64.0,
                          h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0,
                          outliers=0.01),
    # Quantised indexer decode, MXFP8 (e8m0 scale per 32 elements).
    "c4_decode_mxfp8": dict(batch=64, seq_len_range=(16384, 65536), q_len=1, page_size=64,
                            h_i=64, d_i=128, topk=2048, idx_dtype=MXFP8, w_div=64.0,
                            h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0,
                            outliers=0.01),
    # The causal prefill of c3_prefill_bf16 with the indexer's q and K cache
    # quantised as in c4_decode_fp8 / c4_decode_mxfp8 (1% outliers at 20 sigma
    # in the indexer's values); the SFA stays bf16 on N(0,1) values.
    "c3_prefill_fp8": dict(batch=1, seq_len_range=(32768, 32768), q_len=32768, page_size=64,
                           h_i=64, d_i=128, topk=2048, idx_dtype=FP8, w_div=64.0,
                           h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0,
                           idx_outliers=0.01),
    "c3_prefill_mxfp8": dict(batch=1, seq_len_range=(32768, 32768), q_len=32768, page_size=64,
                             h_i=64, d_i=128, topk=2048, idx_dtype=MXFP8, w_div=64.0,
                             h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0,
                             idx_outliers=0.01),
    # Long context: 8192-token chunk appended after 122880 cached tokens.
    "c5_chunk_prefill": dict(batch=8, seq_len_range=(131072, 131072), q_len=8192, page_size=64,
                             h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                             h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0),
    # The decode of c2_decode_bf16 with the SFA KV cache in FP8, one scale per
    # tile of 128 elements of each latent row.
    "c2_decode_fp8kv": dict(batch=32, seq_len_range=(4096, 32768), q_len=1, page_size=64,
                            h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                            h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=0.1,
                            kv_dtype=FP8T),
    # Long context: 4-token multi-query decode at 131072 tokens.
    "c5_decode4": dict(batch=8, seq_len_range=(131072, 131072), q_len=4, page_size=64,
                       h_i=64, d_i=128, topk=2048, idx_dtype=BF16, w_div=64.0,
                       h_s=128, d_qk=576, d_v=512, scale_dim=192, sfa_dtype=BF16, sfa_mult=1.0),
}


def _randn(shape, g, device, mult=1.0, outliers=0.0, og=None):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    if outliers > 0.0:
        # each element independently, with probability `outliers`, becomes +-20
        u = torch.rand(shape, generator=og, device=device)
        sgn = torch.where(torch.rand(shape, generator=og, device=device) < 0.5, -1.0, 1.0)
        x = torch.where(u < outliers, 20.0 * sgn, x)
    return x


def _encode(x: torch.Tensor, dtype: str):
    if dtype == F32:
        return x.float().contiguous(), None
    if dtype == BF16:
        return round_bf16(x).contiguous(), None
    if dtype == FP8:
        return quant_fp8_rows(x)
    if dtype == MXFP8:
        return quant_mx_rows(x)
    if dtype == FP8T:
        return quant_fp8_tiles(x)
    raise ValueError(dtype)


def _poison_value(t: torch.Tensor):
    return 0x7F if t.dtype == torch.uint8 else float("nan")


def _fill_pool(pool, scale_pool, logical_fn, n_rows, phys_rows, dtype, chunk_rows):
    """Draw the logical rows chunk by chunk and scatter them into the pool."""
    flat = pool.view(-1, pool.shape[-1])
    sflat = None if scale_pool is None else scale_pool.view(flat.shape[0], -1)
    for r0 in range(0, n_rows, chunk_rows):
        r1 = min(n_rows, r0 + chunk_rows)
        x = logical_fn(r1 - r0)
        bits, sc = _encode(x, dtype)
        flat[phys_rows[r0:r1]] = bits
        if sflat is not None:
            sflat[phys_rows[r0:r1]] = sc.reshape(r1 - r0, -1)


def make_case(name: str, seed: int = 0, device: str = "cpu", value_seed: Optional[int] = None,
              **overrides) -> Case:
    """Build a preset workload (``PRESETS``) with optional overrides, e.g. a
    smaller ``batch``/``seq_len_range``/``q_len`` for fast checks.  ``seed``
    fixes the lengths and the page permutation; ``value_seed`` (default: seed)
    fixes every drawn value, so several value sets can share one layout."""
    p = dict(PRESETS[name])
    p.update(overrides)
    vseed = seed if value_seed is None else value_seed
    B, P = p["batch"], p["page_size"]
    lo, hi = p["seq_len_range"]
    # 1. sequence lengths
    gl = _gen(seed, "seq_lens", "cpu")
    if lo == hi:
        seq_lens = np.full(B, lo, np.int64)
    else:
        seq_lens = torch.randint(lo, hi + 1, (B,), generator=gl).numpy().astype(np.int64)
    q_lens = np.full(B, p["q_len"], np.int64)
    if "q_lens" in p:
        q_lens = np.asarray(p["q_lens"], np.int64)
    if "seq_lens" in p:
        seq_lens = np.asarray(p["seq_lens"], np.int64)
    assert np.all(q_lens <= seq_lens) and np.all(q_lens >= 0)
    # 2. pages: a seeded permutation handed out to sequences in order; one spare
    # poison page (the last one) backs every unused block-table entry.
    npages_seq = (seq_lens + P - 1) // P
    n_real = int(npages_seq.sum())
    num_pages = n_real + 1
    max_pages = int(max(1, npages_seq.max()))
    gp = _gen(seed, "pages", "cpu")
    perm = torch.randperm(n_real, generator=gp).numpy().astype(np.int64)
    bt = np.full((B, max_pages), num_pages - 1, np.int64)
    off = 0
    for b in range(B):
        bt[b, :npages_seq[b]] = perm[off:off + npages_seq[b]]
        off += npages_seq[b]
    # physical row of every logical key, sequences concatenated
    phys = []
    for b in range(B):
        s = np.arange(seq_lens[b])
        phys.append(bt[b, s // P] * P + s % P)
    phys = np.concatenate(phys) if phys else np.zeros(0, np.int64)
    n_keys = int(seq_lens.sum())
    total_q = int(q_lens.sum())
    dev = device
    phys_t = torch.from_numpy(phys).to(dev)

    h_i, d_i, h_s, d_qk, d_v = p["h_i"], p["d_i"], p["h_s"], p["d_qk"], p["d_v"]
    idt, sdt = p["idx_dtype"], p["sfa_dtype"]
    outl = p.get("outliers", 0.0)
    # the indexer's q and K may take outliers of their own (idx_outliers), so a
    # quantised indexer can be tested on C4's recipe beside a plain SFA
    outl_i = p.get("idx_outliers", outl)
    mult = p["sfa_mult"]
    chunk = 1 << 16

    def storage_dtype(dt):
        return {F32: torch.float32, BF16: torch.bfloat16, FP8: torch.uint8, MXFP8: torch.uint8,
                FP8T: torch.uint8}[dt]

    # 3. indexer q
    g, og = _gen(vseed, "q_i", dev), _gen(vseed, "out_q_i", dev)
    q_i, q_i_scale = _encode(_randn((total_q, h_i, d_i), g, dev, 1.0, outl_i, og), idt)
    # 4. indexer K, logical rows scattered into the pool
    k_pool = torch.empty((num_pages, P, d_i), dtype=storage_dtype(idt), device=dev)
    k_pool.fill_(_poison_value(k_pool))
    k_scale = None
    if idt == FP8:
        k_scale = torch.full((num_pages, P), float("nan"), dtype=torch.float32, device=dev)
    elif idt == MXFP8:
        k_scale = torch.full((num_pages, P, d_i // MX_GROUP), 127, dtype=torch.uint8, device=dev)
    g, og = _gen(vseed, "k_i", dev), _gen(vseed, "out_k_i", dev)
    _fill_pool(k_pool, k_scale, lambda n: _randn((n, d_i), g, dev, 1.0, outl_i, og),
               n_keys, phys_t, idt, chunk)
    # 5. head weights U(0,1)/w_div, or U(-1,1)/w_div with w_signed (the
    # weights are projections of the hidden state and may take either sign)
    g = _gen(vseed, "w", dev)
    u = torch.rand((total_q, h_i), generator=g, device=dev)
    if p.get("w_signed", False):
        u = 2.0 * u - 1.0
    w = (u / p["w_div"]).float()
    # 6. SFA q
    g, og = _gen(vseed, "q_s", dev), _gen(vseed, "out_q_s", dev)
    q_s = torch.empty((total_q, h_s, d_qk), dtype=storage_dtype(sdt), device=dev)
    qrows = max(1, (1 << 22) // (h_s * d_qk))
    for r0 in range(0, total_q, qrows):
        r1 = min(total_q, r0 + qrows)
        q_s[r0:r1] = _encode(_randn((r1 - r0, h_s, d_qk), g, dev, mult, outl, og), sdt)[0]
    # 7. latent KV rows (stored in sfa_dtype, or as FP8 tiles)
    kdt = p.get("kv_dtype", sdt)
    assert kdt == sdt or kdt == FP8T
    kv_pool = torch.empty((num_pages, P, d_qk), dtype=storage_dtype(kdt), device=dev)
    kv_pool.fill_(_poison_value(kv_pool))
    kv_scale = None
    if kdt == FP8T:
        kv_scale = torch.full((num_pages, P, -(-d_qk // KV_TILE)), float("nan"),
                              dtype=torch.float32, device=dev)
    g, og = _gen(vseed, "kv", dev), _gen(vseed, "out_kv", dev)
    _fill_pool(kv_pool, kv_scale, lambda n: _randn((n, d_qk), g, dev, mult, outl, og),
               n_keys, phys_t, kdt, chunk)

    cu_q = np.concatenate([[0], np.cumsum(q_lens)])
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(dev)
    return Case(
        name=name, seed=seed, device=dev, batch=B,
        seq_lens=i32(seq_lens), q_lens=i32(q_lens), cu_q=i32(cu_q),
        page_size=P, num_pages=num_pages, max_pages_per_seq=max_pages,
        block_table=i32(bt),
        h_i=h_i, d_i=d_i, topk=p["topk"], idx_dtype=idt,
        q_i=q_i.contiguous(), q_i_scale=None if q_i_scale is None else q_i_scale.contiguous(),
        w=w.contiguous(), k_pool=k_pool, k_scale=k_scale,
        h_s=h_s, d_qk=d_qk, d_v=d_v, softmax_scale=1.0 / math.sqrt(p["scale_dim"]),
        sfa_dtype=sdt, q_s=q_s, kv_pool=kv_pool,
        seq_lens_host=seq_lens.astype(np.int32), q_lens_host=q_lens.astype(np.int32),
        kv_dtype=kdt, kv_scale=kv_scale,
    )


def case_to(case: Case, device: str) -> Case:
    """Copy every tensor of a case to another device (same values)."""
    d = {}
    for f in dataclasses.fields(case):
        v = getattr(case, f.name)
        d[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
    d["device"] = device
    return Case(**d)


def make_prolog(case: Case, seed: int, d_model: int = 7168, ln_eps: float = 1e-6) -> dict:
    """Seeded synthetic inputs of the indexer prolog for a case's new tokens:
    hidden rows x ~ N(0, 1) in bf16; projection weights in the linear-layer
    layout [out][in], bf16, N(0, 1/d_model) so that the projections are of unit
    scale (the head-weight rows further divided by 64, like the head weights
    of the indexer workloads, and of either sign); LayerNorm gamma ~ 1 +
    0.1 N(0, 1), beta ~ 0.1 N(0, 1) in float32."""
    dev, T, H, D = case.device, case.total_q, case.h_i, case.d_i
    sd = 1.0 / math.sqrt(d_model)

    def nrm(tid, shape, mult=1.0):
        return torch.randn(shape, generator=_gen(seed, tid, dev), device=dev, dtype=torch.float32) * mult

    gl = _gen(seed, "pro_ln", dev)
    return dict(
        d_model=d_model, ln_eps=ln_eps,
        x=round_bf16(nrm("pro_x", (T, d_model))).contiguous(),
        w_q=round_bf16(nrm("pro_wq", (H * D, d_model), sd)).contiguous(),
        w_k=round_bf16(nrm("pro_wk", (D, d_model), sd)).contiguous(),
        w_w=round_bf16(nrm("pro_ww", (H, d_model), sd / 64.0)).contiguous(),
        ln_gamma=(1.0 + 0.1 * torch.randn(D, generator=gl, device=dev)).float().contiguous(),
        ln_beta=(0.1 * torch.randn(D, generator=gl, device=dev)).float().contiguous(),
    )
