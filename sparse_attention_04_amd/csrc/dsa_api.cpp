// C ABI of the DSA hot path: argument validation, workspace planning and the
// launch sequence of each entry point (see include/dsa.h for the contract).
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "api_internal.h"
#include "kernels.h"

using namespace dsa;

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dsa_status hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxGrid = 2048;           // workspace is sized for up to this many indexer workgroups
constexpr int kSfaTargetWG = 256;        // SFA workgroups aimed for (one per compute unit) when splitting index rows
constexpr int kSfaRowTile = 32;
constexpr int kSfaMaxRows = 2048;       // index slots one SFA workgroup stages in LDS
constexpr size_t kLdsMax = 160 * 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------ validation ---

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

dsa_status check_batch(const dsa_batch* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
  if (b->batch < 1) return fail(DSA_ERR_INVALID_ARG, "batch->batch must be >= 1 (got %d)", b->batch);
  if (!b->seq_lens || !b->cu_q || !b->block_table)
    return fail(DSA_ERR_INVALID_ARG, "batch->seq_lens, cu_q and block_table must be non-NULL");
  if (!aligned(b->seq_lens, 4) || !aligned(b->cu_q, 4) || !aligned(b->block_table, 4))
    return fail(DSA_ERR_INVALID_ARG, "batch arrays must be 4-byte aligned");
  if (b->max_pages_per_seq < 1) return fail(DSA_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
  if (b->total_q < 0 || b->max_q_len < 0 || b->max_seq_len < 0)
    return fail(DSA_ERR_INVALID_ARG, "negative total_q / max_q_len / max_seq_len");
  if (b->max_q_len > b->max_seq_len) return fail(DSA_ERR_INVALID_ARG, "max_q_len > max_seq_len");
  if (b->total_q > 0 && b->max_q_len == 0) return fail(DSA_ERR_INVALID_ARG, "total_q > 0 but max_q_len == 0");
  if ((int64_t)b->max_q_len * b->batch < b->total_q)
    return fail(DSA_ERR_INVALID_ARG, "total_q exceeds batch * max_q_len");
  return DSA_OK;
}

// `dtype` is the query dtype; with allow_tile8 the cache may instead hold
// FP8 tile-128 rows (the SFA KV cache).
dsa_status check_cache(const dsa_paged_cache* c, const char* name, int dim, int dtype,
                       const dsa_batch* b, bool allow_tile8 = false) {
  if (!c) return fail(DSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!c->data) return fail(DSA_ERR_INVALID_ARG, "%s->data is NULL", name);
  if (!aligned(c->data, 16)) return fail(DSA_ERR_INVALID_ARG, "%s->data must be 16-byte aligned", name);
  if (c->dtype != DSA_MXFP8_E4M3 && !aligned(c->scale, 4))
    return fail(DSA_ERR_INVALID_ARG, "%s->scale must be 4-byte aligned", name);
  if (c->dtype != dtype && !(allow_tile8 && c->dtype == DSA_FP8_E4M3_TILE128))
    return fail(DSA_ERR_INVALID_ARG, "%s->dtype %d differs from the query dtype %d", name, c->dtype, dtype);
  if (c->dim != dim) return fail(DSA_ERR_INVALID_ARG, "%s->dim %d differs from %d", name, c->dim, dim);
  if (c->page_size < 1 || c->page_size > 4096 || (c->page_size & (c->page_size - 1)))
    return fail(DSA_ERR_UNSUPPORTED, "%s->page_size %d is not a power of two in [1, 4096]", name, c->page_size);
  if (c->num_pages < 1) return fail(DSA_ERR_INVALID_ARG, "%s->num_pages must be >= 1", name);
  if ((int64_t)b->max_pages_per_seq * c->page_size < b->max_seq_len)
    return fail(DSA_ERR_INVALID_ARG, "max_pages_per_seq * page_size < max_seq_len");
  if ((int64_t)c->num_pages * c->page_size >= (1ll << 31))
    return fail(DSA_ERR_UNSUPPORTED, "%s holds 2^31 rows or more", name);
  const bool need_scale = (c->dtype == DSA_FP8_E4M3 || c->dtype == DSA_MXFP8_E4M3 ||
                           c->dtype == DSA_FP8_E4M3_TILE128);
  if (need_scale && !c->scale) return fail(DSA_ERR_INVALID_ARG, "%s->scale is NULL for a quantised dtype", name);
  return DSA_OK;
}

dsa_status check_indexer(const dsa_batch* b, const dsa_indexer_args* a) {
  if (!a) return fail(DSA_ERR_INVALID_ARG, "indexer args are NULL");
  // arrays with one entry per query token may be NULL when there is none
  const bool any_q = b->total_q > 0;
  if (any_q && (!a->q || !a->head_weights)) return fail(DSA_ERR_INVALID_ARG, "indexer q / head_weights are NULL");
  if (!aligned(a->q, 16) || !aligned(a->head_weights, 4) || (a->q_dtype == DSA_FP8_E4M3 && !aligned(a->q_scale, 4)))
    return fail(DSA_ERR_INVALID_ARG, "indexer q must be 16-byte aligned, head_weights and fp8 q_scale 4-byte aligned");
  if (a->topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", a->topk);
  if (a->q_dtype < DSA_F32 || a->q_dtype > DSA_MXFP8_E4M3) return fail(DSA_ERR_INVALID_ARG, "unknown indexer dtype %d", a->q_dtype);
  const bool ok_shape = (a->q_dtype == DSA_F32 && a->n_heads == 4 && a->head_dim == 32) ||
                        (a->q_dtype != DSA_F32 && a->n_heads == 64 && a->head_dim == 128);
  if (!ok_shape)
    return fail(DSA_ERR_UNSUPPORTED, "indexer shape (dtype %d, heads %d, dim %d) is not compiled in; supported: f32 4x32, bf16/fp8/mxfp8 64x128",
                a->q_dtype, a->n_heads, a->head_dim);
  if (any_q && (a->q_dtype == DSA_FP8_E4M3 || a->q_dtype == DSA_MXFP8_E4M3) && !a->q_scale)
    return fail(DSA_ERR_INVALID_ARG, "indexer q_scale is NULL for a quantised dtype");
  return check_cache(a->k_cache, "k_cache", a->head_dim, a->q_dtype, b);
}

dsa_status check_sfa(const dsa_batch* b, const dsa_sfa_args* a) {
  if (!a) return fail(DSA_ERR_INVALID_ARG, "sfa args are NULL");
  if (!a->q && b->total_q > 0) return fail(DSA_ERR_INVALID_ARG, "sfa q is NULL");
  if (!aligned(a->q, 16)) return fail(DSA_ERR_INVALID_ARG, "sfa q must be 16-byte aligned");
  if (a->q_dtype != DSA_F32 && a->q_dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "sfa dtype %d not supported (f32, bf16)", a->q_dtype);
  const bool ok_shape = (a->q_dtype == DSA_F32 && a->n_heads == 8 && a->qk_dim == 80 && a->v_dim == 64) ||
                        (a->q_dtype == DSA_BF16 && a->n_heads == 128 && a->qk_dim == 576 && a->v_dim == 512);
  if (!ok_shape)
    return fail(DSA_ERR_UNSUPPORTED, "sfa shape (dtype %d, heads %d, qk %d, v %d) is not compiled in; supported: f32 8x80/64, bf16 128x576/512",
                a->q_dtype, a->n_heads, a->qk_dim, a->v_dim);
  if (!(a->softmax_scale > 0.f) || !(a->softmax_scale < 1e30f)) return fail(DSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  return check_cache(a->kv_cache, "kv_cache", a->qk_dim, a->q_dtype, b, true);
}

int dt_kernel(int d) {
  switch (d) {
    case DSA_F32: return kF32;
    case DSA_BF16: return kBF16;
    case DSA_FP8_E4M3: return kFP8;
    default: return kMX;
  }
}

BatchView view_of(const dsa_batch* b, int page_size) {
  BatchView v;
  v.batch = b->batch;
  v.seq_lens = b->seq_lens;
  v.cu_q = b->cu_q;
  v.block_table = b->block_table;
  v.max_pages = b->max_pages_per_seq;
  v.page_size = page_size;
  v.page_shift = __builtin_ctz((unsigned)page_size);
  v.total_q = b->total_q;
  return v;
}

// ------------------------------------------------------ workspace planning ---

struct SfaPlan {
  int splits, rows_per_split, hsplit;
  size_t part_o_bytes, part_ml_bytes;
};

SfaPlan plan_sfa(const dsa_batch* b, int H, int Dv, int topk, bool bf16, bool kv8) {
  SfaPlan pl{};
  // A workgroup serves one (token, range of index slots) with all heads.
  // Over an FP8 KV cache two workgroups share a token's heads (the registers
  // of the per-tile scale products do not fit next to all 128).  The slot
  // ranges are split until about kSfaTargetWG workgroups exist.  Ranges are
  // multiples of the row tile and hold at most kSfaMaxRows slots.
  pl.hsplit = (bf16 && kv8) ? 2 : 1;
  const int64_t units = std::max<int64_t>(1, (int64_t)b->total_q * pl.hsplit);
  int splits = (int)std::max<int64_t>(1, std::min<int64_t>(std::max(1, topk / 64), kSfaTargetWG / units));
  splits = std::max(splits, (topk + kSfaMaxRows - 1) / kSfaMaxRows);
  int rps = (int)align_up((size_t)((topk + splits - 1) / splits), kSfaRowTile);
  splits = (topk + rps - 1) / rps;
  pl.splits = splits;
  pl.rows_per_split = rps;
  if (splits > 1) {
    pl.part_o_bytes = align_up((size_t)b->total_q * splits * H * Dv * (bf16 ? 2 : 4), 256);
    pl.part_ml_bytes = align_up((size_t)b->total_q * splits * H * 4, 256);
  }
  return pl;
}

size_t indexer_bytes(const dsa_batch* b) {
  return align_up(indexer_ws_bytes(b->batch, b->total_q, kMaxGrid), 256);
}

struct DeviceInfo {
  int dev = -1, cus = 0;
};
thread_local DeviceInfo g_dev;

dsa_status device_info(DeviceInfo& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (g_dev.dev != dev) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    g_dev.dev = dev;
    g_dev.cus = cus;
  }
  out = g_dev;
  return DSA_OK;
}

bool debug_mode() {
  const char* s = getenv("DSA_DEBUG");
  return s && s[0] == '1';
}

// DSA_TEST_FORCE_TIMEOUT=1 (tests only): every cross-workgroup wait of the
// decode indexer gives up after a few sleeps, as a failed co-residency would
// make it, so the failure path can be checked while every kernel still ends.
bool force_timeout_mode() {
  const char* s = getenv("DSA_TEST_FORCE_TIMEOUT");
  return s && s[0] == '1';
}

// DSA_TEST_WITHHOLD_READY=1 (tests only): the fused decode kernel's indexer
// never publishes a sequence's rows and its attention tasks give up waiting
// after a few sleeps, so the tasks' failure path (an empty range and the
// error bit) can be checked while every kernel still ends.
bool withhold_ready_mode() {
  const char* s = getenv("DSA_TEST_WITHHOLD_READY");
  return s && s[0] == '1';
}

// The boundary-bin handoff of the decode indexer (the sequence's last
// workgroup chooses among the keys of the first pass's boundary bin) is taken
// when that bin holds at most kHandoffCap keys.  DSA_INDEXER_HANDOFF_CAP=n
// lowers the limit (0 turns the handoff off, so every query runs the later
// radix passes); tests use it to run both paths on the same inputs.
int handoff_cap() {
  const char* s = getenv("DSA_INDEXER_HANDOFF_CAP");
  if (!s || !s[0]) return kHandoffCap;
  const long v = strtol(s, nullptr, 10);
  return (int)std::max<long>(0, std::min<long>(v, kHandoffCap));
}

// DSA_PROFILE=1: kernels record per-phase clock sums of their first workgroup
// in the last kProfileBytes of the workspace.
constexpr size_t kProfileBytes = 256;
bool profile_mode() {
  const char* s = getenv("DSA_PROFILE");
  return s && s[0] == '1';
}

// ------------------------------------------------------------ launchers ---

IndexerDecodeParams indexer_decode_params(const dsa_batch* b, const dsa_indexer_args* a, int32_t* idx_out,
                                          uint32_t* ws, int grid, int chunk_cap, int stage) {
  IndexerDecodeParams p{};
  p.bv = view_of(b, a->k_cache->page_size);
  p.q = a->q;
  p.q_scale = a->q_scale;
  p.w = a->head_weights;
  p.k_data = a->k_cache->data;
  p.k_scale = a->k_cache->scale;
  p.topk = a->topk;
  p.idx_out = idx_out;
  p.ws = ws;
  p.ws_nseq = b->batch;
  p.ws_nq = b->total_q;
  p.ws_grid_pad = (kMaxGrid + 31) / 32 * 32;
  p.grid = grid;
  p.chunk_cap = chunk_cap;
  p.stage_pages = stage;
  p.spin_limit = kSpinLimit;
  p.barrier_slack = 0;
  p.ready_spin_limit = kSpinLimit;
  p.publish_ready = 1;
  p.cand_cap = handoff_cap();
  if (withhold_ready_mode()) {
    // test hook: no rows are handed over and the tasks stop waiting quickly
    p.ready_spin_limit = 64;
    p.publish_ready = 0;
  }
  if (force_timeout_mode()) {
    // test hook: no barrier can complete, and every wait gives up quickly
    p.spin_limit = 64;
    p.barrier_slack = 1u << 30;
  }
  return p;
}


dsa_status run_indexer_decode(const dsa_batch* b, const dsa_indexer_args* a, int32_t* idx_out,
                              uint32_t* ws, hipStream_t st) {
  if (b->total_q == 0) return DSA_OK;
  const int maxq = (b->max_q_len <= 1) ? 1 : kMaxDecodeQ;
  if (b->max_q_len > kMaxDecodeQ)
    return fail(DSA_ERR_UNSUPPORTED, "decode indexer handles at most %d query tokens per sequence (max_q_len %d); use dsa_fused_prefill",
                kMaxDecodeQ, b->max_q_len);
  DeviceInfo di;
  dsa_status s = device_info(di);
  if (s != DSA_OK) return s;
  const int P = a->k_cache->page_size;
  const int maxp = (b->max_seq_len + P - 1) / P;
  const int dt = dt_kernel(a->q_dtype);

  hipError_t e = hipSuccess;
  // Pick the largest co-resident grid (2 or 1 workgroups per CU) and the
  // largest sub-batch whose per-workgroup score buffer fits in LDS.
  int grid = 0, chunk_cap = 0, sub = 0, stage = 0;
  for (int per_cu = 2; per_cu >= 1 && grid == 0; per_cu--) {
    const int G = std::min(kMaxGrid, per_cu * di.cus);
    for (int nb = std::min(b->batch, G / 2); nb >= 1; nb = (nb > 1) ? nb / 2 : 0) {
      const int64_t cap_pages = ((int64_t)nb * std::max(1, maxp) + (G - nb) - 1) / (G - nb);
      // rounded up to 8 keys: the kernel's selection sweeps read 8 scores at once
      const int64_t cap_keys = (cap_pages * P + 7) / 8 * 8;
      // a workgroup's keys span at most cap_pages pages (+1 when P does not
      // divide its range start, which the page-aligned assignment avoids)
      const int64_t stage_pages = cap_pages + 1;
      const size_t lds = indexer_decode_lds_bytes(dt, maxq, (int)std::min<int64_t>(cap_keys, 1 << 24),
                                                  (int)std::min<int64_t>(stage_pages, 1 << 24));
      if (lds > kLdsMax) continue;
      int occ = 0;
      e = indexer_decode_occupancy(dt, a->n_heads, a->head_dim, maxq, lds, &occ);
      if (e != hipSuccess) return hip_fail(e, "occupancy query");
      if (occ * di.cus < G) break;  // try fewer workgroups per CU
      grid = G;
      chunk_cap = (int)cap_keys;
      stage = (int)stage_pages;
      sub = nb;
      break;
    }
  }
  if (grid == 0) return fail(DSA_ERR_UNSUPPORTED, "context too long for the decode indexer's on-chip score buffer");

  IndexerDecodeParams p = indexer_decode_params(b, a, idx_out, ws, grid, chunk_cap, stage);
  for (int b0 = 0; b0 < b->batch; b0 += sub) {
    const int nb = std::min(sub, b->batch - b0);
    p.bv = view_of(b, P);
    p.bv.batch = nb;
    p.bv.seq_lens = b->seq_lens + b0;
    p.bv.cu_q = b->cu_q + b0;
    p.bv.block_table = b->block_table + (size_t)b0 * b->max_pages_per_seq;
    p.seq_base = b0;
    e = launch_indexer_decode(dt, a->n_heads, a->head_dim, maxq, p, st);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
  }
  return debug_mode() ? take_error_bits(ws, st) : DSA_OK;
}

dsa_status run_indexer_prefill(const dsa_batch* b, const dsa_indexer_args* a, int32_t* idx_out, hipStream_t st) {
  if (b->total_q == 0) return DSA_OK;
  if (a->q_dtype != DSA_BF16 && a->q_dtype != DSA_FP8_E4M3 && a->q_dtype != DSA_MXFP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "the prefill indexer (more than %d query tokens per sequence) is built for bf16, FP8 and MXFP8 only", kMaxDecodeQ);
  if (a->q_dtype == DSA_MXFP8_E4M3 && !aligned(a->k_cache->scale, 4))
    return fail(DSA_ERR_INVALID_ARG, "the prefill indexer reads MXFP8 key scales as 4-byte words: k_cache->scale must be 4-byte aligned");
  if (a->topk > indexer_prefill_max_topk())
    return fail(DSA_ERR_UNSUPPORTED, "prefill topk %d above %d", a->topk, indexer_prefill_max_topk());
  const int P = a->k_cache->page_size;
  if ((b->max_seq_len + P - 1) / P > indexer_prefill_max_pages())
    return fail(DSA_ERR_UNSUPPORTED, "prefill context of %d pages above %d", (b->max_seq_len + P - 1) / P,
                indexer_prefill_max_pages());
  IndexerPrefillParams p{};
  p.bv = view_of(b, P);
  p.q = a->q;
  p.q_scale = a->q_scale;
  p.w = a->head_weights;
  p.k_data = a->k_cache->data;
  p.k_scale = a->k_cache->scale;
  p.topk = a->topk;
  p.idx_out = idx_out;
  p.grid = indexer_prefill_grid(b->total_q, b->batch);
  hipError_t e = launch_indexer_prefill(dt_kernel(a->q_dtype), a->n_heads, a->head_dim, p, st);
  if (e != hipSuccess) return hip_fail(e, "prefill indexer launch");
  return DSA_OK;
}

// Decode-shaped batches (at most kMaxDecodeQ new tokens per sequence) use the
// cross-workgroup decode indexer; longer query runs use the zigzag prefill one.
dsa_status run_indexer(const dsa_batch* b, const dsa_indexer_args* a, int32_t* idx_out, uint32_t* ws,
                       hipStream_t st) {
  if (b->max_q_len <= kMaxDecodeQ) return run_indexer_decode(b, a, idx_out, ws, st);
  return run_indexer_prefill(b, a, idx_out, st);
}

SfaParams sfa_params(const dsa_batch* b, const dsa_sfa_args* a, const int32_t* idx, int topk, void* out,
                     float* lse, unsigned char* ws, const SfaPlan& pl) {
  SfaParams p{};
  p.bv = view_of(b, a->kv_cache->page_size);
  p.q = a->q;
  p.kv = a->kv_cache->data;
  p.kv8 = (a->kv_cache->dtype == DSA_FP8_E4M3_TILE128) ? 1 : 0;
  p.kv_scale = p.kv8 ? (const float*)a->kv_cache->scale : nullptr;
  p.idx = idx;
  p.topk = topk;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  p.splits = pl.splits;
  p.hsplit = pl.hsplit;
  p.rows_per_split = pl.rows_per_split;
  // Launches with fewer query tokens than workgroup slots (decode) are bound
  // by memory and latency, so the matrix units can afford the weight
  // residuals; large prefill launches are bound by the matrix units and use
  // bf16 weights (each within 2^-8 relative).
  p.precise_weights = (int64_t)b->total_q < kSfaTargetWG ? 1 : 0;
  p.out = out;
  p.lse = lse;
  p.part_o = (float*)ws;
  p.part_ml = (float*)(ws + pl.part_o_bytes);
  p.dbg = profile_mode() ? (unsigned long long*)(ws + pl.part_o_bytes + pl.part_ml_bytes) : nullptr;
  return p;
}

dsa_status run_sfa(const dsa_batch* b, const dsa_sfa_args* a, const int32_t* idx, int topk,
                   void* out, float* lse, unsigned char* ws, hipStream_t st) {
  if (b->total_q == 0) return DSA_OK;
  const bool bf16 = (a->q_dtype == DSA_BF16);
  const bool kv8 = (a->kv_cache->dtype == DSA_FP8_E4M3_TILE128);
  const SfaPlan pl = plan_sfa(b, a->n_heads, a->v_dim, topk, bf16, kv8);
  const SfaParams p = sfa_params(b, a, idx, topk, out, lse, ws, pl);
  const int dt = dt_kernel(a->q_dtype);
  hipError_t e = launch_sfa(dt, a->n_heads, a->qk_dim, a->v_dim, p, st);
  if (e != hipSuccess) return hip_fail(e, "sfa launch");
  e = launch_sfa_combine(dt, a->n_heads, a->v_dim, p, st);
  if (e != hipSuccess) return hip_fail(e, "sfa combine launch");
  return DSA_OK;
}


// The fused decode kernel (indexer and attention in one launch, the combine
// after it) serves a decode call when its shapes have an instance, the whole
// batch fits one indexer launch of one workgroup per CU (every sequence with
// at least two workgroups' worth of slack, as for the indexer alone), and the
// attention's tasks fit that grid, one per workgroup.  Otherwise, or with
// DSA_FUSED_KERNEL=0, the call runs the two stages as separate kernels.
// `launched` tells which happened.
bool fused_kernel_enabled() {
  const char* s = getenv("DSA_FUSED_KERNEL");
  return !(s && s[0] == '0');
}


dsa_status run_fused_kernel(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa, int32_t* idx,
                            void* out, float* lse, uint32_t* ws, unsigned char* sfa_ws, hipStream_t st,
                            bool& launched) {
  launched = false;
  if (!fused_kernel_enabled() || b->total_q == 0 || b->max_q_len > kMaxDecodeQ) return DSA_OK;
  if (sa->q_dtype != DSA_BF16 || sa->kv_cache->dtype == DSA_FP8_E4M3_TILE128 || sa->n_heads != 128 ||
      sa->qk_dim != 576 || sa->v_dim != 512)
    return DSA_OK;
  const int maxq = (b->max_q_len <= 1) ? 1 : kMaxDecodeQ;
  const int dt = dt_kernel(ia->q_dtype);
  const SfaPlan pl = plan_sfa(b, sa->n_heads, sa->v_dim, ia->topk, true, false);
  const bool lo = (int64_t)b->total_q < kSfaTargetWG;
  if (!fused_decode_supported(dt, maxq, lo) || pl.hsplit != 1 || pl.rows_per_split > fused_decode_max_rows())
    return DSA_OK;
  DeviceInfo di;
  dsa_status s = device_info(di);
  if (s != DSA_OK) return s;
  const int G = std::min(kMaxGrid, di.cus) / 8 * 8;
  const int64_t tasks = 8 * (int64_t)((b->total_q + 7) / 8) * pl.splits;
  if (G < 8 || tasks > G || b->batch > G / 2) return DSA_OK;
  // the indexer's geometry for one launch over the whole batch, as the
  // indexer alone computes it
  const int P = ia->k_cache->page_size;
  const int maxp = (b->max_seq_len + P - 1) / P;
  const int64_t cap_pages = ((int64_t)b->batch * std::max(1, maxp) + (G - b->batch) - 1) / (G - b->batch);
  const int64_t cap_keys = (cap_pages * P + 7) / 8 * 8;
  const int64_t stage_pages = cap_pages + 1;
  if (cap_keys > (1 << 24)) return DSA_OK;
  const size_t lds = std::max(indexer_decode_lds_bytes(dt, maxq, (int)cap_keys, (int)stage_pages),
                              fused_decode_sfa_lds_bytes(pl.rows_per_split));
  if (lds > kLdsMax) return DSA_OK;
  int occ = 0;
  hipError_t e = fused_decode_occupancy(dt, maxq, lo, lds, &occ);
  if (e != hipSuccess) return hip_fail(e, "occupancy query (fused decode)");
  if (occ < 1) return DSA_OK;
  const IndexerDecodeParams ip = indexer_decode_params(b, ia, idx, ws, G, (int)cap_keys, (int)stage_pages);
  SfaParams sp = sfa_params(b, sa, idx, ia->topk, out, lse, sfa_ws, pl);
  sp.epoch_word = ws + kWsEpochWord;   // advanced by the combine (or the bump) after the kernel
  e = launch_fused_decode(dt, maxq, ip, sp, lds, st);
  if (e != hipSuccess) return hip_fail(e, "fused decode launch");
  e = sp.splits > 1 ? launch_sfa_combine(kBF16, sa->n_heads, sa->v_dim, sp, st) : launch_fused_epoch_bump(sp.epoch_word, st);
  if (e != hipSuccess) return hip_fail(e, "sfa combine launch");
  launched = true;
  return debug_mode() ? take_error_bits(ws, st) : DSA_OK;
}

// Workspace layout.  The zero state (the decode indexer's cross-workgroup
// counters and histograms, left zero by every call) sits at the start of the
// workspace and the scratch (index rows, attention partials) at its end, so a
// workspace shared by calls of different shapes never finds one call's scratch
// where another keeps its state (it needs room for the largest state and the
// largest scratch at once).  kLayoutSlack covers aligning the scratch down.
constexpr size_t kLayoutSlack = 256;
unsigned char* scratch_at_end(void* ws, size_t ws_bytes, size_t scratch_bytes) {
  const uintptr_t end = ((uintptr_t)ws + ws_bytes) & ~(uintptr_t)255;
  return (unsigned char*)(end - scratch_bytes);
}

size_t sfa_bytes(const dsa_batch* b, const dsa_sfa_args* a, int topk) {
  const SfaPlan pl = plan_sfa(b, a->n_heads, a->v_dim, topk, a->q_dtype == DSA_BF16,
                             a->kv_cache && a->kv_cache->dtype == DSA_FP8_E4M3_TILE128);
  return pl.part_o_bytes + pl.part_ml_bytes + kProfileBytes;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int32_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err.c_str(); }

dsa_status dsa_take_device_errors(void* ws, void* stream) {
  g_err.clear();
  void* p = ws;
  if (!p) {
    dsa_status s = dsa::noalloc_scratch_if_set_up(&p);
    if (s != DSA_OK || !p) return s;
  }
  if (!aligned(p, 16)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  return dsa::take_error_bits((uint32_t*)p, (hipStream_t)stream);
}

size_t dsa_workspace_size(int32_t op, const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa) {
  if (!b || b->batch < 1 || b->total_q < 0) return 0;
  const int topk = ia ? ia->topk : 2048;
  switch (op) {
    case DSA_OP_INDEXER_TOPK:
      return indexer_bytes(b);
    case DSA_OP_SPARSE_ATTN:
      return sa ? sfa_bytes(b, sa, topk) + kLayoutSlack : 0;
    case DSA_OP_FUSED_DECODE:
      // zero state | ... | index rows, attention partials
      if (!ia || !sa) return 0;
      return indexer_bytes(b) + align_up((size_t)b->total_q * std::max(1, topk) * 4, 256) + sfa_bytes(b, sa, topk) +
             kLayoutSlack;
    case DSA_OP_FUSED_PREFILL:
      // scratch only (the prefill indexer keeps no state)
      if (!ia || !sa) return 0;
      return align_up((size_t)b->total_q * std::max(1, topk) * 4, 256) + sfa_bytes(b, sa, topk) + kLayoutSlack;
    default:
      return 0;
  }
}

dsa_status dsa_indexer_topk(const dsa_batch* b, const dsa_indexer_args* a, int32_t* idx_out,
                            void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status s = check_batch(b);
  if (s == DSA_OK) s = check_indexer(b, a);
  if (s != DSA_OK) return s;
  if (!idx_out && b->total_q > 0) return fail(DSA_ERR_INVALID_ARG, "idx_out is NULL");
  if (!aligned(idx_out, 4) || !aligned(ws, 16)) return fail(DSA_ERR_INVALID_ARG, "idx_out must be 4-byte, ws 16-byte aligned");
  const size_t need = dsa_workspace_size(DSA_OP_INDEXER_TOPK, b, a, nullptr);
  if (ws_bytes < need || (!ws && need)) return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  if (debug_mode()) {
    s = debug_check_batch(b, a->k_cache->num_pages, a->k_cache->page_size, nullptr, 0, (hipStream_t)stream);
    if (s != DSA_OK) return s;
  }
  return run_indexer(b, a, idx_out, (uint32_t*)ws, (hipStream_t)stream);
}

dsa_status dsa_sparse_attn(const dsa_batch* b, const dsa_sfa_args* a, const int32_t* idx, int32_t topk,
                           void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status s = check_batch(b);
  if (s == DSA_OK) s = check_sfa(b, a);
  if (s != DSA_OK) return s;
  if ((!idx || !out) && b->total_q > 0) return fail(DSA_ERR_INVALID_ARG, "idx / out is NULL");
  if (!aligned(idx, 4) || !aligned(out, 16) || !aligned(lse, 4) || !aligned(ws, 16))
    return fail(DSA_ERR_INVALID_ARG, "out and ws must be 16-byte, idx and lse 4-byte aligned");
  if (topk < 1) return fail(DSA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", topk);
  const size_t need = sfa_bytes(b, a, topk) + kLayoutSlack;
  if (ws_bytes < need || (!ws && need)) return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  if (debug_mode()) {
    s = debug_check_batch(b, a->kv_cache->num_pages, a->kv_cache->page_size, idx, topk, (hipStream_t)stream);
    if (s != DSA_OK) return s;
  }
  return run_sfa(b, a, idx, topk, out, lse, scratch_at_end(ws, ws_bytes, sfa_bytes(b, a, topk)), (hipStream_t)stream);
}

dsa_status dsa_fused_decode(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa,
                            void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                            void* stream) {
  g_err.clear();
  return dsa::fused_decode_impl(b, ia, sa, out, lse, idx_out, ws, ws_bytes, stream, false);
}

}  // extern "C"

namespace dsa {

dsa_status fused_decode_impl(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa,
                             void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                             void* stream, bool validate_only) {
  dsa_status s = check_batch(b);
  if (s == DSA_OK) s = check_indexer(b, ia);
  if (s == DSA_OK) s = check_sfa(b, sa);
  if (s != DSA_OK) return s;
  if (!out && b->total_q > 0) return fail(DSA_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16) || !aligned(lse, 4) || !aligned(idx_out, 4) || !aligned(ws, 16))
    return fail(DSA_ERR_INVALID_ARG, "out and ws must be 16-byte, lse and idx_out 4-byte aligned");
  if (ia->k_cache->page_size != sa->kv_cache->page_size)
    return fail(DSA_ERR_INVALID_ARG, "k_cache and kv_cache must share the page size (one block table)");
  if (validate_only) return DSA_OK;
  const size_t need = dsa_workspace_size(DSA_OP_FUSED_DECODE, b, ia, sa);
  if (ws_bytes < need || (!ws && need)) return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t rows = align_up((size_t)b->total_q * ia->topk * 4, 256);
  unsigned char* scr = scratch_at_end(ws, ws_bytes, rows + sfa_bytes(b, sa, ia->topk));
  int32_t* idx = idx_out ? idx_out : (int32_t*)scr;
  hipStream_t st = (hipStream_t)stream;
  if (debug_mode()) {
    s = debug_check_batch(b, std::min(ia->k_cache->num_pages, sa->kv_cache->num_pages), ia->k_cache->page_size,
                          nullptr, 0, st);
    if (s != DSA_OK) return s;
  }
  bool launched = false;
  s = run_fused_kernel(b, ia, sa, idx, out, lse, (uint32_t*)ws, scr + rows, st, launched);
  if (s != DSA_OK || launched) return s;
  s = run_indexer(b, ia, idx, (uint32_t*)ws, st);
  if (s != DSA_OK) return s;
  return run_sfa(b, sa, idx, ia->topk, out, lse, scr + rows, st);
}

size_t fused_decode_state_bytes(const dsa_batch* b) { return indexer_bytes(b); }

// Wait for `st` and report (once) the error bits the bounded waits set: with
// DSA_DEBUG after every indexer launch, and in dsa_take_device_errors.
dsa_status take_error_bits(uint32_t* ws, hipStream_t st) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "indexer (error-bit sync)");
  uint32_t flags = 0;
  e = hipMemcpy(&flags, ws, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "indexer (error-bit read)");
  if (flags) {
    const uint32_t zero = 0;
    e = hipMemcpy(ws, &zero, 4, hipMemcpyHostToDevice);   // report each failure once
    if (e != hipSuccess) return hip_fail(e, "indexer (error-bit reset)");
    return fail(DSA_ERR_HIP, "indexer reported error bits 0x%x (bounded wait expired or LDS bound)", flags);
  }
  return DSA_OK;
}

dsa_status set_error(dsa_status st, const char* msg) { return fail(st, "%s", msg); }
void clear_error() { g_err.clear(); }

}  // namespace dsa

extern "C" {

size_t dsa_prolog_workspace_size(const dsa_batch* b, const dsa_prolog_args* a) {
  if (!b || !a || b->total_q < 0 || a->n_heads < 1 || a->head_dim < 1 || a->d_model < 1) return 0;
  const size_t words = prolog_part_words(b->total_q, std::max(a->d_model, prolog_d_model_unit()), a->n_heads,
                                         a->head_dim);
  return align_up((size_t)b->total_q * a->n_heads * a->head_dim * 2, 256) + align_up(words * 4, 256) + 256;
}

dsa_status dsa_indexer_prolog(const dsa_batch* b, const dsa_prolog_args* a, void* q_out, void* q_scale_out,
                              float* w_out, const dsa_paged_cache* kc, void* q_bf16_out, void* k_bf16_out,
                              void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status s = check_batch(b);
  if (s != DSA_OK) return s;
  if (!a) return fail(DSA_ERR_INVALID_ARG, "prolog args are NULL");
  const bool any_q = b->total_q > 0;   // x and the outputs have one row per query token
  if ((any_q && !a->x) || !a->w_q || !a->w_k || !a->w_w || !a->ln_gamma || !a->ln_beta)
    return fail(DSA_ERR_INVALID_ARG, "prolog x, weights and LayerNorm parameters must be non-NULL");
  if (a->out_dtype != DSA_BF16 && a->out_dtype != DSA_FP8_E4M3 && a->out_dtype != DSA_MXFP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "prolog out_dtype %d: bf16, fp8 or mxfp8", a->out_dtype);
  if (a->head_dim != 128 || a->n_heads < 32 || a->n_heads % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "prolog shape (heads %d, dim %d) not compiled in: head_dim 128, heads a multiple of 32",
                a->n_heads, a->head_dim);
  if (a->d_model < prolog_d_model_unit() || a->d_model % prolog_d_model_unit() != 0)
    return fail(DSA_ERR_UNSUPPORTED, "prolog d_model %d must be a positive multiple of %d", a->d_model,
                prolog_d_model_unit());
  if (!(a->ln_eps >= 0.f) || !(a->ln_eps < 1e30f)) return fail(DSA_ERR_INVALID_ARG, "ln_eps must be finite and >= 0");
  const bool quant = a->out_dtype != DSA_BF16;
  if (any_q && (!q_out || !w_out || (quant && !q_scale_out)))
    return fail(DSA_ERR_INVALID_ARG, "q_out, w_out (and q_scale_out for a quantised dtype) must be non-NULL");
  if (!aligned(a->x, 16) || !aligned(a->w_q, 16) || !aligned(a->w_k, 16) || !aligned(a->w_w, 16) ||
      !aligned(q_out, 16) || !aligned(w_out, 16) || !aligned(q_bf16_out, 16) || !aligned(k_bf16_out, 4) ||
      !aligned(a->ln_gamma, 4) || !aligned(a->ln_beta, 4) || !aligned(q_scale_out, 4) || !aligned(ws, 16))
    return fail(DSA_ERR_INVALID_ARG, "prolog x, weights, q_out, q_bf16_out, w_out and ws must be 16-byte aligned, "
                                     "the other arrays 4-byte aligned");
  s = check_cache(kc, "k_cache", a->head_dim, a->out_dtype, b);
  if (s != DSA_OK) return s;
  const size_t need = dsa_prolog_workspace_size(b, a);
  if (ws_bytes < need || (!ws && need)) return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  if (b->total_q == 0) return DSA_OK;
  if (debug_mode()) {
    s = debug_check_batch(b, kc->num_pages, kc->page_size, nullptr, 0, (hipStream_t)stream);
    if (s != DSA_OK) return s;
  }
  unsigned char* w = (unsigned char*)ws;
  PrologParams p{};
  p.bv = view_of(b, kc->page_size);
  p.total_q = b->total_q;
  p.d_model = a->d_model;
  p.H = a->n_heads;
  p.D = a->head_dim;
  p.x = a->x;
  p.w_q = a->w_q;
  p.w_k = a->w_k;
  p.w_w = a->w_w;
  p.ln_gamma = a->ln_gamma;
  p.ln_beta = a->ln_beta;
  p.ln_eps = a->ln_eps;
  p.q_bf16 = !quant ? q_out : (q_bf16_out ? q_bf16_out : (void*)w);
  p.q_out = q_out;
  p.q_scale_out = q_scale_out;
  p.w_out = w_out;
  p.part = (float*)(w + align_up((size_t)b->total_q * a->n_heads * a->head_dim * 2, 256));
  p.k_bf16_out = k_bf16_out;
  p.k_data = const_cast<void*>(kc->data);
  p.k_scale = const_cast<void*>(kc->scale);
  hipError_t e = launch_prolog(dt_kernel(a->out_dtype), p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prolog launch");
  return DSA_OK;
}

dsa_status dsa_fused_prefill(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa,
                             int32_t q_block, void* out, float* lse, int32_t* idx_out, void* ws,
                             size_t ws_bytes, void* stream) {
  g_err.clear();
  dsa_status s = check_batch(b);
  if (s == DSA_OK) s = check_indexer(b, ia);
  if (s == DSA_OK) s = check_sfa(b, sa);
  if (s != DSA_OK) return s;
  if (!out && b->total_q > 0) return fail(DSA_ERR_INVALID_ARG, "out is NULL");
  if (!aligned(out, 16) || !aligned(lse, 4) || !aligned(idx_out, 4) || !aligned(ws, 16))
    return fail(DSA_ERR_INVALID_ARG, "out and ws must be 16-byte, lse and idx_out 4-byte aligned");
  if (q_block != 64) return fail(DSA_ERR_UNSUPPORTED, "q_block must be 64 (got %d)", q_block);
  if (ia->k_cache->page_size != sa->kv_cache->page_size)
    return fail(DSA_ERR_INVALID_ARG, "k_cache and kv_cache must share the page size (one block table)");
  const size_t need = dsa_workspace_size(DSA_OP_FUSED_PREFILL, b, ia, sa);
  if (ws_bytes < need || (!ws && need)) return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
  const size_t rows = align_up((size_t)b->total_q * ia->topk * 4, 256);
  unsigned char* scr = scratch_at_end(ws, ws_bytes, rows + sfa_bytes(b, sa, ia->topk));
  int32_t* idx = idx_out ? idx_out : (int32_t*)scr;
  hipStream_t st = (hipStream_t)stream;
  if (debug_mode()) {
    s = debug_check_batch(b, std::min(ia->k_cache->num_pages, sa->kv_cache->num_pages), ia->k_cache->page_size,
                          nullptr, 0, st);
    if (s != DSA_OK) return s;
  }
  s = run_indexer_prefill(b, ia, idx, st);
  if (s != DSA_OK) return s;
  return run_sfa(b, sa, idx, ia->topk, out, lse, scr + rows, st);
}

}  // extern "C"
