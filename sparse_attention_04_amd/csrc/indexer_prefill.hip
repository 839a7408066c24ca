// Fused Lightning Indexer for causal (chunked) prefill: every new token t of a
// sequence keeps the top n = min(k, t + 1) positions s <= t by the
// head-weighted relevance score, without writing any score row to memory.
//
// Method: relevance scoring, head weighting and Top-K in one pass over the
// paged K cache ("Deep Fusion of LI and SFA", Day0 Inference Optimization on
// Ascend CANN, sec. 2), causal index computation whose cost grows with t, and
// the zigzag layout that pairs a short-history block with a long-history one
// (Adapting and Optimizing Inference for a New Model Architecture on Ascend,
// sec. 5.2; Inference Acceleration for Next-Gen Attention Architectures,
// sec. 5.2).  The pages pair segments across devices; here the unit is one
// workgroup: unit u of a sequence with NB query blocks of 64 tokens owns
// blocks u and NB-1-u, so every unit scores about the same number of (query,
// key) pairs, and results go straight to the rows of their own tokens (the
// "restore order" step is plain indexing).
//
// Inside a unit, queries are taken 4 at a time, one per wave.  64-key tiles of
// the K cache stream through a 2-deep LDS ring shared by the 4 waves; each
// wave scores its query against the tile with 32x32 MFMAs (bf16, or scaled
// e4m3 for the quantised caches, which the pages' fused indexer serves in
// prefill as in decode: Day0 Inference Optimization on Ascend CANN, sec. 2;
// Adapting and Optimizing Inference for a New Model Architecture on Ascend,
// sec. 2.2) and appends the
// keys above its current threshold to its own candidate buffer in LDS.  When a
// buffer fills, a wave-level radix select (four 8-bit digits) keeps exactly
// the k best, stably (so equal scores stay in position order and the smaller
// position wins), and raises the threshold to the k-th best score.  After the
// last tile the same select leaves the final n positions, in ascending order.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kPfThreads = 256;
constexpr int kPfWaves = 4;
constexpr int kQBlock = 64;         // query block of the zigzag schedule
constexpr int kKT = 64;             // keys per tile
constexpr int kCap = 3072;          // candidate buffer entries per query
constexpr int kMaxPages = 4096;                    // block-table entries staged in LDS
constexpr int kHistWords = 260;                    // per-wave select histogram (256 bins, a spare word, padding)

// LDS image of one 64-key tile of 128-dim keys.  bf16: rows of 256 bytes at a
// 272-byte pitch, 20 1-KiB loads (the last three only fill padding).  e4m3
// (FP8 and MXFP8): rows of 128 bytes at a 144-byte pitch (9 loads), then the
// 64 rows' 4-byte scale words (FP8: the float32 per-token scale; MXFP8: the
// four e8m0 bytes of the row's 32-element groups) at byte kScaleOff, loaded
// by a 4-byte-per-lane load in the place of load 9.  Both pitches keep the
// 16-byte operand reads of 16 consecutive rows on distinct banks.
template <int DT>
struct PfTile {
  static constexpr bool kQuant = (DT != kBF16);
  static constexpr int kRowBytes = kQuant ? 128 : 256;
  static constexpr int kPitch = kRowBytes + 16;
  static constexpr int kRowLoads = (64 * kPitch + 1023) / 1024;     // 1-KiB loads that fill the rows
  static constexpr int kScaleOff = 64 * kPitch;                    // bf16: unused
  static constexpr int kLoads = kQuant ? 12 : 20;                   // load slots, 4 waves x kLoads / 4
  static constexpr int kBytes = kQuant ? kScaleOff + 64 * 4 : 20 * 1024;   // ring stride
  static_assert(kQuant ? (kRowLoads == 9 && kRowLoads < kLoads) : kRowLoads <= kLoads, "tile loads");
  static_assert(kBytes % 16 == 0 && kLoads % 4 == 0, "tile layout");
};

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
#define DSA_PF_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ int lane_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Wave-level Top-`need` of a candidate list (keys[], pos[] of `count` > need
// entries, in position order).  The keys and positions are held in registers
// (lane l owns entries l, l + 64, ...).  Radix passes run over y = key -
// min(key), starting at the highest bit in which the entries differ, so the
// first 8-bit digit spreads the entries over the whole histogram rather than
// piling them onto the one or two bins of a shared exponent.  Each pass finds
// the bin that holds the need-th largest entry.
//
// EXACT: passes continue until exactly `need` entries remain; of entries equal
// to the need-th largest key the first ones in list order are kept.  Otherwise
// the select may stop as soon as the entries above and in the current bin are
// at most need + kSelSlack: they always include the need best.
// Compacts in place, stably, and returns the smallest kept key: a later
// candidate must exceed it to enter the top `need` (equal keys at later
// positions lose the tie).  hist: 260 words of this wave's LDS, 16-byte aligned.
constexpr int kSelSlack = 256;
template <bool EXACT>
__device__ uint32_t wave_select(uint32_t* keys, uint32_t* pos, int& count, int need, uint32_t* hist) {
  constexpr int R = kCap / 64;
  const int lane = threadIdx.x & 63;
  uint32_t kv[R], pv[R];
#pragma unroll
  for (int j = 0; j < R; j++) {   // entries at or past `count` are read but never used
    kv[j] = keys[64 * j + lane];
    pv[j] = pos[64 * j + lane];
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int j = 0; j < R; j++) {
    const bool in = 64 * j + lane < count;
    mn = min(mn, in ? kv[j] : 0xFFFFFFFFu);
    mx = max(mx, in ? kv[j] : 0u);
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
#pragma unroll
  for (int j = 0; j < R; j++) kv[j] -= mn;
  const uint32_t range = mx - mn;
  int hi = range ? 31 - __builtin_clz(range) : -1;    // highest bit in which entries differ
  // entries in the current region: (y & pmask) == prefix
  uint32_t prefix = 0u, pmask = (hi >= 0) ? ~((2u << hi) - 1u) : 0xFFFFFFFFu;
  int rem = need;            // entries still wanted from the region
  int bincnt = count;        // entries in the region
  bool whole = false, partial = false;
  while (hi >= 0) {
    const int lo = max(hi - 7, 0);
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
#pragma unroll
    for (int j = 0; j < R; j++) {
      const bool m = (64 * j + lane < count) && (kv[j] & pmask) == prefix;
      atomicAdd(&hist[m ? (kv[j] >> lo) & dmask : 256u], 1u);   // word 256 takes the rest
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    // lane l owns bins 4l .. 4l+3; suffix sums from the top bin down
    const uint4 hv = *(const uint4*)(hist + 4 * lane);
    const uint32_t h[4] = {hv.x, hv.y, hv.z, hv.w};
    const int c = (int)(h[0] + h[1] + h[2] + h[3]);
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_down(x, o);
      if (lane + o < 64) x += v;
    }
    const int above = x - c;   // entries in bins above this lane's four
    int bin = -1, binabove = 0, bc = 0;
    if (above < rem && rem <= above + c) {
      int run = above;
      for (int j = 3; j >= 0; j--) {
        if (run + (int)h[j] >= rem) {
          bin = 4 * lane + j;
          binabove = run;
          bc = (int)h[j];
          break;
        }
        run += (int)h[j];
      }
    }
    const uint64_t m = __ballot(bin >= 0);
    const int src = m ? (__ffsll((unsigned long long)m) - 1) : 0;
    bin = __shfl(bin, src);
    binabove = __shfl(binabove, src);
    bc = __shfl(bc, src);
    if (bin < 0) bin = 0;  // cannot happen for need < count
    rem -= binabove;
    bincnt = bc;
    prefix |= (uint32_t)bin << lo;
    pmask |= dmask << lo;
    hi = lo - 1;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // histogram read before the next clear
    if (bincnt == rem) { whole = true; break; }
    if (!EXACT && bincnt - rem <= kSelSlack) { partial = true; break; }
  }
  const bool keep_all = whole || partial;
  // stable in-place compaction (every read above precedes these writes)
  int out = 0, ties = 0;
  uint32_t kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < R; j++) {
    if (64 * j < count) {
      const bool in = 64 * j + lane < count;
      const uint32_t ym = kv[j] & pmask;
      const bool gt = in && ym > prefix;
      const bool eq = in && ym == prefix;
      const uint64_t me = __ballot(eq);
      const bool keep = gt || (eq && (keep_all || ties + lane_rank(me) < rem));
      const uint64_t mk = __ballot(keep);
      const int r = out + lane_rank(mk);
      if (keep) {
        keys[r] = kv[j] + mn;
        pos[r] = pv[j];
        kmin = min(kmin, kv[j]);
      }
      out += __popcll(mk);
      ties += __popcll(me);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  count = out;
  return wave_min_u32(kmin) + mn;
}

// Query operands of one wave in the 32x32 MFMA layout, and the tile product.
// bf16 (32x32x16): lane half h holds dims [64h, 64h + 64) of its head row and
// of its key row, which fixes one order of the contraction index for both.
// e4m3 (scaled 32x32x64): a lane's bytes 0..15 belong to the instruction's
// k-block 0 and bytes 16..31 to k-block 1, and the scale of block b of row m
// is taken from lane m + 32b; K-step kk covers the 32-element groups 2kk and
// 2kk + 1, so lane half h carries dims 64kk + 16h .. +15 and 64kk + 32 + 16h
// .. +15 and supplies the scale of group 2kk + h.  FP8 enters with unit
// block scales: its per-(token, head) query scale is folded into the head
// weight and the per-token key scale multiplies the head-weighted sum.
template <int DT, int H, int D>
struct PfQuery;

template <int H, int D>
struct PfQuery<kBF16, H, D> {
  static constexpr int MT = H / 32, KS = D / 16;
  bf16x8 a[MT][KS];
  float wr[MT][16];
  __device__ void load(const IndexerPrefillParams& p, size_t tok) {
    const int lane = threadIdx.x & 63;
    const uint16_t* qp = (const uint16_t*)p.q + tok * H * D;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const bf16x8* src = (const bf16x8*)(qp + (size_t)(32 * mt + (lane & 31)) * D + (lane >> 5) * (D / 2));
#pragma unroll
      for (int kk = 0; kk < KS; kk++) a[mt][kk] = src[kk];
#pragma unroll
      for (int i = 0; i < 16; i++)
        wr[mt][i] = p.w[tok * H + 32 * mt + 8 * (i / 4) + 4 * (lane >> 5) + (i & 3)];
    }
  }
  // both 32-key N-tiles at once: four independent accumulator chains
  __device__ void mma(const unsigned char* cur, f32x16 (&acc)[2][MT]) const {
    constexpr int PITCH = PfTile<kBF16>::kPitch;
    const int lane = threadIdx.x & 63;
    const unsigned char* kp = cur + (lane & 31) * PITCH + (lane >> 5) * D;
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      const bf16x8 kb0 = *(const bf16x8*)(kp + 16 * kk);
      const bf16x8 kb1 = *(const bf16x8*)(kp + 32 * PITCH + 16 * kk);
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        acc[0][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][kk], kb0, acc[0][mt], 0, 0, 0);
        acc[1][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][kk], kb1, acc[1][mt], 0, 0, 0);
      }
    }
  }
  __device__ float key_scale(const unsigned char*) const { return 1.f; }
};

template <int DT, int H, int D>
struct PfQueryF8 {
  static constexpr int MT = H / 32, KS = D / 64;
  i32x8 a[MT][KS];
  int32_t sa[MT][KS];     // MXFP8: e8m0 byte of group 2kk + h of this lane's head row
  float wr[MT][16];       // FP8: w * q_scale
  __device__ static i32x8 step(const unsigned char* rowp, int kk, int h) {
    const u32x4* v = (const u32x4*)rowp;
    const u32x4 lo = v[4 * kk + h], hi = v[4 * kk + 2 + h];
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  __device__ void load(const IndexerPrefillParams& p, size_t tok) {
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const unsigned char* qp = (const unsigned char*)p.q + tok * H * D;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const int hrow = 32 * mt + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < KS; kk++) {
        a[mt][kk] = step(qp + (size_t)hrow * D, kk, h);
        if constexpr (DT == kMX)
          sa[mt][kk] = ((const uint8_t*)p.q_scale)[(tok * H + hrow) * (D / 32) + 2 * kk + h];
        else
          sa[mt][kk] = 127;   // 2^0
      }
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int hh = 32 * mt + 8 * (i / 4) + 4 * h + (i & 3);
        float wv = p.w[tok * H + hh];
        if constexpr (DT == kFP8) wv *= ((const float*)p.q_scale)[tok * H + hh];
        wr[mt][i] = wv;
      }
    }
  }
  __device__ void mma(const unsigned char* cur, f32x16 (&acc)[2][MT]) const {
    constexpr int PITCH = PfTile<DT>::kPitch;
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const unsigned char* kp = cur + (lane & 31) * PITCH;
    uint32_t sw[2] = {127u, 127u};
    if constexpr (DT == kMX) {
      const uint32_t* st = (const uint32_t*)(cur + PfTile<DT>::kScaleOff);
      sw[0] = st[lane & 31];
      sw[1] = st[32 + (lane & 31)];
    }
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      const i32x8 kb0 = step(kp, kk, h);
      const i32x8 kb1 = step(kp + 32 * PITCH, kk, h);
      const int sb0 = (DT == kMX) ? (int)((sw[0] >> (8 * (2 * kk + h))) & 0xFFu) : 127;
      const int sb1 = (DT == kMX) ? (int)((sw[1] >> (8 * (2 * kk + h))) & 0xFFu) : 127;
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        acc[0][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mt][kk], kb0, acc[0][mt], 0, 0, 0, sa[mt][kk], 0, sb0);
        acc[1][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mt][kk], kb1, acc[1][mt], 0, 0, 0, sa[mt][kk], 0, sb1);
      }
    }
  }
  // FP8: the per-token scale of key `lane` of the tile
  __device__ float key_scale(const unsigned char* cur) const {
    if constexpr (DT == kFP8) return ((const float*)(cur + PfTile<DT>::kScaleOff))[threadIdx.x & 63];
    return 1.f;
  }
};
template <int H, int D>
struct PfQuery<kFP8, H, D> : PfQueryF8<kFP8, H, D> {};
template <int H, int D>
struct PfQuery<kMX, H, D> : PfQueryF8<kMX, H, D> {};

template <int DT, int H, int D, bool BIG_PAGE>
__global__ __launch_bounds__(kPfThreads, 1) void indexer_prefill_kernel(IndexerPrefillParams p) {
  static_assert(H == 64 && D == 128, "prefill indexer is compiled for 64 heads x 128");
  using TL = PfTile<DT>;
  using Q = PfQuery<DT, H, D>;
  constexpr int MT = H / 32;        // M-tiles over heads
  constexpr int LPW = TL::kLoads / kPfWaves;          // load slots per wave per tile (5 bf16, 3 e4m3)
  extern __shared__ __attribute__((aligned(16))) unsigned char pf_smem[];
  unsigned char* ring = pf_smem;                                              // 2 tiles
  uint32_t* cand = (uint32_t*)(pf_smem + 2 * TL::kBytes);                     // [4][2][kCap]
  uint32_t* hist = cand + kPfWaves * 2 * kCap;                                // [4][kHistWords]
  int32_t* s_bt = (int32_t*)(hist + kPfWaves * kHistWords);                   // [kMaxPages]
  __shared__ int s_unit[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  const int K = p.topk;
  // ---- unit -> (sequence, first block): sequence b has NB_b = ceil(T_b/64)
  // blocks and ceil(NB_b/2) units; unit u owns blocks u and NB_b-1-u.
  if (wave == 0) {
    int acc = 0, found = 0;
    for (int b0 = 0; b0 < bv.batch && !found; b0 += 64) {
      const int b = b0 + lane;
      int nu = 0;
      if (b < bv.batch) {
        const int T = bv.cu_q[b + 1] - bv.cu_q[b];
        const int nb = (T + kQBlock - 1) / kQBlock;
        nu = (nb + 1) / 2;
      }
      int inc = nu;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      const int start = acc + inc - nu;
      const bool mine = b < bv.batch && (int)blockIdx.x >= start && (int)blockIdx.x < start + nu;
      const uint64_t m = __ballot(mine);
      if (m) {
        if (lane == __ffsll((unsigned long long)m) - 1) {
          s_unit[0] = b;
          s_unit[1] = (int)blockIdx.x - start;
        }
        found = 1;
      }
      acc += __shfl(inc, 63);
    }
    if (lane == 0 && !found) s_unit[0] = -1;
  }
  __syncthreads();
  const int b = s_unit[0];
  if (b < 0) return;
  const int u = s_unit[1];
  const int L = bv.seq_lens[b];
  const int tok0 = bv.cu_q[b];
  const int T = bv.cu_q[b + 1] - tok0;
  const int NB = (T + kQBlock - 1) / kQBlock;
  // the sequence's block-table row, staged once (page lookups stay on chip)
  {
    const int* btg = bv.block_table + (size_t)b * bv.max_pages;
    const int npg = min((L + P - 1) >> bv.page_shift, kMaxPages);
    for (int i = tid; i < npg; i += kPfThreads) s_bt[i] = btg[i];
  }
  __syncthreads();
  const int* bt = s_bt;
  const int blocks[2] = {u, NB - 1 - u};
  const int nblk = (blocks[1] != blocks[0]) ? 2 : 1;

  // per-lane source of each of this wave's LPW tile loads: load slot c = wave
  // + 4k fills LDS bytes 1024c + 16 * lane, row off / pitch, 16-byte column
  // (off % pitch) / 16; padding bytes load row 0, column 0.  e4m3: slot 9
  // loads the 64 rows' scale words (lane = row), slots 10 and 11 are unused.
  int lrow[LPW], lcol[LPW];
#pragma unroll
  for (int k = 0; k < LPW; k++) {
    const int off = (wave + kPfWaves * k) * 1024 + lane * 16;
    const int r = off / TL::kPitch, c = (off % TL::kPitch) / 16;
    const bool real = r < kKT && c < TL::kRowBytes / 16;
    lrow[k] = real ? r : 0;
    lcol[k] = real ? c * 16 : 0;
  }
  const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(ring));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t* ckey = cand + (size_t)wave * 2 * kCap;
  uint32_t* cpos = ckey + kCap;
  uint32_t* whist = hist + wave * kHistWords;

  for (int bi = 0; bi < nblk; bi++) {
    const int q0 = blocks[bi] * kQBlock;
    const int q1 = min(T, q0 + kQBlock);
    for (int qg = q0; qg < q1; qg += kPfWaves) {
      const int q = qg + wave;                  // this wave's query (may be >= q1)
      const bool have_q = q < q1;
      const int t = L - T + (have_q ? q : q1 - 1);
      const int tmax = L - T + min(q1, qg + kPfWaves) - 1;   // last position any wave needs
      int32_t* row = p.idx_out + (size_t)(tok0 + (have_q ? q : 0)) * K;
      // queries that keep every visible position need no scores
      const bool all_keep = have_q && (t + 1 <= K);
      if (all_keep) {
        for (int s = lane; s < K; s += 64) row[s] = (s <= t) ? s : -1;
      }
      const bool groups_all_keep = (tmax + 1 <= K);  // uniform: every wave's t <= tmax
      if (groups_all_keep) continue;

      Q qo;
      qo.load(p, (size_t)(tok0 + (have_q ? q : q1 - 1)));
      __builtin_amdgcn_s_waitcnt(0);
      int count = 0;
      uint32_t thr = 0u;    // keys must exceed this to become candidates
      const int nt = (tmax + 1 + kKT - 1) / kKT;
      // tile `tile`'s keys tile*64 .. tile*64+63 (rows past tmax repeat row
      // tmax) go to ring buffer tile & 1
      auto issue = [&](int tile) {
        const int s0 = tile * kKT;
        const int lim = tmax - s0;     // rows above lim repeat row lim
        const uint32_t m0 = ring_lds + (uint32_t)(tile & 1) * TL::kBytes + (uint32_t)wave_u * 1024u;
        const unsigned char* src[LPW];
        if constexpr (BIG_PAGE) {
          // the whole tile lies in one page
          const int64_t prow0 = ((int64_t)bt[s0 >> bv.page_shift] << bv.page_shift) + (s0 & (P - 1));
#pragma unroll
          for (int k = 0; k < LPW; k++) {
            const int c = wave_u + kPfWaves * k;
            src[k] = (TL::kQuant && c == TL::kRowLoads)
                         ? (const unsigned char*)p.k_scale + (prow0 + min(lane, lim)) * 4
                         : (const unsigned char*)p.k_data + (prow0 + min(lrow[k], lim)) * TL::kRowBytes + lcol[k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < LPW; k++) {
            const int c = wave_u + kPfWaves * k;
            const bool sl = TL::kQuant && c == TL::kRowLoads;
            const int srow = s0 + min(sl ? lane : lrow[k], lim);
            const int64_t prow = ((int64_t)bt[srow >> bv.page_shift] << bv.page_shift) + (srow & (P - 1));
            src[k] = sl ? (const unsigned char*)p.k_scale + prow * 4
                        : (const unsigned char*)p.k_data + prow * TL::kRowBytes + lcol[k];
          }
        }
#pragma unroll
        for (int k = 0; k < LPW; k++) {
          const int c = wave_u + kPfWaves * k;   // uniform over the wave
          if (!TL::kQuant || c < TL::kRowLoads) dma16(src[k], m0 + k * kPfWaves * 1024u);
          else if (c == TL::kRowLoads) dma4(src[k], ring_lds + (uint32_t)(tile & 1) * TL::kBytes + TL::kScaleOff);
        }
      };
      // 2-buffer ring: tile t + 1 is loaded while t is scored.  The barrier at
      // the top of iteration t also tells that every wave is done with the
      // buffer of tile t - 1, which tile t + 1 then overwrites.
      issue(0);
      for (int tile = 0; tile < nt; tile++) {
        DSA_PF_WAIT_VMCNT(0);
        lds_barrier();
        if (tile + 1 < nt) issue(tile + 1);
        const unsigned char* cur = ring + (tile & 1) * TL::kBytes;
        // ---- scores of the 64 keys of this tile for this wave's query
        float sc[2];
        {
          f32x16 acc[2][MT];
#pragma unroll
          for (int n = 0; n < 2; n++)
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
              for (int e = 0; e < 16; e++) acc[n][mt][e] = 0.f;
          qo.mma(cur, acc);
#pragma unroll
          for (int n = 0; n < 2; n++) {
            // four partial sums (entries i mod 4 of each M-tile), added
            // pairwise: shorter dependency chains than one running sum
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
              for (int i = 0; i < 16; i++) s4[i & 3] = fmaf(qo.wr[mt][i], acc[n][mt][i], s4[i & 3]);
            const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
            sc[n] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);   // lanes l and l ^ 32 summed
          }
        }
        // lane l takes key tile*64 + l: N-tile l/32, column l%32
        const int spos = tile * kKT + lane;
        const float v = ((lane < 32) ? sc[0] : sc[1]) * qo.key_scale(cur);
        const uint32_t x = (have_q && spos <= t) ? float_key(v) : 0u;
        bool cnd = x > thr;
        uint64_t m = __ballot(cnd);
        if (count + __popcll(m) > kCap) {
          thr = wave_select<false>(ckey, cpos, count, K, whist);
          cnd = x > thr;
          m = __ballot(cnd);
        }
        // count + 64 <= kCap always holds here (see indexer_prefill_max_topk);
        // the bound below only keeps a broken invariant inside the buffer
        if (cnd) {
          const int r = count + lane_rank(m);
          if (r < kCap) {
            ckey[r] = x;
            cpos[r] = (uint32_t)spos;
          }
        }
        count = min(count + __popcll(m), kCap);
      }
      if (have_q && !all_keep) {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        if (count > K) wave_select<true>(ckey, cpos, count, K, whist);
        // count == K here (t + 1 > K keys were visible); positions ascend
        for (int i = lane; i < K; i += 64) row[i] = (i < count) ? (int32_t)cpos[i] : -1;
      }
      __syncthreads();
    }
  }
}

}  // namespace

size_t indexer_prefill_lds_bytes(int dtype) {
  const size_t tile = (dtype == kBF16) ? PfTile<kBF16>::kBytes : PfTile<kFP8>::kBytes;
  return 2 * tile + (size_t)kPfWaves * 2 * kCap * 4 + kPfWaves * kHistWords * 4 + kMaxPages * 4;
}

int indexer_prefill_max_pages() { return kMaxPages; }
// A mid-query select may keep up to k + kSelSlack candidates, and the next
// tile appends at most kKT more before the buffer is checked again, so the
// buffer holds k + kSelSlack + kKT entries at most: k <= kCap - kSelSlack - kKT.
constexpr int kMaxTopk = kCap - kSelSlack - kKT;
static_assert(kMaxTopk == 2752, "prefill Top-K bound");
int indexer_prefill_max_topk() { return kMaxTopk; }

int indexer_prefill_grid(int total_q, int batch) {
  const int blocks = (total_q + kQBlock - 1) / kQBlock + batch;   // >= sum of ceil(T_b/64)
  return (blocks + batch + 1) / 2;                                // >= sum of ceil(NB_b/2)
}

hipError_t launch_indexer_prefill(int dtype, int H, int D, const IndexerPrefillParams& p, hipStream_t st) {
  if ((dtype != kBF16 && dtype != kFP8 && dtype != kMX) || H != 64 || D != 128) return hipErrorInvalidValue;
  if (p.grid <= 0) return hipSuccess;
  // pages of 64 tokens or more hold each 64-key tile whole
  const bool big = p.bv.page_size >= kKT;
  void (*kern)(IndexerPrefillParams) = nullptr;
  switch (dtype) {
    case kBF16: kern = big ? indexer_prefill_kernel<kBF16, 64, 128, true> : indexer_prefill_kernel<kBF16, 64, 128, false>; break;
    case kFP8: kern = big ? indexer_prefill_kernel<kFP8, 64, 128, true> : indexer_prefill_kernel<kFP8, 64, 128, false>; break;
    default: kern = big ? indexer_prefill_kernel<kMX, 64, 128, true> : indexer_prefill_kernel<kMX, 64, 128, false>; break;
  }
  const size_t lds = indexer_prefill_lds_bytes(dtype);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kPfThreads), lds, st, p);
  return hipGetLastError();
}

}  // namespace dsa
