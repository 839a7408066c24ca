// Device side of the decode indexer: the scorers and the work of one
// workgroup as a function, shared by the indexer kernel and the fused decode
// kernel.  The method, the workspace protocol and the launch rules are
// described in indexer_decode.hip.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dsa {

// One workgroup of 8 waves per CU: the CU's waves share one key range (two
// co-resident workgroups of 4 waves each finished up to 1.6x apart, the
// younger one getting the smaller share of the CU), and half as many
// workgroups take part in each sequence's radix barriers.
constexpr int kIdxThreads = 512;
constexpr int kIdxWaves = kIdxThreads / kWave;
constexpr int kBinsPerThread = kRadixBins / kIdxThreads;
static_assert(kMaxDecodeQ <= 4 && kIdxWaves % 4 == 0, "wave groups per decode query");
static_assert(kRadixBins % kIdxThreads == 0, "histogram bins split evenly over the threads");
// bf16 keys with three or four query tokens: 64-key steps whose quarter tiles
// a wave holds in registers (one being staged, kXchgRing - 1 in flight), and
// the two 16-KiB LDS slots they are shared through
constexpr int kXchgRing = 4;
constexpr int kXchgSlotWords = 64 * 128 * 2 / 4;

__host__ __device__ constexpr size_t xchg_offset_words(int maxq, int chunk_cap, int stage_pages) {
  return ((size_t)maxq * chunk_cap + (size_t)maxq * kRadixBins + stage_pages + 3) / 4 * 4;
}

// Workspace layout (uint32 words).  The whole region is zero when a call
// starts and the call leaves it zero: the last workgroup of each sequence to
// finish clears what the sequence's workgroups used (see the end of the
// kernel), so no fill is needed between calls, whatever the batch shape.
//   [0, 64)                        header: error bits (sticky), profiling stamps
//   [64, 64 + 32*B)                per sequence, one 128-B line: barrier counter,
//                                  exit counter, failure flag, and for the fused
//                                  decode kernel the ready word (the call's epoch
//                                  once every index row of the sequence is
//                                  written) and the attention's exit counter
//   then per query {hist0[2048], outcnt, candcnt (+30 pad)}
//   then per query {hist1[2048], hist2[2048], tie[grid_pad]}, which a query
//                                  whose boundary bin is handed to the last
//                                  workgroup (section 3c) uses instead as its
//                                  list of (key, position) candidate pairs
struct WsLayout {
  uint32_t* base;
  int32_t nseq, nq, grid_pad;
  __host__ __device__ uint32_t* err() const { return base; }
  __host__ __device__ uint32_t* call_epoch() const { return base + kWsEpochWord; }
  __host__ __device__ uint32_t* seq_ctr(int b) const { return base + 64 + 32 * b; }
  __host__ __device__ uint32_t* seq_exit(int b) const { return seq_ctr(b) + 1; }
  __host__ __device__ uint32_t* seq_failed(int b) const { return seq_ctr(b) + 2; }
  __host__ __device__ uint32_t* seq_ready(int b) const { return seq_ctr(b) + 3; }
  __host__ __device__ uint32_t* seq_attn_exit(int b) const { return seq_ctr(b) + 4; }
  __host__ __device__ uint32_t* qa(int g) const { return base + 64 + 32 * nseq + (size_t)g * 2080; }
  __host__ __device__ uint32_t* hist(int g, int pass) const {
    if (pass == 0) return qa(g);
    return base + 64 + 32 * nseq + (size_t)nq * 2080 + (size_t)g * (4096 + grid_pad) + (pass - 1) * 2048;
  }
  __host__ __device__ uint32_t* outcnt(int g) const { return qa(g) + 2048; }
  __host__ __device__ uint32_t* candcnt(int g) const { return qa(g) + 2049; }
  __host__ __device__ uint64_t* cand(int g) const { return (uint64_t*)hist(g, 1); }
  __host__ __device__ int cand_pairs() const { return (4096 + grid_pad) / 2; }
  __host__ __device__ uint32_t* tie(int g) const {
    return base + 64 + 32 * nseq + (size_t)nq * 2080 + (size_t)g * (4096 + grid_pad) + 4096;
  }
  __host__ __device__ size_t total_words() const {
    return 64 + 32 * (size_t)nseq + (size_t)nq * 2080 + (size_t)nq * (4096 + grid_pad);
  }
};


// ----------------------------------------------------------------- scoring ---

// Score one 32-key tile per wave with 32x32 MFMAs.  Lane l owns key column
// l%32; lane half h = l/32 holds the contiguous half [h*D/2, (h+1)*D/2) of the
// key (and of every query row), which fixes the order of the contraction index
// for both operands alike.  Returns the head-weighted score of key l%32 in
// every lane (both halves).
template <int DT, int H, int D>
struct MfmaScorer;

template <int H, int D>
struct MfmaScorer<kBF16, H, D> {
  static constexpr int MT = H / 32;       // M-tiles over heads
  static constexpr int KS = D / 16;       // K-steps of 16 (8 per lane half)
  bf16x8 a[MT][KS];
  float wr[MT][16];
  __device__ void load_query(const IndexerDecodeParams& p, int tok) {
    const int lane = threadIdx.x & 63;
    const uint16_t* q = (const uint16_t*)p.q + (size_t)tok * H * D;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const bf16x8* src = (const bf16x8*)(q + (size_t)(32 * mt + (lane & 31)) * D + (lane >> 5) * (D / 2));
#pragma unroll
      for (int kk = 0; kk < KS; kk++) a[mt][kk] = src[kk];
#pragma unroll
      for (int i = 0; i < 16; i++)
        wr[mt][i] = p.w[(size_t)tok * H + 32 * mt + 8 * (i / 4) + 4 * (lane >> 5) + (i & 3)];
    }
  }
  struct Tile { u32x4 v[KS]; };
  __device__ void load_tile(const IndexerDecodeParams& p, int64_t row, Tile& t) const {
    const int lane = threadIdx.x & 63;
    const u32x4* src = (const u32x4*)((const uint16_t*)p.k_data + row * D + (lane >> 5) * (D / 2));
#pragma unroll
    for (int kk = 0; kk < KS; kk++) t.v[kk] = src[kk];
  }

  // per-head products of the tile's 32 keys: acc[mt] = heads 32 mt .. +31
  __device__ void mma(const Tile& t, f32x16 (&acc)[MT]) const {
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[mt][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      bf16x8 b = __builtin_bit_cast(bf16x8, t.v[kk]);
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt][kk], b, acc[mt], 0, 0, 0);
    }
  }
  // head-weighted sum: lane n and lane n + 32 both return key n's score.
  // One running sum: here the sum overlaps the other wave's MFMAs, and four
  // partial sums (the prefill indexer's order) measured slightly slower.
  __device__ float head_sum(const f32x16 (&acc)[MT]) const {
    float s = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) s = fmaf(wr[mt][i], acc[mt][i], s);
    return s + __shfl_xor(s, 32);
  }
  __device__ float score(const IndexerDecodeParams& p, int64_t row, const Tile& t) const {
    f32x16 acc[MT];
    mma(t, acc);
    return head_sum(acc);
  }
};

// FP8 (per-token K scale, per-token-head Q scale) and MXFP8 (e8m0 per 32
// elements): 32x32x64 scaled MFMAs on e4m3 bytes.  In this instruction a
// lane's bytes 0..15 belong to k-block 0 and bytes 16..31 to k-block 1, and the
// scale of block b of row m is taken from lane m + 32*b.  K-step kk covers the
// two 32-element groups 2kk and 2kk+1 of the row, so lane half h carries the
// h-th 16-byte half of each: bytes 0..15 <- dims 64kk + 16h .. +15 (group 2kk),
// bytes 16..31 <- dims 64kk + 32 + 16h .. +15 (group 2kk+1), and supplies the
// scale of group 2kk + h.
template <int DT, int H, int D>
struct MfmaScorerF8 {
  static constexpr int MT = H / 32;
  static constexpr int KS = D / 64;       // K-steps of 64
  i32x8 a[MT][KS];
  int32_t sa[MT][KS];                     // MX: e8m0 byte of group 2kk + h of this lane's row
  float wr[MT][16];                       // FP8: w * q_scale
  __device__ static i32x8 load_step(const uint8_t* rowp, int kk, int h) {
    const u32x4* v = (const u32x4*)rowp;
    const u32x4 lo = v[4 * kk + h], hi = v[4 * kk + 2 + h];
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  __device__ void load_query(const IndexerDecodeParams& p, int tok) {
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const uint8_t* q = (const uint8_t*)p.q + (size_t)tok * H * D;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const int hrow = 32 * mt + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < KS; kk++) {
        a[mt][kk] = load_step(q + (size_t)hrow * D, kk, h);
        if constexpr (DT == kMX)
          sa[mt][kk] = ((const uint8_t*)p.q_scale)[((size_t)tok * H + hrow) * (D / 32) + 2 * kk + h];
        else
          sa[mt][kk] = 127;
      }
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int hh = 32 * mt + 8 * (i / 4) + 4 * h + (i & 3);
        float wv = p.w[(size_t)tok * H + hh];
        if constexpr (DT == kFP8) wv *= ((const float*)p.q_scale)[(size_t)tok * H + hh];
        wr[mt][i] = wv;
      }
    }
  }
  struct Tile { i32x8 v[KS]; uint32_t sc; };

  __device__ void load_tile(const IndexerDecodeParams& p, int64_t row, Tile& t) const {
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const uint8_t* kr = (const uint8_t*)p.k_data + row * D;
#pragma unroll
    for (int kk = 0; kk < KS; kk++) t.v[kk] = load_step(kr, kk, h);
    if constexpr (DT == kFP8) {
      t.sc = __float_as_uint(((const float*)p.k_scale)[row]);
    } else {
      const uint8_t* s8 = (const uint8_t*)p.k_scale + row * (D / 32);
      uint32_t v = 0;
#pragma unroll
      for (int kk = 0; kk < KS; kk++) v |= (uint32_t)s8[2 * kk + h] << (8 * kk);
      t.sc = v;
    }
  }
  __device__ float score(const IndexerDecodeParams& p, int64_t row, const Tile& t) const {
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) acc[mt][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; kk++) {
      const int sb = (DT == kMX) ? (int)((t.sc >> (8 * kk)) & 0xFFu) : 127;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
        acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[mt][kk], t.v[kk], acc[mt], 0, 0,
                                                                  0, sa[mt][kk], 0, sb);
    }
    // four partial sums added pairwise (as in the prefill indexer)
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 16; i++) s4[i & 3] = fmaf(wr[mt][i], acc[mt][i], s4[i & 3]);
    float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    s += __shfl_xor(s, 32);
    if constexpr (DT == kFP8) {
      // the key's per-token scale (lane l%32 loaded it for its own key)
      s *= __uint_as_float(t.sc);
    }
    return s;
  }
};

template <int H, int D>
struct MfmaScorer<kFP8, H, D> : MfmaScorerF8<kFP8, H, D> {};
template <int H, int D>
struct MfmaScorer<kMX, H, D> : MfmaScorerF8<kMX, H, D> {};

// ---------------------------------------------------------- block helpers ---

// Exclusive rank of `pred` among the block's threads in thread order, and the
// block total.  `scratch` holds kIdxWaves+1 ints of LDS.
__device__ __forceinline__ int block_rank(bool pred, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(pred);
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  if (lane == 0) scratch[wave] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kIdxWaves; w++) {
    const int c = scratch[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + in_wave;
}

// ------------------------------------------------------------------ kernel ---

enum : int { kActive = 0, kTakeBin = 1, kTiePass = 2, kAll = 3, kHandoff = 4 };

// Exact choice, inside the sequence's last workgroup, of the s_need[q] best
// of the s_nc[q] candidate pairs (key in the low word, position in the high
// word) of every handed-off query q; all of a query's candidates share their
// leading 11 key bits.  Order: larger key first, and among equal keys the
// smaller position.  Each pair becomes a 52-bit composite, key bits 20..0
// above (2^31 - 1 - position), so the candidates are distinct and ordered as
// the selection orders them.  A radix select over the composites takes
// digits from the top (11, 11, 11, 11, 8 bits) and stops, query by query, once
// the boundary digit's candidates are all needed.  The composites stay in
// registers (thread t holds candidates t + 512 r); each query has two LDS
// histograms used in turn, so a pass costs two barriers, and the first pass's
// counts are taken as the candidates arrive.  The chosen positions go to the
// query's row from slot K - s_need[q] on, in no particular order.  One call
// serves queries q0 .. q0 + MAXQ - 1; the kernels call it one query at a time,
// since the four-query kernels have no registers to spare for more (they
// already keep part of their scalars in vector-register lanes).
// LDS: 2 * MAXQ * 2048 words from `lds`.
constexpr int kHandRegs = (kHandoffCap + kIdxThreads - 1) / kIdxThreads;

template <int MAXQ, typename Put>
__device__ void handoff_select(const WsLayout& W, int tok0, int T, const int* s_hand, const int* s_nc,
                               const int* s_need, int32_t* idx_out, int K, uint32_t* lds, Put put_row) {
  static_assert(kBinsPerThread == 4 && kRadixBins == 4 * kIdxThreads, "four bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();   // the previous call's LDS reads are done
  __shared__ int s_wsum[MAXQ][kIdxWaves], s_hb[MAXQ][3], s_slot[MAXQ];
  uint32_t* hist = lds;   // [2][MAXQ][2048]
  for (int i = tid; i < 2 * MAXQ * kRadixBins / 4; i += kIdxThreads) ((u32x4*)hist)[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid < MAXQ) s_slot[tid] = 0;
  bool act[MAXQ];
  int n[MAXQ], need[MAXQ];
  uint64_t pre[MAXQ], pm[MAXQ];
  uint64_t c[MAXQ][kHandRegs];
#pragma unroll
  for (int q = 0; q < MAXQ; q++) {
    act[q] = q < T && s_hand[q];
    n[q] = act[q] ? s_nc[q] : 0;
    need[q] = act[q] ? s_need[q] : 0;
    pre[q] = 0;
    pm[q] = 0;
    const uint64_t* cl = W.cand(tok0 + q);
#pragma unroll
    for (int r = 0; r < kHandRegs; r++) {
      const int i = tid + kIdxThreads * r;
      c[q][r] = (i < n[q]) ? __hip_atomic_load(const_cast<uint64_t*>(cl) + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0ull;
    }
  }
  __syncthreads();   // histograms clear
#pragma unroll
  for (int q = 0; q < MAXQ; q++) {
#pragma unroll
    for (int r = 0; r < kHandRegs; r++) {
      const int i = tid + kIdxThreads * r;
      const uint32_t key = (uint32_t)c[q][r], pos = (uint32_t)(c[q][r] >> 32);
      c[q][r] = ((uint64_t)(key & 0x1FFFFFu) << 31) | (uint64_t)(0x7FFFFFFFu - pos);
      if (i < n[q]) atomicAdd(&hist[q * kRadixBins + (uint32_t)(c[q][r] >> 41)], 1u);
    }
  }
  for (int ps = 0; ps < 5; ps++) {
    bool any = false;
#pragma unroll
    for (int q = 0; q < MAXQ; q++) any |= act[q];
    if (!any) break;   // uniform: every thread holds the same act[]
    const int shift = (ps < 4) ? 41 - 11 * ps : 0;
    const uint32_t dmask = (ps < 4) ? 0x7FFu : 0xFFu;
    uint32_t* H = hist + (ps & 1) * MAXQ * kRadixBins;
    uint32_t* Hn = hist + ((ps + 1) & 1) * MAXQ * kRadixBins;
    if (ps > 0) {
#pragma unroll
      for (int q = 0; q < MAXQ; q++) {
        if (!act[q]) continue;
#pragma unroll
        for (int r = 0; r < kHandRegs; r++) {
          const int i = tid + kIdxThreads * r;
          if (i < n[q] && (c[q][r] & pm[q]) == pre[q])
            atomicAdd(&H[q * kRadixBins + ((uint32_t)(c[q][r] >> shift) & dmask)], 1u);
        }
      }
    }
    // the other set, read by the previous pass's scan (finished before the
    // barrier that ended it), is cleared for the next pass
#pragma unroll
    for (int q = 0; q < MAXQ; q++)
      if (act[q]) ((u32x4*)(Hn + q * kRadixBins))[tid] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // boundary bin of every active query: suffix sums over 4 bins per thread
    u32x4 v[MAXQ];
    int cs[MAXQ], x[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      if (!act[q]) continue;
      v[q] = ((const u32x4*)(H + q * kRadixBins))[tid];
      cs[q] = (int)(v[q][0] + v[q][1] + v[q][2] + v[q][3]);
      x[q] = cs[q];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_down(x[q], o);
        if (lane + o < 64) x[q] += t;
      }
      if (lane == 0) s_wsum[q][wave] = x[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      if (!act[q]) continue;
      int later = 0;
#pragma unroll
      for (int w = 0; w < kIdxWaves; w++) later += (w > wave) ? s_wsum[q][w] : 0;
      const int incl = x[q] + later, above = incl - cs[q];
      if (above < need[q] && need[q] <= incl) {
        int run = above;
#pragma unroll
        for (int e = 3; e >= 0; e--) {
          if (run + (int)v[q][e] >= need[q]) {
            s_hb[q][0] = 4 * tid + e;
            s_hb[q][1] = run;
            s_hb[q][2] = (int)v[q][e];
            break;
          }
          run += (int)v[q][e];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      if (!act[q]) continue;
      need[q] -= s_hb[q][1];
      pre[q] |= (uint64_t)s_hb[q][0] << shift;
      pm[q] |= (uint64_t)dmask << shift;
      if (s_hb[q][2] == need[q]) act[q] = false;   // the boundary digit is taken whole
    }
  }
  // every composite at or above the final prefix is chosen
#pragma unroll
  for (int q = 0; q < MAXQ; q++) {
    if (!(q < T && s_hand[q])) continue;
    int32_t* row = idx_out + (size_t)(tok0 + q) * K;
    const int m = s_need[q];
#pragma unroll
    for (int r = 0; r < kHandRegs; r++) {
      const int i = tid + kIdxThreads * r;
      if (i < n[q] && (c[q][r] & pm[q]) >= pre[q]) {
        const int k = atomicAdd(&s_slot[q], 1);
        if (k < m) put_row(row, K - m + k, (int)(0x7FFFFFFFu - (uint32_t)(c[q][r] & 0x7FFFFFFFu)));
      }
    }
  }
}

// Phase timestamps of workgroup 0 (100 MHz real-time counter) in header words
// 16.. of the workspace, for profiling the phases of one launch; compiled in
// only with DSA_INDEXER_STAMPS (each costs workgroup 0 a scalar-memory wait).
#ifdef DSA_INDEXER_STAMPS
#define DSA_STAMP(i)                                                                          \
  do {                                                                                        \
    if (blockIdx.x == 0 && threadIdx.x == 0 && (i) < 24)                                      \
      ((unsigned long long*)(W.base + 16))[(i)] = __builtin_amdgcn_s_memrealtime();            \
  } while (0)
#else
#define DSA_STAMP(i) \
  do {               \
  } while (0)
#endif

// ------------------------------------------------------- f32 (small shapes) ---
// VALU scorer: one key per thread, q and w staged in LDS.  Same selection code
// path is shared by instantiating the kernel above with a VALU scorer.
template <int H, int D>
struct MfmaScorer<kF32, H, D> {
  // Tile = one key per lane (64 keys per wave-tile would break the 32-key tile
  // contract, so only lanes 0..31 score; lanes 32..63 duplicate the work).
  float qv[H][D];
  float wv[H];
  __device__ void load_query(const IndexerDecodeParams& p, int tok) {
    const float* q = (const float*)p.q + (size_t)tok * H * D;
    for (int h = 0; h < H; h++) {
      wv[h] = p.w[(size_t)tok * H + h];
      for (int d = 0; d < D; d++) qv[h][d] = q[h * D + d];
    }
  }
  struct Tile { float k[D]; };

  __device__ void load_tile(const IndexerDecodeParams& p, int64_t row, Tile& t) const {
    const float* src = (const float*)p.k_data + row * D;
#pragma unroll
    for (int d = 0; d < D; d++) t.k[d] = src[d];
  }
  __device__ float score(const IndexerDecodeParams& p, int64_t row, const Tile& t) const {
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < H; h++) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; d++) dot = fmaf(qv[h][d], t.k[d], dot);
      s = fmaf(wv[h], dot, s);
    }
    return s;
  }
};

// The work of workgroup `wg` of a launch: its page range of one sequence, the
// sequence's radix select and its selected positions.  FUSED (the fused
// decode kernel): the index rows are written with agent-scope stores, and the
// sequence's last workgroup to finish writes `epoch` into the sequence's ready
// word once every row of the sequence is complete, for the attention that
// follows in the same launch.
template <int DT, int H, int D, int MAXQ, bool FUSED>
__device__ __forceinline__ void indexer_decode_body(const IndexerDecodeParams& p, int wg, uint32_t* smem,
                                                    uint32_t epoch) {
  // dynamic LDS: sc[MAXQ][cap] | qhist[MAXQ][2048] (one radix histogram per
  // query) | s_bt[stage_pages] | xs (bf16 with several queries: the two 16-KiB
  // slots of the shared key steps, 16-B aligned)
  uint32_t* sc = smem;
  uint32_t* qhist = smem + (size_t)MAXQ * p.chunk_cap;
  int* s_bt = (int*)(qhist + MAXQ * kRadixBins);
  u32x4* xs = (u32x4*)(smem + xchg_offset_words(MAXQ, p.chunk_cap, p.stage_pages));
  __shared__ int s_seqinfo[8];
  __shared__ int s_scan[kIdxThreads];
  __shared__ int s_rank[kIdxWaves + 1];
  __shared__ uint32_t s_prefix[MAXQ], s_pmask[MAXQ];
  __shared__ int s_need[MAXQ], s_state[MAXQ], s_take[MAXQ], s_candn[MAXQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  WsLayout W{p.ws, p.ws_nseq, p.ws_nq, p.ws_grid_pad};
  DSA_STAMP(0);

  // ---- 1. which sequence / page range this workgroup owns ------------------
  // pages_b = ceil(L_b / P); sequence b gets ceil(pages_b / cap) workgroups of
  // at most cap pages each, cap being the smallest with sum_b ceil(pages_b /
  // cap) <= grid.  Binary search between ceil(sum pages / grid) and
  // ceil(sum pages / (grid - B)), which always fits (each sequence's last
  // workgroup wastes less than one) and is the bound the host sizes LDS by.
  if (tid < kWave) {
    // page counts of the first kPgRegs * 64 sequences stay in registers for
    // the search below (each pass would otherwise wait on a reload)
    constexpr int kPgRegs = 4;
    int pgr[kPgRegs];
#pragma unroll
    for (int r = 0; r < kPgRegs; r++) {
      const int b = 64 * r + lane;
      pgr[r] = (b < bv.batch) ? (bv.seq_lens[b] + P - 1) >> bv.page_shift : 0;
    }
    auto pages = [&](int b0) -> int {
      const int b = b0 + lane;
      int v = 0;
#pragma unroll
      for (int r = 0; r < kPgRegs; r++) v = (b0 == 64 * r) ? pgr[r] : v;
      if (b0 >= 64 * kPgRegs) v = (b < bv.batch) ? (bv.seq_lens[b] + P - 1) >> bv.page_shift : 0;
      return v;
    };
    int tot = 0;
    for (int b0 = 0; b0 < bv.batch; b0 += kWave) tot += wave_sum(pages(b0));
    int cap = (tot + (p.grid - bv.batch) - 1) / (p.grid - bv.batch);
    if (tot > 0) {
      int lo = (tot + p.grid - 1) / p.grid;
      while (lo < cap) {  // uniform over the wave: every bound comes from a wave sum
        const int mid = (lo + cap) / 2;
        int wgs = 0;
        for (int b0 = 0; b0 < bv.batch; b0 += kWave) wgs += wave_sum((pages(b0) + mid - 1) / mid);
        if (wgs <= p.grid) cap = mid;
        else lo = mid + 1;
      }
    }
    int acc = 0, found = 0;
    for (int b0 = 0; b0 < bv.batch && !found; b0 += kWave) {
      const int b = b0 + lane;
      const int pg = pages(b0);
      const int nb = (cap > 0) ? (pg + cap - 1) / cap : 0;
      // inclusive prefix of nb over the wave
      int inc = nb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(inc, o);
        if (lane >= o) inc += v;
      }
      const int start = acc + inc - nb;
      const bool mine = (b < bv.batch) && wg >= start && wg < start + nb;
      const uint64_t m = __ballot(mine);
      if (m) {
        const int src = __ffsll((unsigned long long)m) - 1;
        if (lane == src) {
          s_seqinfo[0] = b;
          s_seqinfo[1] = wg - start;  // j
          s_seqinfo[2] = nb;
          s_seqinfo[3] = cap;
          s_seqinfo[4] = pg;
        }
        found = 1;
      }
      acc += __shfl(inc, 63);
    }
    if (lane == 0 && !found) s_seqinfo[0] = -1;
  }
  __syncthreads();
  const int b = s_seqinfo[0];
  if (b < 0) return;  // surplus workgroup: owns nothing, joins no barrier
  const int j = s_seqinfo[1], nb = s_seqinfo[2], cap = s_seqinfo[3], npg = s_seqinfo[4];
  const int L = bv.seq_lens[b];
  const int tok0 = bv.cu_q[b];
  const int T = bv.cu_q[b + 1] - tok0;
  const int s0 = j * cap * P;
  int s1 = min(min(npg, (j + 1) * cap) * P, L);
  if (s1 - s0 > p.chunk_cap) {  // cannot happen with the host's bound; stay in LDS bounds
    if (tid == 0) atomic_add_agent(W.err(), 2u);
    s1 = s0 + p.chunk_cap;
  }
  const int nloc = s1 - s0;
  const int* bt = bv.block_table + (size_t)b * bv.max_pages;
  const int K = p.topk;
  uint32_t* ctr = W.seq_ctr(p.seq_base + b);
  uint32_t* failed = W.seq_failed(p.seq_base + b);
  auto put_row = [&](int32_t* row, int i, int v) {
    if constexpr (FUSED) store_agent_i32(row + i, v);
    else row[i] = v;
  };

  if (tid < MAXQ) {
    s_prefix[tid] = 0u;
    s_pmask[tid] = 0u;
    s_need[tid] = K;
    int st = kActive;
    if (tid >= T) st = kAll;                       // no such query
    else if (L - T + tid + 1 <= K) st = kAll;      // every visible position is kept
    s_state[tid] = st;
    s_take[tid] = 0;
    s_candn[tid] = 0;
  }
  __syncthreads();

  // ---- queries that keep every visible position: slot s <- position s -------
  for (int q = 0; q < T && q < MAXQ; q++) {
    const int t = L - T + q;
    if (t + 1 > K) continue;
    int32_t* row = p.idx_out + (size_t)(tok0 + q) * K;
    for (int s = s0 + tid; s < s1; s += kIdxThreads)
      if (s <= t) put_row(row, s, s);
    if (j == 0)
      for (int s = t + 1 + tid; s < K; s += kIdxThreads) put_row(row, s, -1);
  }
  bool any_active = false;
  for (int q = 0; q < MAXQ; q++) any_active |= (s_state[q] == kActive);
  if (!any_active) {  // uniform over the sequence's workgroups
    if constexpr (FUSED) {
      // rows written above; the last workgroup out publishes them
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) {
        const uint32_t tk = atomic_add_agent(W.seq_exit(p.seq_base + b), 1u);
        if (tk == (uint32_t)(nb - 1)) {
          store_relaxed_agent(W.seq_exit(p.seq_base + b), 0u);
          if (T > 0 && p.publish_ready) store_relaxed_agent(W.seq_ready(p.seq_base + b), epoch);
        }
      }
    }
    return;
  }
  DSA_STAMP(1);

  // ---- 2. scores of this page range, kept in LDS as orderable keys ----------
  // The workgroup's slice of the block table is staged in LDS first, so the
  // address of a tile is an LDS lookup rather than a dependent global load.
  const int PS = bv.page_shift;
  const int pg0 = s0 >> PS;
  const int npg_loc = (s1 > s0) ? ((s1 - 1) >> PS) + 1 - pg0 : 0;
  const bool staged = npg_loc <= p.stage_pages;
  if (!staged && tid == 0) atomic_add_agent(W.err(), 4u);  // host sizing guarantees staging
  for (int i = tid; i < npg_loc && staged; i += kIdxThreads) s_bt[i] = bt[pg0 + i];
  // the first radix pass's histograms fill while the keys are scored
  for (int i = tid; i < MAXQ * kRadixBins / 4; i += kIdxThreads) ((u32x4*)qhist)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  {
    MfmaScorer<DT, H, D> scorer;
    using Tile = typename MfmaScorer<DT, H, D>::Tile;
    // tiles held per wave: the one being scored and kAhead in flight
    constexpr int kAhead = (DT == kFP8 || DT == kMX) ? 4 : 2;
    constexpr int RD = kAhead + 1;
    const int ntiles = (nloc + 31) / 32;
    // STAGED: the page table slice is in LDS (always, by the host's sizing);
    // the other instance is the fallback that reads it from memory.  Kept as
    // two loops so the staged one's lookups stay LDS loads: a pointer that
    // may point to either compiles to flat loads, which count as memory loads,
    // so the wait for a page id would drain the whole tile ring.
    auto score_range = [&](auto staged_c) {
      constexpr bool STAGED = decltype(staged_c)::value;
      auto page_of = [&](int s) { return STAGED ? s_bt[(s >> PS) - pg0] : bt[s >> PS]; };
      auto fetch = [&](int tile, Tile& t) {
        if (tile < ntiles) {
          const int s = min(s0 + 32 * tile + (lane & 31), s1 - 1);
          scorer.load_tile(p, ((int64_t)page_of(s) << PS) + (s & (P - 1)), t);
        }
      };
      // Every query of the sequence is scored in the same sweep over the
      // tiles, so each key is brought from memory once: the waves form QG
      // groups, one per query (QG = 1 for one query, 2 for two, 4 for three
      // or four), and the waves of a group take every (8 / QG)-th tile.  The
      // waves that read the same tile do so close together, on one CU.
      const int QG = (MAXQ == 1 || T <= 1) ? 1 : (T == 2) ? 2 : 4;
      const int q = wave % QG;
      if (q < T && q < MAXQ && s_state[q] == kActive) {
        const int t = L - T + q;
        const int phase = wave / QG, stride = kIdxWaves / QG;
        scorer.load_query(p, tok0 + q);
        uint32_t* scq = sc + (size_t)q * p.chunk_cap;
        uint32_t* hq = qhist + q * kRadixBins;
        Tile ring[RD];
#pragma unroll
        for (int d = 0; d < RD - 1; d++) fetch(phase + d * stride, ring[d]);
        for (int base = phase; base < ntiles; base += RD * stride) {
#pragma unroll
          for (int d = 0; d < RD; d++) {
            const int tile = base + d * stride;
            if (tile < ntiles) {
              // refill the slot of the previous tile with the one kAhead later
              fetch(tile + kAhead * stride, ring[(d + RD - 1) % RD]);
              const float v = scorer.score(p, 0, ring[d]);
              const int s = s0 + 32 * tile + lane;
              if (lane < 32 && s < s1) {
                const uint32_t x = (s <= t) ? float_key(v) : 0u;
                scq[s - s0] = x;
                if (x) atomicAdd(&hq[x >> 21], 1u);
              }
            }
          }
        }
      }
    };
    // Three or four query tokens (bf16): the four waves that score one 32-key
    // tile for different queries each load a quarter of a 64-key step and the
    // step is shared through LDS, so a wave's registers hold four times as
    // many distinct keys in flight as when every wave loads the whole tile.
    // Step c: 64 keys x 16 granules of 16 B; wave w loads LDS positions
    // 128 w + 64 i + lane (i = 0, 1), position n*16 + g holding granule
    // g ^ (n & 15) of key n, so the tile reads below hit 16 distinct bank
    // groups per 16 lanes.  Two slots alternate, one barrier per step: a slot
    // is rewritten two steps after it was read, across the barrier between.
    bool shared_done = false;
    if constexpr (DT == kBF16 && MAXQ == 4) {
      static_assert(D == 128 && kIdxWaves == 8, "four queries x two 32-key halves of a 64-key step");
      if (T >= 3 && staged && nloc > 0) {
        constexpr int R = kXchgRing;
        const int nsteps = (nloc + 63) / 64;
        const int q = wave & 3, ph = wave >> 2;
        const bool act = q < T && s_state[q] == kActive;
        if (act) scorer.load_query(p, tok0 + q);
        int key_i[2], seg_i[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          const int pos = 128 * wave + 64 * i + lane;
          key_i[i] = pos >> 4;
          seg_i[i] = (pos & 15) ^ (key_i[i] & 15);
        }
        auto fetch = [&](int c, u32x4 (&r)[2]) {
          c = min(c, nsteps - 1);  // past the end: reload the last step, unused
#pragma unroll
          for (int i = 0; i < 2; i++) {
            const int s = min(s0 + 64 * c + key_i[i], s1 - 1);
            const int64_t row = ((int64_t)s_bt[(s >> PS) - pg0] << PS) + (s & (P - 1));
            r[i] = ((const u32x4*)((const uint16_t*)p.k_data + row * D))[seg_i[i]];
          }
        };
        const int n = 32 * ph + (lane & 31);
        const int rbase = 16 * n, rx = n & 15, rh = 8 * (lane >> 5);
        const int t = L - T + q;
        uint32_t* scq = sc + (size_t)q * p.chunk_cap;
        uint32_t* hq = qhist + q * kRadixBins;
        auto store = [&](int c, float v) {
          const int s = s0 + 64 * c + 32 * ph + lane;
          if (lane < 32 && s < s1) {
            const uint32_t x = (s <= t) ? float_key(v) : 0u;
            scq[s - s0] = x;
            if (x) atomicAdd(&hq[x >> 21], 1u);
          }
        };
        f32x16 pacc[MfmaScorer<DT, H, D>::MT];
        int pc = -1;  // step whose products pacc holds, not yet summed
        u32x4 rg[R][2];
        // issued in step order (kept so by the scheduling barriers): the wait
        // before each step's LDS store then leaves the later steps in flight
#pragma unroll
        for (int d = 0; d < R - 1; d++) {
          fetch(d, rg[d]);
          __builtin_amdgcn_sched_barrier(0);
        }
        for (int base = 0; base < nsteps; base += R) {
#pragma unroll
          for (int d = 0; d < R; d++) {
            const int c = base + d;
            u32x4* slot = xs + (c & 1) * (kXchgSlotWords / 4);
            slot[128 * wave + lane] = rg[d][0];
            slot[128 * wave + 64 + lane] = rg[d][1];
            fetch(c + R - 1, rg[(d + R - 1) % R]);
            lds_barrier();
            // The two waves on a SIMD (phases 0 and 1) would otherwise run
            // their MFMAs together and then their head sums together; phase 1
            // sums its previous step after this barrier instead, so one
            // wave's VALU work overlaps the other's MFMAs.
            if (act) {
              Tile tl;
              if (c < nsteps) {
#pragma unroll
                for (int kk = 0; kk < MfmaScorer<DT, H, D>::KS; kk++) tl.v[kk] = slot[rbase + ((rh + kk) ^ rx)];
              }
              if (ph == 1 && pc >= 0) store(pc, scorer.head_sum(pacc));
              pc = -1;
              if (c < nsteps) {
                // the SIMD prefers this wave's MFMA issue over its partner's
                // VALU work while the products are queued
                __builtin_amdgcn_s_setprio(1);
                scorer.mma(tl, pacc);
                __builtin_amdgcn_s_setprio(0);
                pc = c;
              }
              if (ph == 0 && pc >= 0) store(pc, scorer.head_sum(pacc));
            }
          }
        }
        if (act && ph == 1 && pc >= 0) store(pc, scorer.head_sum(pacc));
        shared_done = true;
      }
    }
    if (!shared_done) {
      if (staged) score_range(std::true_type{});
      else score_range(std::false_type{});
    }
  }
  __syncthreads();
  DSA_STAMP(2);

  // ---- 3. radix passes ------------------------------------------------------
  // Every active query of the sequence goes through a pass together: one LDS
  // histogram per query (pass 0's filled while the keys were scored), one
  // cross-workgroup barrier per pass, and the global bin loads of all queries
  // in flight at once.
  __shared__ int s_scanq[MAXQ][kIdxWaves];
  __shared__ int s_binq[MAXQ], s_aboveq[MAXQ], s_bincntq[MAXQ];
  const int hand_cap = min(p.cand_cap, W.cand_pairs());
  int round = 0;
  for (int pass = 0; pass < kMaxPasses; pass++) {
    bool act = false;
    for (int q = 0; q < MAXQ; q++) act |= (s_state[q] == kActive);
    if (!act) break;
    const int shift = (pass == 0) ? 21 : (pass == 1) ? 10 : 0;
    const uint32_t dmask = (pass < 2) ? 0x7FFu : 0x3FFu;
    // pass 0's histograms were filled while scoring
    for (int q = 0; q < T && q < MAXQ && pass > 0; q++) {
      if (s_state[q] != kActive) continue;
      for (int i = tid; i < kRadixBins / 4; i += kIdxThreads) ((u32x4*)(qhist + q * kRadixBins))[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // each thread takes 8 consecutive keys per round (two 16-B LDS reads ahead
    // of their atomics; chunk_cap is a multiple of 8, so the reads stay inside
    // the buffer and keys past nloc are masked)
    for (int q = 0; q < T && q < MAXQ && pass > 0; q++) {
      if (s_state[q] != kActive) continue;
      const uint32_t pre = s_prefix[q], pm = s_pmask[q];
      const uint32_t* scq = sc + (size_t)q * p.chunk_cap;
      uint32_t* h = qhist + q * kRadixBins;
      for (int i0 = 8 * tid; i0 < nloc; i0 += 8 * kIdxThreads) {
        const u32x4 va = *(const u32x4*)(scq + i0);
        const u32x4 vb = *(const u32x4*)(scq + i0 + 4);
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const uint32_t x = (i0 + e < nloc) ? ((e < 4) ? va[e & 3] : vb[e & 3]) : 0u;
          if (x != 0u && (x & pm) == pre) atomicAdd(&h[(x >> shift) & dmask], 1u);
        }
      }
    }
    __syncthreads();
    for (int q = 0; q < T && q < MAXQ; q++) {
      if (s_state[q] != kActive) continue;
      uint32_t* gh = W.hist(tok0 + q, pass);
      for (int i = tid; i < kRadixBins; i += kIdxThreads) {
        const uint32_t c = qhist[q * kRadixBins + i];
        if (c) atomic_add_agent(&gh[i], c);
      }
    }
    DSA_STAMP(3 + 3 * pass);
    round++;
    group_barrier(ctr, (uint32_t)(nb * round) + p.barrier_slack, W.err(), failed, p.spin_limit);
    DSA_STAMP(4 + 3 * pass);
    // each thread owns kBinsPerThread consecutive bins of every query; suffix
    // sums from the top bin down
    uint32_t h8[MAXQ][kBinsPerThread];
    bool qa[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      qa[q] = q < T && s_state[q] == kActive;
      const uint32_t* gh = W.hist(tok0 + q, pass);
#pragma unroll
      for (int e = 0; e < kBinsPerThread; e++)
        h8[q][e] = qa[q] ? load_relaxed_agent(&gh[kBinsPerThread * tid + e]) : 0u;
    }
    if (tid < MAXQ) {
      s_binq[tid] = 0;
      s_aboveq[tid] = 0;
      s_bincntq[tid] = 0;
    }
    int xq[MAXQ];
    uint32_t csq[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      csq[q] = 0;
#pragma unroll
      for (int e = 0; e < kBinsPerThread; e++) csq[q] += h8[q][e];
      // suffix sums over the wave: counts of this lane and the lanes above
      int x = (int)csq[q];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(x, o);
        if (lane + o < 64) x += v;
      }
      xq[q] = x;
      if (lane == 0) s_scanq[q][wave] = x;  // wave total
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      if (!qa[q]) continue;
      int later = 0;
#pragma unroll
      for (int w = 0; w < kIdxWaves; w++) later += (w > wave) ? s_scanq[q][w] : 0;
      const int incl = xq[q] + later;            // this thread's bins and everything above
      const int above = incl - (int)csq[q];      // bins above this thread's own
      const int need = s_need[q];
      if (above < need && need <= above + (int)csq[q]) {
        int run = above;
        for (int e = kBinsPerThread - 1; e >= 0; e--) {
          if (run + (int)h8[q][e] >= need) {
            s_binq[q] = kBinsPerThread * tid + e;
            s_aboveq[q] = run;
            s_bincntq[q] = (int)h8[q][e];
            break;
          }
          run += (int)h8[q][e];
        }
      }
    }
    __syncthreads();
    if (tid < T && tid < MAXQ && s_state[tid] == kActive) {
      const int q = tid;
      const int nneed = s_need[q] - s_aboveq[q];
      s_need[q] = nneed;
      s_prefix[q] |= ((uint32_t)s_binq[q]) << shift;
      s_pmask[q] |= dmask << shift;
      if (s_bincntq[q] == nneed) {
        s_state[q] = kTakeBin;
      } else if (pass == 0 && s_bincntq[q] <= hand_cap) {
        // few enough keys share the boundary bin: the sequence's last
        // workgroup chooses among them (3c) instead of two more passes
        s_state[q] = kHandoff;
        s_candn[q] = s_bincntq[q];
      } else if (pass == kMaxPasses - 1) {
        s_state[q] = kTiePass;
      }
    }
    __syncthreads();
    DSA_STAMP(5 + 3 * pass);
  }
  DSA_STAMP(12);

  __shared__ int s_failed;
  __shared__ uint32_t s_ticket;
  uint32_t ticket = 0u;     // thread 0: this workgroup's exit ticket
  // ---- 3b. equal keys straddle the boundary: smallest positions win ---------
  bool any_tie = false;
  for (int q = 0; q < MAXQ; q++) any_tie |= (s_state[q] == kTiePass);
  if (any_tie) {
    for (int q = 0; q < T && q < MAXQ; q++) {
      if (s_state[q] != kTiePass) continue;
      const uint32_t pre = s_prefix[q];
      const uint32_t* scq = sc + (size_t)q * p.chunk_cap;
      int cnt = 0;
      for (int i = tid; i < nloc; i += kIdxThreads) cnt += (scq[i] == pre) ? 1 : 0;
      cnt = wave_sum(cnt);
      if (lane == 0) s_scan[wave] = cnt;
      __syncthreads();
      if (tid == 0) {
        int c = 0;
        for (int w = 0; w < kIdxWaves; w++) c += s_scan[w];
        __hip_atomic_store(&W.tie(tok0 + q)[j], (uint32_t)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
    round++;
    group_barrier(ctr, (uint32_t)(nb * round) + p.barrier_slack, W.err(), failed, p.spin_limit);
    for (int q = 0; q < T && q < MAXQ; q++) {
      if (s_state[q] != kTiePass) continue;
      if (tid == 0) {
        int lower = 0;
        const uint32_t* tc = W.tie(tok0 + q);
        for (int jj = 0; jj < j; jj++) lower += (int)load_relaxed_agent(&tc[jj]);
        s_take[q] = max(0, s_need[q] - lower);
      }
      __syncthreads();
    }
  }

  DSA_STAMP(13);
  // ---- 4. append this workgroup's selected positions ------------------------
  // Queries whose boundary bin is taken whole: every key at or above it.  Each
  // wave counts its keys of every such query; the workgroup reserves its slots
  // with one atomic per query (all a sequence's workgroups add to the same
  // counter, so fewer, larger reservations wait less on each other); then
  // each wave writes its keys from its offset within the workgroup's range.
  // Handed-off queries: the keys above the boundary bin go to the row the
  // same way, and the keys in it to the query's candidate list.
  bool any_hand = false;
  for (int q = 0; q < MAXQ; q++) any_hand |= (s_state[q] == kHandoff);
  {
    __shared__ int s_wcnt[MAXQ][kIdxWaves], s_wccnt[MAXQ][kIdxWaves];
    __shared__ int s_wgbase[MAXQ], s_cbase[MAXQ];
    bool tb[MAXQ], hd[MAXQ];
    int cnt[MAXQ], ccnt[MAXQ];
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      hd[q] = q < T && s_state[q] == kHandoff;
      tb[q] = hd[q] || (q < T && s_state[q] == kTakeBin);
      cnt[q] = 0;
      ccnt[q] = 0;
      if (!tb[q]) continue;
      const uint32_t pre = s_prefix[q], pm = s_pmask[q];
      const uint32_t* scq = sc + (size_t)q * p.chunk_cap;
      // lane: 4 consecutive keys per round, one 16-B LDS read
      int c = 0, cd = 0;
      for (int i0 = 4 * kWave * wave; i0 < nloc; i0 += 4 * kIdxThreads) {
        const int i = i0 + 4 * lane;
        const u32x4 v = (i < nloc) ? *(const u32x4*)(scq + i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t x = (i + e < nloc) ? v[e] : 0u;
          const uint32_t xm = x & pm;
          c += (x != 0u && (hd[q] ? xm > pre : xm >= pre)) ? 1 : 0;
          cd += (hd[q] && x != 0u && xm == pre) ? 1 : 0;
        }
      }
      cnt[q] = wave_sum(c);
      ccnt[q] = hd[q] ? wave_sum(cd) : 0;
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < MAXQ; q++) {
        s_wcnt[q][wave] = cnt[q];
        s_wccnt[q][wave] = ccnt[q];
      }
    }
    __syncthreads();
    // One thread reserves the workgroup's slots of every query and reads the
    // sequence's failure flag; without a tie pass or a handoff these are its
    // last accesses to shared workspace state, so it then takes the exit
    // ticket (ordered after the reservations).  The ticket's value is only
    // needed after the row writes, so it stays in a register and its latency
    // overlaps them.
    if (tid == 0) {
      uint32_t got[MAXQ], gotc[MAXQ];
#pragma unroll
      for (int q = 0; q < MAXQ; q++) {
        int tot = 0, totc = 0;
#pragma unroll
        for (int w = 0; w < kIdxWaves; w++) {
          tot += s_wcnt[q][w];
          totc += s_wccnt[q][w];
        }
        got[q] = tot ? atomic_add_agent(W.outcnt(tok0 + q), (uint32_t)tot) : 0u;
        gotc[q] = totc ? atomic_add_agent(W.candcnt(tok0 + q), (uint32_t)totc) : 0u;
      }
      const uint32_t fl = load_relaxed_agent(failed);
#pragma unroll
      for (int q = 0; q < MAXQ; q++) {
        s_wgbase[q] = (int)got[q];
        s_cbase[q] = (int)gotc[q];
      }
      s_failed = fl != 0u;
      if (!FUSED && !any_tie && !any_hand) {
        __builtin_amdgcn_s_waitcnt(0);
        ticket = atomic_add_agent(W.seq_exit(p.seq_base + b), 1u);
      }
    }
    __syncthreads();
    // a failed sequence writes no rows: its last workgroup out poisons them
    const bool write_rows = !s_failed;
#pragma unroll
    for (int q = 0; q < MAXQ; q++) {
      if (!tb[q] || !write_rows) continue;
      const uint32_t pre = s_prefix[q], pm = s_pmask[q];
      const uint32_t* scq = sc + (size_t)q * p.chunk_cap;
      int32_t* row = p.idx_out + (size_t)(tok0 + q) * K;
      uint64_t* cl = W.cand(tok0 + q);
      int base = s_wgbase[q], cbase = s_cbase[q];
#pragma unroll
      for (int w = 0; w < kIdxWaves; w++) {
        base += (w < wave) ? s_wcnt[q][w] : 0;
        cbase += (w < wave) ? s_wccnt[q][w] : 0;
      }
      for (int i0 = 4 * kWave * wave; i0 < nloc; i0 += 4 * kIdxThreads) {
        const int i = i0 + 4 * lane;
        const u32x4 v = (i < nloc) ? *(const u32x4*)(scq + i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t x = (i + e < nloc) ? v[e] : 0u;
          const uint32_t xm = x & pm;
          const bool sel = x != 0u && (hd[q] ? xm > pre : xm >= pre);
          const uint64_t m = __ballot(sel);
          const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          if (sel && base + r < K) put_row(row, base + r, s0 + i + e);
          base += __popcll(m);
          if (hd[q]) {
            const bool cd = x != 0u && xm == pre;
            const uint64_t mc = __ballot(cd);
            const int rc = __builtin_amdgcn_mbcnt_hi((uint32_t)(mc >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mc, 0));
            if (cd && cbase + rc < hand_cap)
              __hip_atomic_store(cl + cbase + rc, (uint64_t)x | ((uint64_t)(uint32_t)(s0 + i + e) << 32),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            cbase += __popcll(mc);
          }
        }
      }
    }
  }
  for (int q = 0; q < T && q < MAXQ; q++) {
    const int st = s_state[q];
    if (st != kTiePass) continue;
    const uint32_t pre = s_prefix[q], pm = s_pmask[q];
    const int take = s_take[q];
    const uint32_t* scq = sc + (size_t)q * p.chunk_cap;
    int32_t* row = p.idx_out + (size_t)(tok0 + q) * K;
    uint32_t* oc = W.outcnt(tok0 + q);
    // equal keys straddle the boundary: ties are taken in position order, so
    // rank them across the whole workgroup
    __shared__ int s_base;
    int mine = 0, ties_seen = 0;
    for (int i0 = 0; i0 < nloc; i0 += kIdxThreads) {
      const int i = i0 + tid;
      const uint32_t x = (i < nloc) ? scq[i] : 0u;
      const bool above = x != 0u && (x & pm) > pre;
      const bool tie = x != 0u && (x & pm) == pre;
      int tot_tie;
      const int r = block_rank(tie, s_rank, tot_tie);
      const bool sel = above || (tie && ties_seen + r < take);
      int tot_sel;
      (void)block_rank(sel, s_rank, tot_sel);
      mine += tot_sel;
      ties_seen += tot_tie;
    }
    if (tid == 0) {
      s_base = (int)atomic_add_agent(oc, (uint32_t)mine);
      s_failed = load_relaxed_agent(failed) != 0u;
    }
    __syncthreads();
    int base = s_base;
    ties_seen = 0;
    for (int i0 = 0; i0 < nloc; i0 += kIdxThreads) {
      const int i = i0 + tid;
      const uint32_t x = (i < nloc) ? scq[i] : 0u;
      const bool above = x != 0u && (x & pm) > pre;
      const bool tie = x != 0u && (x & pm) == pre;
      int tot_tie;
      const int r = block_rank(tie, s_rank, tot_tie);
      const bool sel = above || (tie && ties_seen + r < take);
      int tot_sel;
      const int rs = block_rank(sel, s_rank, tot_sel);
      if (sel && base + rs < K && !s_failed) put_row(row, base + rs, s0 + i);
      base += tot_sel;
      ties_seen += tot_tie;
    }
    __syncthreads();
  }
  DSA_STAMP(14);

  // ---- 5. the sequence's last workgroup out ---------------------------------
  // A workgroup takes its exit ticket after its last access to the shared
  // workspace state (its histogram atomics, tie counts and slot reservations
  // are performed by then), so the one that draws the last ticket sees the
  // sequence's use of the workspace finished.  If any of the sequence's
  // bounded waits gave up, the workgroups that saw the failure flag wrote no
  // rows and this one overwrites the scored queries' rows with -1 (a visible
  // failure: no valid row has -1 in slot 0).  It then clears everything the
  // sequence used in the workspace; plain stores suffice, as the next launch
  // sees them.
  {
    __shared__ int s_last;
    // (FUSED: the ticket also follows this workgroup's row writes, so the
    // last one out knows every row of the sequence complete; a handoff: it
    // follows the candidate writes, so the last one out finds every list
    // complete)
    if (FUSED || any_tie || any_hand) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0) ticket = atomic_add_agent(W.seq_exit(p.seq_base + b), 1u);
    }
    if (tid == 0) s_ticket = ticket;
    __syncthreads();
    if (tid == 0) s_last = (s_ticket == (uint32_t)(nb - 1));
    __syncthreads();
    if (s_last) {
      const bool poison = load_relaxed_agent(failed) != 0u;
      // ---- 3c. handed-off boundary bins: the last workgroup out chooses the
      // remaining s_need keys among the bin's candidates (every workgroup's
      // list entries were written before its ticket).  The list holds exactly
      // the bin's count unless a wait gave up, which poisons the rows anyway.
      // (every query's count is read: after a failed wait the workgroups may
      // not all have agreed on the handoff, and the list is cleared below)
      __shared__ int s_nc[MAXQ];
      if (tid < MAXQ)
        s_nc[tid] = (tid < T && L - T + tid + 1 > K)
                        ? (int)min(load_relaxed_agent(W.candcnt(tok0 + tid)), (uint32_t)hand_cap) : 0;
      __syncthreads();
      __shared__ int s_hand[MAXQ];
      if (tid < MAXQ) s_hand[tid] = tid < T && s_state[tid] == kHandoff && !poison && s_nc[tid] == s_candn[tid];
      __syncthreads();
      bool any_sel = false;
      for (int q = 0; q < T && q < MAXQ; q++) {
        any_sel |= s_hand[q] != 0;
        if (s_state[q] != kHandoff || poison || s_hand[q]) continue;
        // the list does not hold the bin's count: cannot happen when no
        // wait gave up; the row is poisoned and the error reported
        int32_t* row = p.idx_out + (size_t)(tok0 + q) * K;
        if (tid == 0) atomic_add_agent(W.err(), 8u);
        for (int s = tid; s < K; s += kIdxThreads) put_row(row, s, -1);
      }
      if (any_sel) {
        for (int q0 = 0; q0 < T && q0 < MAXQ; q0++)
          handoff_select<1>(W, tok0 + q0, T - q0, s_hand + q0, s_nc + q0, s_need + q0, p.idx_out, K, smem, put_row);
      }
      for (int q = 0; q < T && q < MAXQ; q++) {
        if (L - T + q + 1 <= K) continue;        // kept every position: no scores, no workspace
        const int g = tok0 + q;
        if (poison) {
          int32_t* row = p.idx_out + (size_t)g * K;
          for (int s = tid; s < K; s += kIdxThreads) put_row(row, s, -1);
        }
        u32x4* h0 = (u32x4*)W.qa(g);              // hist0, outcnt, candcnt and the pad
        for (int i = tid; i < 2080 / 4; i += kIdxThreads) h0[i] = u32x4{0u, 0u, 0u, 0u};
        u32x4* h12 = (u32x4*)W.hist(g, 1);        // hist1, hist2 (or the candidate list)
        for (int i = tid; i < 4096 / 4; i += kIdxThreads) h12[i] = u32x4{0u, 0u, 0u, 0u};
        uint32_t* tw = W.tie(g);                  // tie counts (or the list's tail)
        const int tail = max(nb, 2 * s_nc[q] - 4096);
        for (int i = tid; i < tail; i += kIdxThreads) tw[i] = 0u;
      }
      if (tid < 3) W.seq_ctr(p.seq_base + b)[tid] = 0u;   // barrier, exit, failure
      if constexpr (FUSED) {
        // every workgroup's rows were complete before its ticket, the
        // poisoning above before this
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0 && T > 0 && p.publish_ready) store_relaxed_agent(W.seq_ready(p.seq_base + b), epoch);
      }
    }
  }
}

}  // namespace dsa
