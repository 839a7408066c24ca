// Sparse Flash Attention over the rows the indexer selected.
//
// Method: SFA reads the main-attention KV entries at the selected indices and
// computes attention over that sparse subset only ("Deep Fusion of LI and SFA",
// Day0 Inference Optimization on Ascend CANN, sec. 2; Adapting and Optimizing
// Inference for a New Model Architecture on Ascend, sec. 3.1; Inference
// Acceleration for Next-Gen Attention Architectures, sec. 3.2 on the
// non-contiguous paged gather).  MLA is used in its absorbed form: one latent
// row [Dqk] per position is shared by every head, the logits use all Dqk
// columns and V is the first Dv columns of the same row.
//
// bf16 kernel (H = 128, Dqk = 576, Dv = 512): a workgroup owns one query token,
// a group of 64 heads and a contiguous range of index slots.  Per tile of 32
// slots it gathers the 32 latent rows through the block table into LDS
// (double-buffered), then every wave (16 heads) computes
//   S^T[row, head] = KV[row, :] . q[head, :]     (16x16x32 bf16 MFMAs, rows on M)
// so that after the online-softmax update the probabilities already sit in the
// B-operand layout of the second product
//   O^T[v, head] += V^T[v, row] P^T[row, head]   (V^T read with ds_read_b64_tr_b16).
// Slots holding -1 are masked.  With several slot ranges per token, each range
// writes a normalised partial and its log-sum-exp, merged by sfa_combine.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kSfaThreads = 256;

__device__ __forceinline__ int find_seq(const BatchView& bv, int tok) {
  // largest b with cu_q[b] <= tok (binary search over cu_q[0..batch])
  int lo = 0, hi = bv.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bv.cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Workgroup barrier that waits only for this wave's LDS traffic, not for its
// outstanding global->LDS tile loads (a plain __syncthreads() waits for every
// memory operation, which would drain the load pipeline at each barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte-per-lane global->LDS load (64 lanes fill lds_base .. +1 KiB in
// lane order).  Issued through inline assembly so that the compiler's
// wait-count pass, which cannot tell these LDS writes apart from the LDS reads
// of other ring slots, does not drain every in-flight tile before each read;
// the kernel orders them itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima): gfx9 encoding.
#define DSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

constexpr int kSfaHeadsPerWG = 64;
constexpr int kSfaBf16Threads = 512;

// bf16 SFA, H = 128, Dqk = 576, Dv = 512.
//
// A workgroup serves 64 heads of one token and one range of index slots with
// 8 waves (two per SIMD): wave w takes the 16 heads 16*(w%4) .. +15 of the
// group together with its partner w ^ 4.  The pair splits the QK^T
// contraction (half = w/4 takes dims [288*half, 288*half + 288)) and exchanges
// the 32x16 partial logits through LDS, then splits the PV columns (half takes
// v in [256*half, 256*half + 256)).  Per wave that is q^T in 36 registers and
// the O^T accumulators in 64.  The two head groups of a token run as
// workgroups 8 apart in launch order, which places them on the same XCD, so
// the second gather of each row hits that XCD's L2.
//
// Per tile of 32 index slots:
//   S^T[row, head] = KV[row, :] . q[head, :]     16x16x32 bf16 MFMAs, rows on M
//   online softmax per head (lazy rescaling, see below)
//   O^T[v, head] += V^T[v, row] P^T[row, head]   V^T read with ds_read_b64_tr_b16
// The probabilities leave the first product already in the B-operand layout
// of the second.  Rows stream through a 3-deep ring of LDS tiles filled by
// direct global->LDS loads; slots holding -1 are masked.
template <int DQK, int DV>
__global__ __launch_bounds__(kSfaBf16Threads, 1) void sfa_bf16_kernel(SfaParams p) {
  constexpr int ROWB = DQK * 2;              // bytes of one latent row (1152)
  constexpr int PITCH = ROWB + 16;           // LDS bytes per row (73 chunks of 16 B)
  constexpr int TR = 32;                     // rows per tile
  constexpr int TILE = 40 * 1024;            // 32 rows of PITCH bytes, rounded up to whole loads
  constexpr int NBUF = 3;                    // tiles in flight
  constexpr int NW = kSfaBf16Threads / 64;   // 8 waves
  constexpr int LPW = TILE / 1024 / NW;      // 1-KiB load instructions per wave per tile (5)
  constexpr int KSH = DQK / 32 / 2;          // QK^T K-steps of 32 per wave (9)
  constexpr int MVH = DV / 16 / 2;           // PV M-tiles of 16 columns per wave (16)
  static_assert(TILE % (1024 * NW) == 0, "tile must split into whole 1-KiB loads per wave");
  static_assert(TR * PITCH <= TILE, "tile rows must fit the buffer");
  extern __shared__ __attribute__((aligned(16))) unsigned char sfa_smem[];
  float* s_x = (float*)(sfa_smem + NBUF * TILE);                      // [8 waves][8][64] partial logits
  int32_t* s_rows = (int32_t*)(sfa_smem + NBUF * TILE + NW * 2048);   // [rows_per_split]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, l16 = lane & 15;
  // optional phase clocks of the first workgroup's first wave (profiling)
  const bool prof = p.dbg && blockIdx.x == 0 && blockIdx.z == 0 && tid == 0;
  unsigned long long ph[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  unsigned long long tprev = prof ? __builtin_amdgcn_s_memtime() : 0;
#define DSA_PHASE(i)                                             \
  if (prof) {                                                    \
    const unsigned long long tn = __builtin_amdgcn_s_memtime();  \
    ph[i] += tn - tprev;                                         \
    tprev = tn;                                                  \
  }
  const int hg = wave & 3, half = wave >> 2;
  // launch order L -> (token, head block): L = 16*(t/8) + 8*hb + t%8
  const int L = blockIdx.x;
  const int g = 8 * (L >> 4) + (L & 7);
  const int hb = (L >> 3) & 1;
  const int split = blockIdx.z;
  if (g >= p.bv.total_q) return;
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  const int H = 2 * kSfaHeadsPerWG;
  const int b = find_seq(bv, g);
  const int* bt = bv.block_table + (size_t)b * bv.max_pages;
  const int slot0 = split * p.rows_per_split;
  const int nslots = max(0, min(p.topk - slot0, p.rows_per_split));
  const int32_t* idx = p.idx + (size_t)g * p.topk + slot0;

  for (int r = tid; r < nslots; r += kSfaBf16Threads) {
    const int pos = idx[r];
    s_rows[r] = (pos >= 0) ? bt[pos / P] * P + (pos % P) : -1;
  }
  __syncthreads();
  int fallback = -1;
  for (int r = 0; r < nslots && fallback < 0; r++) fallback = s_rows[r];
  DSA_PHASE(0);

  // q^T as the B operand of S^T = KV q^T (16x16x32): lane l holds head
  // 16*hg + l%16 and dims 288*half + 32*kk + 8*(l/16) .. +7 of K-step kk.
  const int head = kSfaHeadsPerWG * hb + 16 * hg + l16;
  bf16x8 qb[KSH];
  {
    const bf16x8* qs = (const bf16x8*)((const uint16_t*)p.q + ((size_t)g * H + head) * DQK);
#pragma unroll
    for (int k = 0; k < KSH; k++) qb[k] = qs[4 * (KSH * half + k) + grp];
  }
  f32x4 o[MVH];
#pragma unroll
  for (int i = 0; i < MVH; i++) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // every compiler-visible load is complete before the tile loop, so the
  // compiler's own waits never count the loop's asm-issued tile loads
  __builtin_amdgcn_s_waitcnt(0);
  DSA_PHASE(1);

  const int ntiles = (fallback >= 0) ? (nslots + TR - 1) / TR : 0;
  // Row r of a tile sits at byte r * PITCH of its buffer.  The 16-byte pad
  // makes consecutive rows start 9 bank groups apart (73 = 9 mod 16), so 16
  // rows read at one column, and 4 rows x 2 chunks read by the transposing
  // loads, hit distinct banks.  Each wave fills whole 1-KiB stretches of the
  // buffer; lanes that land on a pad or on the slack after row 31 load chunk 0
  // of the tile's row 0.
  int ld_row[LPW], ld_col[LPW];
#pragma unroll
  for (int k = 0; k < LPW; k++) {
    const int off = (wave + NW * k) * 1024 + lane * 16;
    const int r = off / PITCH, c = (off % PITCH) / 16;
    const bool real = r < TR && c < ROWB / 16;
    ld_row[k] = real ? r : 0;
    ld_col[k] = real ? c * 16 : 0;
  }
  auto issue = [&](int tile) {
    unsigned char* buf = sfa_smem + (tile % NBUF) * TILE;
    int rows[LPW];
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      const int slot = tile * TR + ld_row[k];
      rows[k] = (slot < nslots) ? s_rows[slot] : -1;
    }
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      const int row = (rows[k] < 0) ? fallback : rows[k];
      const unsigned char* src = (const unsigned char*)p.kv + (size_t)row * ROWB + ld_col[k];
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(buf + (wave + NW * k) * 1024)));
    }
  };
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  for (int tile = 0; tile < ntiles; tile++) {
    if (tile + 2 < ntiles) {
      issue(tile + 2);
      DSA_WAIT_VMCNT(2 * LPW);
    } else if (tile + 1 < ntiles) {
      DSA_WAIT_VMCNT(LPW);
    } else {
      DSA_WAIT_VMCNT(0);
    }
    // rows of this tile that hold a selected position (bit r)
    const int rslot = tile * TR + (lane & 31);
    const uint32_t valid = (uint32_t)__ballot(lane < 32 && rslot < nslots && s_rows[rslot] >= 0);
    DSA_PHASE(2);
    lds_barrier();
    DSA_PHASE(3);
    const unsigned char* cur = sfa_smem + (tile % NBUF) * TILE;

    // ---- partial S^T[row, head] over this half's dims: two 16-row M-tiles
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    {
      const unsigned char* rp = cur + l16 * PITCH + (288 * half + 8 * grp) * 2;
#pragma unroll
      for (int k = 0; k < KSH; k++) {
        const bf16x8 a0 = *(const bf16x8*)(rp + 64 * k);
        const bf16x8 a1 = *(const bf16x8*)(rp + 16 * PITCH + 64 * k);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb[k], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb[k], s1, 0, 0, 0);
      }
    }
    float* xw = s_x + wave * 512 + lane;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      xw[64 * e] = s0[e];
      xw[64 * (4 + e)] = s1[e];
    }
    DSA_PHASE(4);
    lds_barrier();
    const float* xr = s_x + (wave ^ 4) * 512 + lane;
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      z[e] = s0[e] + xr[64 * e];
      z[4 + e] = s1[e] + xr[64 * (4 + e)];
    }

    // ---- online softmax for head l%16; this lane holds rows 4*grp + i and
    // 16 + 4*grp + i (i < 4)
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int r = 16 * (e >> 2) + 4 * grp + (e & 3);
      z[e] = ((valid >> r) & 1u) ? z[e] * p.scale_log2 : -INFINITY;
      mt = fmaxf(mt, z[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // Lazy rescaling: the reference maximum m_run only moves when the tile's
    // maximum exceeds it by more than 8 (log2 units), so probabilities stay
    // below 2^8 (exact in fp32, in range for bf16) and the accumulators are
    // rescaled only on those rare jumps.  The result is independent of m_run.
    float alpha = 1.f;
    if (m_run == -INFINITY) {
      m_run = mt;                         // nothing accumulated yet
    } else if (mt > m_run + 8.f) {
      alpha = exp2f(m_run - mt);
      m_run = mt;
    }
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < MVH; i++) o[i] *= alpha;
    }
    const bool none = (m_run == -INFINITY);
    float psum = 0.f;
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      // the denominator sums the same bf16-rounded weights the PV product uses
      const __bf16 pv = (__bf16)(none ? 0.f : __builtin_amdgcn_exp2f(z[e] - m_run));
      psum += (float)pv;
      pb[e] = pv;
    }
    l_run = l_run * alpha + psum;
    DSA_PHASE(5);

    // ---- O^T[v, head] += V^T[v, rows] P^T[rows, head]: 16 columns on M, heads
    // on N, K = the tile's 32 rows.  This lane's K-slots 8*grp .. +7 hold rows
    // 4*grp + j and 16 + 4*grp + j (j < 4), matching pb.  V^T comes from
    // ds_read_b64_tr_b16: in each 16-lane group, source lane s = 4j + r reads
    // columns vbase + 4r .. +3 of row j of the group's 4 rows; lane i then holds
    // column vbase + i of those 4 rows.
    {
      const int r0 = 4 * grp + (l16 >> 2);
      const unsigned char* rp0 = cur + r0 * PITCH + (256 * half + 4 * (l16 & 3)) * 2;
      const unsigned char* rp1 = rp0 + 16 * PITCH;
#pragma unroll
      for (int mv = 0; mv < MVH; mv++) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rp0 + 32 * mv));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rp1 + 32 * mv));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, o[mv], 0, 0, 0);
      }
    }
    lds_barrier();
    DSA_PHASE(6);
  }

  // ---- epilogue: o[mv][i] holds head l%16, v = 256*half + 16*mv + 4*grp + i
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  if (p.splits == 1) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)g * H + head) * DV;
#pragma unroll
    for (int mv = 0; mv < MVH; mv++) {
      const int v = 256 * half + 16 * mv + 4 * grp;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(o[mv][0] * inv) | ((uint32_t)f32_to_bf16(o[mv][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(o[mv][2] * inv) | ((uint32_t)f32_to_bf16(o[mv][3] * inv) << 16);
      *(uint2*)(out + v) = pk;
    }
    if (p.lse && grp == 0 && half == 0)
      p.lse[(size_t)g * H + head] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  } else {
    float* po = p.part_o + (((size_t)g * p.splits + split) * H + head) * DV;
#pragma unroll
    for (int mv = 0; mv < MVH; mv++) *(f32x4*)(po + 256 * half + 16 * mv + 4 * grp) = o[mv] * inv;
    if (grp == 0 && half == 0)
      p.part_ml[((size_t)g * p.splits + split) * H + head] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
  }
  DSA_PHASE(7);
  if (prof)
    for (int i = 0; i < 8; i++) p.dbg[i] = ph[i];
#undef DSA_PHASE
}

// Merge the per-range partials of one token: weights 2^(lse_j - lse).  One
// workgroup per (token, group of 4 heads); each thread owns DV/64 columns.
template <int DV, bool BF16OUT>
__global__ __launch_bounds__(256) void sfa_combine_kernel(SfaParams p, int H) {
  constexpr int CPT = DV / 64;  // columns per thread
  const int g = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int c0 = (threadIdx.x & 63) * CPT;
  const int S = p.splits;
  if (h >= H) return;
  float mx = -INFINITY;
  for (int j = 0; j < S; j++) mx = fmaxf(mx, p.part_ml[((size_t)g * S + j) * H + h]);
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c++) acc[c] = 0.f;
  float den = 0.f;
  for (int j = 0; j < S; j++) {
    const float l = p.part_ml[((size_t)g * S + j) * H + h];
    if (l == -INFINITY) continue;
    const float wj = exp2f(l - mx);
    den += wj;
    const float* src = p.part_o + (((size_t)g * S + j) * H + h) * DV + c0;
    if constexpr (CPT % 4 == 0) {
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        const f32x4 v = *(const f32x4*)(src + c);
        acc[c] += wj * v[0]; acc[c + 1] += wj * v[1]; acc[c + 2] += wj * v[2]; acc[c + 3] += wj * v[3];
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPT; c++) acc[c] += wj * src[c];
    }
  }
  const float inv = (den > 0.f) ? 1.f / den : 0.f;
  if constexpr (BF16OUT && CPT % 4 == 0) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)g * H + h) * DV + c0;
#pragma unroll
    for (int c = 0; c < CPT; c += 4) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc[c] * inv) | ((uint32_t)f32_to_bf16(acc[c + 1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc[c + 2] * inv) | ((uint32_t)f32_to_bf16(acc[c + 3] * inv) << 16);
      *(uint2*)(out + c) = pk;
    }
  } else {
    float* out = (float*)p.out + ((size_t)g * H + h) * DV + c0;
#pragma unroll
    for (int c = 0; c < CPT; c++) out[c] = acc[c] * inv;
  }
  if (p.lse && (threadIdx.x & 63) == 0)
    p.lse[(size_t)g * H + h] = (den > 0.f) ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
}

// f32 SFA for small head counts and widths: one workgroup per (token, range),
// scalar FMAs.  Thread (h, r) computes one logit per tile; thread (h, v) keeps
// output columns.
template <int H, int DQK, int DV>
__global__ __launch_bounds__(256) void sfa_f32_kernel(SfaParams p) {
  constexpr int TR = 32;
  __shared__ float s_q[H][DQK];
  __shared__ float s_kv[TR][DQK + 1];
  __shared__ float s_p[H][TR];
  __shared__ float s_m[H], s_l[H], s_alpha[H];
  __shared__ int s_row[TR];
  const int tid = threadIdx.x;
  const int g = blockIdx.x, split = blockIdx.z;
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  const int b = find_seq(bv, g);
  const int* bt = bv.block_table + (size_t)b * bv.max_pages;
  const int slot0 = split * p.rows_per_split;
  const int nslots = max(0, min(p.topk - slot0, p.rows_per_split));
  const int32_t* idx = p.idx + (size_t)g * p.topk + slot0;
  const float* q = (const float*)p.q + (size_t)g * H * DQK;
  for (int e = tid; e < H * DQK; e += 256) s_q[e / DQK][e % DQK] = q[e] * p.scale_log2;
  if (tid < H) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
  constexpr int OPT = (H * DV + 255) / 256;
  float o[OPT];
#pragma unroll
  for (int i = 0; i < OPT; i++) o[i] = 0.f;
  __syncthreads();
  for (int t0 = 0; t0 < nslots; t0 += TR) {
    if (tid < TR) {
      const int slot = t0 + tid;
      const int pos = (slot < nslots) ? idx[slot] : -1;
      s_row[tid] = (pos >= 0) ? bt[pos / P] * P + (pos % P) : -1;
    }
    __syncthreads();
    for (int e = tid; e < TR * DQK; e += 256) {
      const int r = e / DQK, c = e % DQK;
      const int row = s_row[r];
      s_kv[r][c] = (row >= 0) ? ((const float*)p.kv)[(size_t)row * DQK + c] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < H * TR; e += 256) {
      const int h = e / TR, r = e % TR;
      float z = -INFINITY;
      if (s_row[r] >= 0) {
        z = 0.f;
        for (int c = 0; c < DQK; c++) z = fmaf(s_q[h][c], s_kv[r][c], z);
      }
      s_p[h][r] = z;
    }
    __syncthreads();
    if (tid < H) {
      const int h = tid;
      float mt = -INFINITY;
      for (int r = 0; r < TR; r++) mt = fmaxf(mt, s_p[h][r]);
      const float mn = fmaxf(s_m[h], mt);
      const bool none = (mn == -INFINITY);
      const float al = none ? 1.f : exp2f(s_m[h] - mn);
      float ls = 0.f;
      for (int r = 0; r < TR; r++) {
        const float pv = none ? 0.f : exp2f(s_p[h][r] - mn);
        s_p[h][r] = pv;
        ls += pv;
      }
      s_l[h] = s_l[h] * al + ls;
      s_m[h] = mn;
      s_alpha[h] = al;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < OPT; i++) {
      const int e = tid + 256 * i;
      if (e < H * DV) {
        const int h = e / DV, v = e % DV;
        float acc = o[i] * s_alpha[h];
        for (int r = 0; r < TR; r++) acc = fmaf(s_p[h][r], s_kv[r][v], acc);
        o[i] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < OPT; i++) {
    const int e = tid + 256 * i;
    if (e < H * DV) {
      const int h = e / DV, v = e % DV;
      const float l = s_l[h];
      const float val = (l > 0.f) ? o[i] / l : 0.f;
      if (p.splits == 1) ((float*)p.out)[(size_t)g * H * DV + e] = val;
      else p.part_o[(((size_t)g * p.splits + split) * H + h) * DV + v] = val;
    }
  }
  if (tid < H) {
    const float l = s_l[tid];
    const float lse2 = (l > 0.f) ? s_m[tid] + log2f(l) : -INFINITY;
    if (p.splits == 1) {
      if (p.lse) p.lse[(size_t)g * H + tid] = lse2 * 0.69314718055994531f;
    } else {
      p.part_ml[((size_t)g * p.splits + split) * H + tid] = lse2;
    }
  }
}

}  // namespace

hipError_t launch_sfa(int dtype, int H, int Dqk, int Dv, const SfaParams& p, hipStream_t st) {
  if (p.bv.total_q == 0) return hipSuccess;
  if (dtype == kBF16 && H == 128 && Dqk == 576 && Dv == 512) {
    auto kern = sfa_bf16_kernel<576, 512>;
    const size_t lds = 3 * 40 * 1024 + 8 * 2048 + (size_t)p.rows_per_split * 4;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int tok8 = (p.bv.total_q + 7) / 8 * 8;
    hipLaunchKernelGGL(kern, dim3(2 * tok8, 1, p.splits), dim3(kSfaBf16Threads), lds, st, p);
    return hipGetLastError();
  }
  if (dtype == kF32 && H == 8 && Dqk == 80 && Dv == 64) {
    hipLaunchKernelGGL((sfa_f32_kernel<8, 80, 64>), dim3(p.bv.total_q, 1, p.splits), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sfa_combine(int dtype, int H, int Dv, const SfaParams& p, hipStream_t st) {
  if (p.bv.total_q == 0 || p.splits <= 1) return hipSuccess;
  if (dtype == kBF16 && Dv == 512) {
    hipLaunchKernelGGL((sfa_combine_kernel<512, true>), dim3(p.bv.total_q, (H + 3) / 4), dim3(256), 0, st, p, H);
    return hipGetLastError();
  }
  if (dtype == kF32 && Dv == 64) {
    hipLaunchKernelGGL((sfa_combine_kernel<64, false>), dim3(p.bv.total_q, (H + 3) / 4), dim3(256), 0, st, p, H);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
