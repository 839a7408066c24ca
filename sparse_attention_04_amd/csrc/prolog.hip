// Indexer prolog: the steps before the fused indexer for the tokens of this
// step ("Three-Stream Coordination for Indexer Prolog", Day0 Inference
// Optimization on Ascend CANN, sec. 2; Adapting and Optimizing Inference for a
// New Model Architecture on Ascend, sec. 3.2 and 4.2; Inference Acceleration
// for Next-Gen Attention Architectures, sec. 3.3): Q projection, K projection
// and normalisation, head-weight projection, dynamic quantisation of the index
// Q and K (FP8 with one float32 scale per row, or MXFP8 with one e8m0 scale
// per 32 elements), and the append of the new keys to the paged K cache.
//
// The pages run the independent preparation operators on separate streams so
// that they overlap.  Here the three projections are one launch: its
// workgroups take 128-row tiles of W_q, W_k and W_w (8192 + 128 + 64 rows
// for the 64 x 128 indexer) and, for the few tokens of a decode step, one of
// up to four ranges of d_model each, so every projection streams its weights
// at the same time with no stream synchronisation.  A second launch, one
// workgroup per token and 16 heads, adds the ranges' partial sums, quantises
// q per (token, head) or per 32-group, normalises and quantises k and writes
// it into the cache.
//
//   prolog_gemm_kernel: out[t][c] = sum_k x[t][k] W[c][k] over a range of
//     d_model, the weights staged through LDS (see the kernel), as float32
//     partial sums (or, for launches with one range, q rounded to bf16).  For
//     decode (tens of tokens) the launch is bound by the weight stream
//     (d_model x 8384 bf16).
//   prolog_finish_kernel: add up the partials; round q to bf16 and quantise
//     it; LayerNorm k in float32, round to bf16, quantise, append at
//     t = L_b - T_b + i through the block table.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kPgThreads = 256;    // 4 waves
constexpr int kPgM = 64;            // tokens per workgroup (each wave: 16)
constexpr int kPgN = 144;           // weight rows (output columns) per tile
constexpr int kPgKC = 128;          // d_model elements per staged chunk
constexpr int kPgRowB = kPgKC * 2;  // bytes of one row's chunk (256)
constexpr int kPgRows = kPgN + kPgM;                    // weight rows, then token rows
constexpr int kPgChunkB = kPgRows * kPgRowB;            // 52 KiB per chunk
constexpr int kPgLoads = kPgChunkB / 1024;              // 1-KiB loads per chunk (52)
constexpr int kPgLPW = kPgLoads / 4;                    // per wave (13)
constexpr int kPgNBuf = 3;                              // chunks in the LDS ring
constexpr int kPgNT = kPgN / 16;                        // 16-column N-tiles per wave (9)
constexpr int kPgDmodelUnit = kPgKC;
constexpr int kPgMaxSplit = 4;                          // d_model ranges of a decode-sized launch
static_assert(kPgMaxSplit == 4, "the finish kernel reads two k parts and one w part per thread");
static_assert(kPgLoads % 4 == 0 && kPgRowB * 4 == 1024, "four rows per 1-KiB load");

__device__ __forceinline__ int find_seq_pg(const BatchView& bv, int tok) {
  int lo = 0, hi = bv.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bv.cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
#define DSA_PG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Row r of the concatenated weights [W_q | W_k | W_w] (H*D + D + H rows; r
// is also the output column): its source row.
__device__ __forceinline__ const uint16_t* weight_row(const PrologParams& p, int r) {
  const int hd = p.H * p.D;
  if (r < hd) return (const uint16_t*)p.w_q + (size_t)r * p.d_model;
  if (r < hd + p.D) return (const uint16_t*)p.w_k + (size_t)(r - hd) * p.d_model;
  return (const uint16_t*)p.w_w + (size_t)(r - hd - p.D) * p.d_model;
}

// out[t][c] = sum_k x[t][k] W[c][k].  A workgroup computes 64 tokens x 144
// rows of the concatenated weights over one range of d_model; wave w owns
// tokens 16w .. 16w + 15 with 16x16x32 bf16 MFMAs (nine 16-column N-tiles),
// so no partial sums cross waves.  Its d_model range streams in chunks of 128
// elements through a 3-deep LDS ring: 52 one-KiB direct global->LDS loads per
// chunk (four rows each, fully coalesced), rows of 256 bytes whose 16-byte
// pieces are XOR-swizzled by row (piece c of row r sits in slot c ^ (r % 16)),
// so the operand reads of 16 rows hit 16 distinct bank groups.  With 8384 rows
// (the 64 x 128 indexer) and four ranges the grid is 59 x 4 = 236 workgroups:
// one round on 256 compute units.
//
// A decode-sized launch (one block of at most 64 tokens, grid z = p.n_parts
// ranges of d_model) writes float32 partial sums of every output column to
// part[range][token][column of q | k | w]; the finish kernel adds them in
// range order and rounds q to bf16.  Larger launches (one range) round q to
// bf16 here and write the k and w columns to part[0].  Splitting d_model
// gives the weight stream enough workgroups with 144 rows each: a compute
// unit then has 72 KiB of weights in flight, and re-reads a quarter as many
// token rows as with one range.
__global__ __launch_bounds__(kPgThreads, 1) void prolog_gemm_kernel(PrologParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char pg_smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * kPgM;
  const int dm = p.d_model;
  const int nch_all = dm / kPgKC;
  const int split = blockIdx.z, nsplit = gridDim.z;
  const int c_begin = (int)((int64_t)nch_all * split / nsplit), c_end = (int)((int64_t)nch_all * (split + 1) / nsplit);
  const int nch = c_end - c_begin;
  const int ncol = p.H * p.D + p.D + p.H;
  const int row0 = blockIdx.x * kPgN;
  const uint32_t ring = lds_addr(pg_smem);
  // load ins of a chunk fills rows 4 ins .. 4 ins + 3 (weight rows first,
  // then token rows; rows past the weights or past total_q repeat the last)
  const uint16_t* src_row[kPgLPW];
#pragma unroll
  for (int k = 0; k < kPgLPW; k++) {
    const int R = 4 * (wave + 4 * k) + (lane >> 4);
    src_row[k] = (R < kPgN) ? weight_row(p, min(row0 + R, ncol - 1))
                            : (const uint16_t*)p.x + (size_t)min(m0 + R - kPgN, p.total_q - 1) * dm;
  }
  auto issue = [&](int j) {
    const int c = c_begin + j;
    const uint32_t buf = ring + (uint32_t)(j % kPgNBuf) * kPgChunkB;
#pragma unroll
    for (int k = 0; k < kPgLPW; k++) {
      const int ins = wave + 4 * k;
      const int R = 4 * ins + (lane >> 4);
      const int piece = (lane & 15) ^ (R & 15);
      dma16(src_row[k] + c * kPgKC + piece * 8, __builtin_amdgcn_readfirstlane(buf + ins * 1024u));
    }
  };
  issue(0);
  if (nch > 1) issue(1);

  const int g16 = lane >> 4, l16 = lane & 15;
  f32x4 acc[kPgNT];
#pragma unroll
  for (int n = 0; n < kPgNT; n++) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nch; j++) {
    if (j + 1 < nch) DSA_PG_WAIT_VMCNT(kPgLPW); else DSA_PG_WAIT_VMCNT(0);
    // every wave's loads of chunk j have landed, and every wave is done with
    // the buffer of chunk j - 1, which chunk j + 2 refills
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 2 < nch) issue(j + 2);
    const unsigned char* buf = pg_smem + (size_t)(j % kPgNBuf) * kPgChunkB;
    // A: token row kPgN + 16 wave + l16; B: weight rows 16 n + l16;
    // K-step ks takes pieces 4 ks + g16 (8 elements each)
    const int ra = kPgN + 16 * wave + l16;
#pragma unroll
    for (int ks = 0; ks < kPgKC / 32; ks++) {
      const int pc = 4 * ks + g16;
      const bf16x8 a = *(const bf16x8*)(buf + ra * kPgRowB + ((pc ^ (ra & 15)) * 16));
#pragma unroll
      for (int n = 0; n < kPgNT; n++) {
        const int rb = 16 * n + l16;
        const bf16x8 bv = *(const bf16x8*)(buf + rb * kPgRowB + ((pc ^ (rb & 15)) * 16));
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[n], 0, 0, 0);
      }
    }
  }
  // C layout of a 16x16 tile: lane l holds column l % 16 and rows
  // 4 (l / 16) + i.  Tokens past total_q and rows past the weights are not
  // written.
#pragma unroll
  for (int n = 0; n < kPgNT; n++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int tok = m0 + 16 * wave + 4 * g16 + i;
      const int r = row0 + 16 * n + l16;
      if (tok >= p.total_q || r >= ncol) continue;
      if (nsplit > 1) {
        p.part[((size_t)split * p.total_q + tok) * ncol + r] = acc[n][i];
      } else if (r < p.H * p.D) {
        ((uint16_t*)p.q_bf16)[(size_t)tok * p.H * p.D + r] = f32_to_bf16(acc[n][i]);
      } else {
        p.part[(size_t)tok * (p.D + p.H) + (r - p.H * p.D)] = acc[n][i];
      }
    }
}

// float -> e4m3fn byte, round to nearest even, saturated to +-448 first.
__device__ __forceinline__ uint32_t e4m3_byte(float y) {
  y = fminf(fmaxf(y, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}

// MX exponent of a group maximum: floor(log2 amax) - 8 clamped to
// [-127, 127] (amax = 0 or below 2^-126: -127).
__device__ __forceinline__ int mx_exponent(float amax) {
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return ex == 0 ? -127 : max(ex - 127 - 8, -127);
}

constexpr int kFinThreads = 256;   // 4 waves; 4 workgroups per token, 16 heads each

template <int OUT>
__global__ __launch_bounds__(kFinThreads) void prolog_finish_kernel(PrologParams p) {
  const int tok = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = p.H, D = p.D;          // D == 128: two elements per lane
  // The key's cache row (wave 0 of workgroup 0 of the token), found first so
  // that its chain of loads overlaps the sums below: the token's sequence from
  // one wave-wide load of cu_q (a binary search for batches above 65), then
  // its length and offsets, then the block-table entry.
  const BatchView& bv = p.bv;
  int64_t krow = 0;
  if (blockIdx.y == 0 && wave == 0) {
    int b;
    if (bv.batch <= 65) {
      const int cq = (1 + lane < bv.batch) ? bv.cu_q[1 + lane] : 0x7FFFFFFF;
      b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(cq <= tok)));
    } else {
      b = find_seq_pg(bv, tok);
    }
    const int c0 = bv.cu_q[b], c1 = bv.cu_q[b + 1], L = bv.seq_lens[b];
    const int t = L - (c1 - c0) + (tok - c0);
    krow = ((int64_t)bv.block_table[(size_t)b * bv.max_pages + (t >> bv.page_shift)] << bv.page_shift) +
           (t & (bv.page_size - 1));
  }
  const int S = p.n_parts;                   // d_model ranges of the GEMM
  const int ncol = H * D + D + H;
  // The k and w partials of workgroup 0 of the token, loaded now for use
  // after q.  part[range][token][column]: all columns of [q | k | w] with
  // several ranges, the k and w columns only with one.  Thread t takes parts
  // c = t / 128 and c + 2 of k column t % 128, and part c = t / 64 of w column
  // t % 64 (S <= kPgMaxSplit = 4).
  const int KW = (S > 1) ? ncol : D + H;
  const float* pk = p.part + (size_t)tok * KW + ((S > 1) ? H * D : 0);
  const size_t pstride = (size_t)p.total_q * KW;
  const int kc = tid & 127, kh = tid >> 7, wc = tid & 63, wh = tid >> 6;
  float k0 = 0.f, k1 = 0.f, w0 = 0.f;
  if (blockIdx.y == 0) {
    k0 = (kh < S) ? pk[kh * pstride + kc] : 0.f;
    k1 = (kh + 2 < S) ? pk[(kh + 2) * pstride + kc] : 0.f;
    w0 = (H <= 64 && wh < S && wc < H) ? pk[wh * pstride + D + wc] : 0.f;
  }
  // ---- q: workgroup y quantises heads 16y .. 16y + 15, four per wave (all
  // four loaded before any is used).  With several ranges, q is the sum of
  // their float32 partials in range order, rounded to bf16 here.
  if (OUT != kBF16 || S > 1) {
    const uint16_t* q = (const uint16_t*)p.q_bf16 + (size_t)tok * H * D;
    const int hb = 16 * blockIdx.y + 4 * wave;
    uint32_t two[4];
    if (S > 1) {
      // every range's partials of the four heads are loaded before any is
      // added (S <= kPgMaxSplit)
      float2 v[kPgMaxSplit][4];
#pragma unroll
      for (int sp = 0; sp < kPgMaxSplit; sp++) {
        const float* ps = p.part + ((size_t)sp * p.total_q + tok) * ncol;
#pragma unroll
        for (int u = 0; u < 4; u++)
          v[sp][u] = (sp < S && hb + u < H) ? *(const float2*)(ps + (size_t)(hb + u) * D + 2 * lane) : float2{0.f, 0.f};
      }
      float2 sum[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        sum[u] = v[0][u];
#pragma unroll
        for (int sp = 1; sp < kPgMaxSplit; sp++) {
          sum[u].x += v[sp][u].x;
          sum[u].y += v[sp][u].y;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        two[u] = (uint32_t)f32_to_bf16(sum[u].x) | ((uint32_t)f32_to_bf16(sum[u].y) << 16);
        if (hb + u < H && (OUT == kBF16 || p.q_bf16 != p.q_out))
          *(uint32_t*)((uint16_t*)p.q_bf16 + (size_t)tok * H * D + (size_t)(hb + u) * D + 2 * lane) = two[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; u++) two[u] = (hb + u < H) ? *(const uint32_t*)(q + (size_t)(hb + u) * D + 2 * lane) : 0u;
    }
    if (OUT != kBF16) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int h = hb + u;
      if (h >= H) break;
      const float a = bf16_to_f32((uint16_t)(two[u] & 0xFFFFu)), b = bf16_to_f32((uint16_t)(two[u] >> 16));
      float m = fmaxf(fabsf(a), fabsf(b));
      uint32_t bytes;
      if (OUT == kFP8) {
        m = wave_max(m);
        const float s = (m > 0.f) ? m / 448.f : 1.f;
        bytes = e4m3_byte(a / s) | (e4m3_byte(b / s) << 8);
        if (lane == 0) ((float*)p.q_scale_out)[(size_t)tok * H + h] = s;
      } else {
        // group g = lane / 16 holds elements 32 g .. 32 g + 31
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const int E = mx_exponent(m);
        bytes = e4m3_byte(ldexpf(a, -E)) | (e4m3_byte(ldexpf(b, -E)) << 8);
        if ((lane & 15) == 0) ((uint8_t*)p.q_scale_out)[((size_t)tok * H + h) * (D / 32) + (lane >> 4)] = (uint8_t)(E + 127);
      }
      *(uint16_t*)((uint8_t*)p.q_out + ((size_t)tok * H + h) * D + 2 * lane) = (uint16_t)bytes;
    }
    }
  }
  if (blockIdx.y != 0) return;
  // ---- k and w: the sums of their partials (loaded at the start); the
  // sub-sums meet in LDS in a fixed order
  __shared__ float s_k[2][128], s_w[4][64];
  s_k[kh][kc] = k0 + k1;
  if (H <= 64) s_w[wh][wc] = w0;
  __syncthreads();
  if (H <= 64) {
    if (tid < H) p.w_out[(size_t)tok * H + tid] = (s_w[0][tid] + s_w[1][tid]) + (s_w[2][tid] + s_w[3][tid]);
  } else if (wave == 1) {
    for (int h = lane; h < H; h += 64) {
      float acc = 0.f;
      for (int c = 0; c < S; c++) acc += pk[c * pstride + D + h];
      p.w_out[(size_t)tok * H + h] = acc;
    }
  }
  if (wave != 0) return;
  // ---- k: LayerNorm over D (wave 0), bf16, quantise, append
  const float a0 = s_k[0][2 * lane] + s_k[1][2 * lane];
  const float a1 = s_k[0][2 * lane + 1] + s_k[1][2 * lane + 1];
  const float mean = wave_sum(a0 + a1) / (float)D;
  const float d0 = a0 - mean, d1 = a1 - mean;
  const float var = wave_sum(d0 * d0 + d1 * d1) / (float)D;
  const float inv = 1.f / sqrtf(var + p.ln_eps);
  const uint16_t k0 = f32_to_bf16(d0 * inv * p.ln_gamma[2 * lane] + p.ln_beta[2 * lane]);
  const uint16_t k1 = f32_to_bf16(d1 * inv * p.ln_gamma[2 * lane + 1] + p.ln_beta[2 * lane + 1]);
  if (p.k_bf16_out) *(uint32_t*)((uint16_t*)p.k_bf16_out + (size_t)tok * D + 2 * lane) = (uint32_t)k0 | ((uint32_t)k1 << 16);
  // cache row of this token: t = L_b - T_b + i (found above)
  const int64_t row = krow;
  if (OUT == kBF16) {
    *(uint32_t*)((uint16_t*)p.k_data + row * D + 2 * lane) = (uint32_t)k0 | ((uint32_t)k1 << 16);
    return;
  }
  const float b0 = bf16_to_f32(k0), b1 = bf16_to_f32(k1);
  float m = fmaxf(fabsf(b0), fabsf(b1));
  uint32_t bytes;
  if (OUT == kFP8) {
    m = wave_max(m);
    const float s = (m > 0.f) ? m / 448.f : 1.f;
    bytes = e4m3_byte(b0 / s) | (e4m3_byte(b1 / s) << 8);
    if (lane == 0) ((float*)p.k_scale)[row] = s;
  } else {
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int E = mx_exponent(m);
    bytes = e4m3_byte(ldexpf(b0, -E)) | (e4m3_byte(ldexpf(b1, -E)) << 8);
    if ((lane & 15) == 0) ((uint8_t*)p.k_scale)[row * (D / 32) + (lane >> 4)] = (uint8_t)(E + 127);
  }
  *(uint16_t*)((uint8_t*)p.k_data + row * D + 2 * lane) = (uint16_t)bytes;
}

}  // namespace

int prolog_d_model_unit() { return kPgDmodelUnit; }

// Ranges of d_model a launch splits the GEMM into (the partial-sum slots it
// needs): a decode-sized launch (one block of tokens) takes up to four ranges
// of at least two chunks each; larger launches one.
int prolog_n_parts(int total_q, int d_model) {
  if (total_q > kPgM) return 1;
  return std::max(1, std::min(kPgMaxSplit, d_model / kPgKC / 2));
}

// float32 words of the partial-sum workspace.
size_t prolog_part_words(int total_q, int d_model, int H, int D) {
  const int S = prolog_n_parts(total_q, d_model);
  return (size_t)S * total_q * ((S > 1) ? (size_t)H * D + D + H : (size_t)D + H);
}

hipError_t launch_prolog(int out_dtype, const PrologParams& p0, hipStream_t st) {
  if (p0.total_q == 0) return hipSuccess;
  if (p0.D != 128 || (p0.H % 32) != 0 || p0.d_model <= 0 || (p0.d_model % kPgDmodelUnit) != 0)
    return hipErrorInvalidValue;
  PrologParams p = p0;
  const int mblocks = (p.total_q + kPgM - 1) / kPgM;
  p.n_parts = prolog_n_parts(p.total_q, p.d_model);
  const int ntiles = (p.H * p.D + p.D + p.H + kPgN - 1) / kPgN;
  const size_t lds = (size_t)kPgNBuf * kPgChunkB;
  hipError_t e = hipFuncSetAttribute((const void*)prolog_gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prolog_gemm_kernel, dim3(ntiles, mblocks, p.n_parts), dim3(kPgThreads), lds, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(p.total_q, (p.H + 15) / 16);
  if (out_dtype == kBF16)
    hipLaunchKernelGGL(prolog_finish_kernel<kBF16>, g2, dim3(kFinThreads), 0, st, p);
  else if (out_dtype == kFP8)
    hipLaunchKernelGGL(prolog_finish_kernel<kFP8>, g2, dim3(kFinThreads), 0, st, p);
  else
    hipLaunchKernelGGL(prolog_finish_kernel<kMX>, g2, dim3(kFinThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
