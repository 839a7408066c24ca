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
// workgroups take 32-column tiles of [W_q | W_k | W_w] (8192 + 128 + 64
// columns for the 64 x 128 indexer), so every projection streams its weights
// at the same time with no stream synchronisation.  A second launch, one
// workgroup per token, quantises q per (token, head) or per 32-group,
// normalises and quantises k and writes it into the cache.
//
//   prolog_gemm_kernel: out[t][c] = sum_k x[t][k] W[c][k] over d_model, the
//     weights staged through LDS (see the kernel); q columns are rounded to
//     bf16, k and w stay float32.  For decode (tens of tokens) the launch is
//     bound by the weight stream (d_model x 8384 bf16).
//   prolog_finish_kernel: quantise q; add up the k and w partials; LayerNorm k
//     in float32, round to bf16, quantise, append at t = L_b - T_b + i through
//     the block table.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kPgThreads = 256;    // 4 waves
constexpr int kPgM = 64;            // tokens per workgroup (each wave: 16)
constexpr int kPgN = 32;            // weight rows (output columns) per tile
constexpr int kPgKC = 256;          // d_model elements per staged chunk
constexpr int kPgRowB = kPgKC * 2;  // bytes of one row's chunk (512)
constexpr int kPgRows = kPgN + kPgM;                    // weight rows, then token rows
constexpr int kPgChunkB = kPgRows * kPgRowB;            // 48 KiB per chunk
constexpr int kPgLoads = kPgChunkB / 1024;              // 1-KiB loads per chunk (48)
constexpr int kPgLPW = kPgLoads / 4;                    // per wave (12)
constexpr int kPgNBuf = 3;                              // chunks in the LDS ring
constexpr int kPgDmodelUnit = kPgKC;
static_assert(kPgLoads % 4 == 0 && kPgRowB * 2 == 1024, "two rows per 1-KiB load");

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

// Tile t of the concatenated weight rows [W_q | W_k | W_w] (all multiples of
// 32 rows): its matrix (0 q, 1 k, 2 w) and first row in that matrix.
__device__ __forceinline__ void tile_of(const PrologParams& p, int tile, int& mat, int& row0) {
  const int nq = p.H * p.D / kPgN, nk = p.D / kPgN;
  if (tile < nq) { mat = 0; row0 = tile * kPgN; }
  else if (tile < nq + nk) { mat = 1; row0 = (tile - nq) * kPgN; }
  else { mat = 2; row0 = (tile - nq - nk) * kPgN; }
}

// out[t][c] = sum_k x[t][k] W[c][k].  A workgroup computes 64 tokens x 32
// weight rows; wave w owns tokens 16w .. 16w + 15 with 16x16x32 bf16 MFMAs
// (two 16-column N-tiles), so no partial sums cross waves.  d_model streams in
// chunks of 256 elements through a 3-deep LDS ring: 48 one-KiB direct
// global->LDS loads per chunk (two rows each, fully coalesced), rows of 512
// bytes whose 16-byte pieces are XOR-swizzled by row (piece c of row r sits in
// slot c ^ (r % 32)), so the operand reads of 16 rows hit 16 distinct bank
// groups.
//
// Jobs: the workgroup's main tile over every chunk, then (decode launches, a
// single token block) its share of slices: the K and head-weight tiles split
// by chunk over the workgroups, so the grid is exactly the q tiles and one
// round of workgroups covers it.  Their partial sums go to part[chunk] and the
// finish kernel adds them in chunk order.  Launches with several token blocks
// (many workgroups anyway) give every tile, K and head-weight ones included,
// a workgroup of its own (part[0]).
__global__ __launch_bounds__(kPgThreads, 1) void prolog_gemm_kernel(PrologParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char pg_smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * kPgM;
  const int dm = p.d_model;
  const int nch = dm / kPgKC;
  const int nq_tiles = p.H * p.D / kPgN, nx_tiles = (p.D + p.H) / kPgN;
  const bool split = p.split_extra != 0;
  const int nmain = nch;
  int nextra = 0;
  if (split)
    for (int e = blockIdx.x; e < nx_tiles * nch; e += nq_tiles) nextra++;
  const int njobs = nmain + nextra;
  int main_mat, main_row0;
  tile_of(p, blockIdx.x, main_mat, main_row0);

  // job -> (weight matrix, first row, chunk)
  auto job = [&](int j, int& mat, int& row0, int& c) {
    if (j < nmain) {
      mat = main_mat; row0 = main_row0; c = j;
    } else {
      const int e = blockIdx.x + (j - nmain) * nq_tiles;
      tile_of(p, nq_tiles + e / nch, mat, row0);
      c = e % nch;
    }
  };
  const uint32_t ring = lds_addr(pg_smem);
  auto issue = [&](int j) {
    int mat, row0, c;
    job(j, mat, row0, c);
    const uint16_t* W = (const uint16_t*)(mat == 0 ? p.w_q : mat == 1 ? p.w_k : p.w_w);
    const uint32_t buf = ring + (uint32_t)(j % kPgNBuf) * kPgChunkB;
#pragma unroll
    for (int k = 0; k < kPgLPW; k++) {
      const int ins = wave + 4 * k;
      const int R = 2 * ins + (lane >> 5);
      const int piece = (lane & 31) ^ (R & 31);
      const uint16_t* src = (R < kPgN)
          ? W + (size_t)(row0 + R) * dm
          : (const uint16_t*)p.x + (size_t)min(m0 + R - kPgN, p.total_q - 1) * dm;
      dma16(src + c * kPgKC + piece * 8, __builtin_amdgcn_readfirstlane(buf + ins * 1024u));
    }
  };
  issue(0);
  if (njobs > 1) issue(1);

  const int g16 = lane >> 4, l16 = lane & 15;
  f32x4 acc[2], acce[2];
#pragma unroll
  for (int n = 0; n < 2; n++) {
    acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    acce[n] = acc[n];
  }
  for (int j = 0; j < njobs; j++) {
    if (j + 1 < njobs) DSA_PG_WAIT_VMCNT(kPgLPW); else DSA_PG_WAIT_VMCNT(0);
    // every wave's loads of job j have landed, and every wave is done with the
    // buffer of job j - 1, which job j + 2 refills
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (j + 2 < njobs) issue(j + 2);
    const unsigned char* buf = pg_smem + (size_t)(j % kPgNBuf) * kPgChunkB;
    const bool is_main = j < nmain;
    if (!is_main) {
#pragma unroll
      for (int n = 0; n < 2; n++) acce[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // A: token row kPgN + 16 wave + l16; B: weight rows l16 and 16 + l16;
    // K-step ks takes pieces 4 ks + g16 (8 elements each)
    const int ra = kPgN + 16 * wave + l16;
#pragma unroll
    for (int ks = 0; ks < kPgKC / 32; ks++) {
      const int pc = 4 * ks + g16;
      const bf16x8 a = *(const bf16x8*)(buf + ra * kPgRowB + ((pc ^ (ra & 31)) * 16));
      const bf16x8 b0 = *(const bf16x8*)(buf + l16 * kPgRowB + ((pc ^ l16) * 16));
      const bf16x8 b1 = *(const bf16x8*)(buf + (16 + l16) * kPgRowB + ((pc ^ (16 + l16)) * 16));
      if (is_main) {
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[1], 0, 0, 0);
      } else {
        acce[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acce[0], 0, 0, 0);
        acce[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acce[1], 0, 0, 0);
      }
    }
    // C layout of a 16x16 tile: lane l holds column l % 16 and rows
    // 4 (l / 16) + i.  Tokens past total_q are not written.
    const bool last_main = (j == nmain - 1);
    if (!last_main && is_main) continue;
    int mat, row0, c;
    job(j, mat, row0, c);
    f32x4 v[2];
#pragma unroll
    for (int n = 0; n < 2; n++) v[n] = is_main ? acc[n] : acce[n];
#pragma unroll
    for (int n = 0; n < 2; n++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int tok = m0 + 16 * wave + 4 * g16 + i;
        if (tok >= p.total_q) continue;
        const int col = row0 + 16 * n + l16;
        if (mat == 0) {
          ((uint16_t*)p.q_bf16)[(size_t)tok * p.H * p.D + col] = f32_to_bf16(v[n][i]);
        } else {
          const int kc = (mat == 1) ? col : p.D + col;     // column of [k | w]
          const int part = is_main ? 0 : c;
          p.kw_part[((size_t)part * p.total_q + tok) * (p.D + p.H) + kc] = v[n][i];
        }
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
  // ---- q: workgroup y quantises heads 16y .. 16y + 15, four per wave (all
  // four loaded before any is used)
  if (OUT != kBF16) {
    const uint16_t* q = (const uint16_t*)p.q_bf16 + (size_t)tok * H * D;
    const int hb = 16 * blockIdx.y + 4 * wave;
    uint32_t two[4];
#pragma unroll
    for (int u = 0; u < 4; u++) two[u] = (hb + u < H) ? *(const uint32_t*)(q + (size_t)(hb + u) * D + 2 * lane) : 0u;
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
  if (blockIdx.y != 0) return;
  // ---- k and w: the sums of their partials.  Thread t adds parts
  // c = t / 128 (mod 2) of k column t % 128, and parts c = t / 64 (mod 4) of w
  // column t % 64 (loads unrolled); the sub-sums then meet in LDS in a fixed
  // order.
  __shared__ float s_k[2][128], s_w[4][64];
  const int KW = D + H;
  const float* pk = p.kw_part + (size_t)tok * KW;
  const size_t pstride = (size_t)p.total_q * KW;
  {
    const int kc = tid & 127, kh = tid >> 7;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int c = kh, u = 0;
#pragma unroll 4
    for (; c < p.n_parts; c += 2, u = (u + 1) & 3) acc[u] += pk[c * pstride + kc];
    s_k[kh][kc] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    if (H <= 64) {
      const int wc = tid & 63, wh = tid >> 6;
      float aw[4] = {0.f, 0.f, 0.f, 0.f};
      int cw = wh, uw = 0;
      const bool has = wc < H;
#pragma unroll 4
      for (; cw < p.n_parts; cw += 4, uw = (uw + 1) & 3) aw[uw] += has ? pk[cw * pstride + D + wc] : 0.f;
      s_w[wh][wc] = (aw[0] + aw[1]) + (aw[2] + aw[3]);
    }
  }
  __syncthreads();
  if (H <= 64) {
    if (tid < H) p.w_out[(size_t)tok * H + tid] = (s_w[0][tid] + s_w[1][tid]) + (s_w[2][tid] + s_w[3][tid]);
  } else if (wave == 1) {
    for (int h = lane; h < H; h += 64) {
      float acc = 0.f;
      for (int c = 0; c < p.n_parts; c++) acc += pk[c * pstride + D + h];
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
  // cache row of this token: t = L_b - T_b + i
  const BatchView& bv = p.bv;
  const int b = find_seq_pg(bv, tok);
  const int i = tok - bv.cu_q[b];
  const int t = bv.seq_lens[b] - (bv.cu_q[b + 1] - bv.cu_q[b]) + i;
  const int64_t row = ((int64_t)bv.block_table[(size_t)b * bv.max_pages + (t >> bv.page_shift)] << bv.page_shift) +
                      (t & (bv.page_size - 1));
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

// Partial-sum slots of the K / head-weight columns a launch needs.
int prolog_n_parts(int total_q, int d_model) {
  return (total_q <= kPgM) ? d_model / kPgKC : 1;
}

hipError_t launch_prolog(int out_dtype, const PrologParams& p0, hipStream_t st) {
  if (p0.total_q == 0) return hipSuccess;
  if (p0.D != 128 || (p0.H % kPgN) != 0 || p0.d_model <= 0 || (p0.d_model % kPgDmodelUnit) != 0)
    return hipErrorInvalidValue;
  PrologParams p = p0;
  const int mblocks = (p.total_q + kPgM - 1) / kPgM;
  p.split_extra = (mblocks == 1) ? 1 : 0;
  p.n_parts = prolog_n_parts(p.total_q, p.d_model);
  const int ntiles = p.H * p.D / kPgN + (p.split_extra ? 0 : (p.D + p.H) / kPgN);
  const size_t lds = (size_t)kPgNBuf * kPgChunkB;
  hipError_t e = hipFuncSetAttribute((const void*)prolog_gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prolog_gemm_kernel, dim3(ntiles, mblocks), dim3(kPgThreads), lds, st, p);
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
