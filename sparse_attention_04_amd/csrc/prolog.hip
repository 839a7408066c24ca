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
//   prolog_gemm_kernel: out[t][c] = sum_k x[t][k] W[c][k] over d_model; eight
//     waves split d_model and their partial tiles are summed in LDS in a fixed
//     order (deterministic).  q columns are rounded to bf16, k and w stay
//     float32.  32x32x16 bf16 MFMAs: x rows on M (tokens, 64 per workgroup),
//     weight rows on N (32 columns per workgroup).  For decode (tens of tokens)
//     the launch is bound by the weight stream (d_model x 8384 bf16).
//   prolog_finish_kernel: quantise q; LayerNorm k in float32, round to bf16,
//     quantise, append at t = L_b - T_b + i through the block table.
#include "common.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kPgWaves = 8;
constexpr int kPgThreads = 64 * kPgWaves;
constexpr int kPgM = 64;            // tokens per workgroup (two 32-row M-tiles)
constexpr int kPgN = 32;            // weight rows (output columns) per workgroup
constexpr int kPgChunk = 8;         // K-steps of 16 loaded together
constexpr int kPgDmodelUnit = kPgWaves * 16 * kPgChunk;   // d_model granularity (1024)

__device__ __forceinline__ int find_seq_pg(const BatchView& bv, int tok) {
  int lo = 0, hi = bv.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bv.cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Column tile -> (matrix, first row of that matrix).  Matrices: 0 = W_q
// (H*D rows), 1 = W_k (D rows), 2 = W_w (H rows); all are multiples of 32.
__device__ __forceinline__ void tile_of(const PrologParams& p, int tile, int& mat, int& row0) {
  const int nq = p.H * p.D / kPgN, nk = p.D / kPgN;
  if (tile < nq) { mat = 0; row0 = tile * kPgN; }
  else if (tile < nq + nk) { mat = 1; row0 = (tile - nq) * kPgN; }
  else { mat = 2; row0 = (tile - nq - nk) * kPgN; }
}

// Eight waves split d_model; each streams its slice in chunks of 8 K-steps
// through two register buffers used alternately (unrolled by two, so the next
// chunk's loads stay in flight while the current chunk's MFMAs run, with no
// register copies that would wait for them).
__global__ __launch_bounds__(kPgThreads) void prolog_gemm_kernel(PrologParams p) {
  __shared__ __attribute__((aligned(16))) float part[4][2][16][64];   // [wave % 4][mt][i][lane]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mat, row0;
  tile_of(p, blockIdx.x, mat, row0);
  const uint16_t* W = (const uint16_t*)(mat == 0 ? p.w_q : mat == 1 ? p.w_k : p.w_w);
  const int m0 = blockIdx.y * kPgM;
  const int dm = p.d_model;
  const int kw = dm / kPgWaves;                       // this wave's slice of d_model
  const int kbeg = wave * kw;
  // lane l: A rows (tokens) m0 + 32 mt + l%32, B row (column) row0 + l%32;
  // K elements 8 (l/32) .. +7 of each 16-wide step
  const int t0 = min(m0 + (lane & 31), p.total_q - 1);
  const int t1 = min(m0 + 32 + (lane & 31), p.total_q - 1);
  const int koff = kbeg + 8 * (lane >> 5);
  const u32x4* xa0 = (const u32x4*)((const uint16_t*)p.x + (size_t)t0 * dm + koff);
  const u32x4* xa1 = (const u32x4*)((const uint16_t*)p.x + (size_t)t1 * dm + koff);
  const u32x4* wb = (const u32x4*)(W + (size_t)(row0 + (lane & 31)) * dm + koff);
  f32x16 acc0, acc1;
#pragma unroll
  for (int i = 0; i < 16; i++) { acc0[i] = 0.f; acc1[i] = 0.f; }
  struct Buf { u32x4 a0[kPgChunk], a1[kPgChunk], b[kPgChunk]; };
  // a step is 16 elements = 2 u32x4 apart in each row
  auto load = [&](int c, Buf& f) {
#pragma unroll
    for (int s = 0; s < kPgChunk; s++) {
      const int st = c * kPgChunk + s;
      f.a0[s] = xa0[2 * st];
      f.a1[s] = xa1[2 * st];
      f.b[s] = wb[2 * st];
    }
  };
  auto mma = [&](const Buf& f) {
#pragma unroll
    for (int s = 0; s < kPgChunk; s++) {
      const bf16x8 bv = __builtin_bit_cast(bf16x8, f.b[s]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a0[s]), bv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.a1[s]), bv, acc1, 0, 0, 0);
    }
  };
  const int nchunks = kw / (16 * kPgChunk);
  Buf f0, f1;
  load(0, f0);
  if (nchunks > 1) load(1, f1);
  for (int c = 0; c < nchunks; c += 2) {
    mma(f0);
    if (c + 2 < nchunks) load(c + 2, f0);
    if (c + 1 < nchunks) {
      mma(f1);
      if (c + 3 < nchunks) load(c + 3, f1);
    }
  }
  // sum the eight waves' tiles in a fixed order: waves 4..7 into 0..3, then
  // the four
  if (wave >= 4) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      part[wave - 4][0][i][lane] = acc0[i];
      part[wave - 4][1][i][lane] = acc1[i];
    }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      acc0[i] += part[wave][0][i][lane];
      acc1[i] += part[wave][1][i][lane];
    }
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      part[wave][0][i][lane] = acc0[i];
      part[wave][1][i][lane] = acc1[i];
    }
  }
  __syncthreads();
  // thread t: token m0 + t/8, columns 4 (t%8) .. +3 of the tile.  C layout of
  // a 32x32 tile: lane l holds column l%32 and rows 8 (i/4) + 4 (l/32) + i%4.
  const int tl = tid >> 3, cg = tid & 7;
  const int tok = m0 + tl;
  if (tok >= p.total_q) return;
  const int mt = tl >> 5, r = tl & 31;
  const int ii = (r >> 3) * 4 + (r & 3), lh = (r >> 2) & 1;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int ln = lh * 32 + 4 * cg + j;
    v[j] = ((part[0][mt][ii][ln] + part[1][mt][ii][ln]) + part[2][mt][ii][ln]) + part[3][mt][ii][ln];
  }
  const int col = row0 + 4 * cg;
  if (mat == 0) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *(uint2*)((uint16_t*)p.q_bf16 + (size_t)tok * p.H * p.D + col) = pk;
  } else {
    float* dst = (mat == 1) ? p.k_f32 + (size_t)tok * p.D + col : p.w_out + (size_t)tok * p.H + col;
    *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
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
  // ---- k: LayerNorm over D (workgroup 0's wave 0), bf16, quantise, append
  if (wave != 0 || blockIdx.y != 0) return;
  const float* kv = p.k_f32 + (size_t)tok * D;
  const float a0 = kv[2 * lane], a1 = kv[2 * lane + 1];
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

int prolog_n_tiles(int H, int D) { return (H * D + D + H) / kPgN; }
int prolog_d_model_unit() { return kPgDmodelUnit; }

hipError_t launch_prolog(int out_dtype, const PrologParams& p, hipStream_t st) {
  if (p.total_q == 0) return hipSuccess;
  if (p.D != 128 || (p.H % kPgN) != 0 || p.d_model <= 0 || (p.d_model % kPgDmodelUnit) != 0) return hipErrorInvalidValue;
  const dim3 g1(prolog_n_tiles(p.H, p.D), (p.total_q + kPgM - 1) / kPgM);
  hipLaunchKernelGGL(prolog_gemm_kernel, g1, dim3(kPgThreads), 0, st, p);
  hipError_t e = hipGetLastError();
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
