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
// all of its heads (half of them over an FP8 cache) and a contiguous range of
// index slots.  Per tile of 32 slots it gathers the 32 latent rows through the
// block table into LDS (a 4-deep ring), then every wave (16 heads: 8 waves
// over bf16 rows, 4 over FP8 rows) computes
//   S^T[row, head] = KV[row, :] . q[head, :]     (16x16x32 bf16 MFMAs, rows on M)
// so that after the softmax weights are formed the probabilities already sit in the
// B-operand layout of the second product
//   O^T[v, head] += V^T[v, row] P^T[row, head]   (V^T read with ds_read_b64_tr_b16).
// Slots holding -1 are masked.  With several slot ranges per token, each range
// writes a normalised partial and its log-sum-exp, merged by sfa_combine.
//
// FP8 KV cache (e4m3 bytes, one fp32 scale per token and tile of 128 elements
// of the latent row: Adapting and Optimizing Inference for a New Model
// Architecture on Ascend, sec. 4.3): the gather brings the 576-byte rows and
// their five scales into an LDS staging ring, and the workgroup converts each
// tile of rows once into the bf16 tile layout above.  The conversion is exact
// (every e4m3 value is a bf16 value) and leaves the scales out; they enter in
// fp32: S^T is accumulated per 128-column tile and each partial is multiplied
// by its rows' scales before it is summed, and the softmax weights are
// multiplied by the scale of each 128-column V tile before they are rounded
// into the PV product's operand (the denominator then sums the fp32 weights,
// as no single rounded set serves all four V tiles).
#include "common.h"
#include "kernels.h"
#include "sfa_body.h"

namespace dsa {

namespace {

// Workgroup L runs on XCD L % 8 (round-robin dispatch); each XCD takes a
// contiguous run of tokens, and all slot ranges of a token share one XCD.
template <int DQK, int DV, bool LO, int HG, bool KV8, int NWV = 4>
__global__ __launch_bounds__(64 * NWV, 1) void sfa_bf16_kernel(SfaParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sfa_smem[];
  const int chunk = gridDim.x / 8;
  const int g = (blockIdx.x & 7) * chunk + (blockIdx.x >> 3);
  if (g >= p.bv.total_q) return;
  sfa_bf16_body<DQK, DV, LO, HG, KV8, NWV>(p, g, blockIdx.y, blockIdx.z,
                                          blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0, sfa_smem);
}

// Merge the per-range partials of one token: weights 2^(lse_j - lse).  One
// workgroup per (token, group of 4 heads); each thread owns DV/64 columns.
// Partials are fp16 for the bf16 kernel (BF16OUT) and f32 otherwise.
template <int DV, bool BF16OUT>
__global__ __launch_bounds__(256) void sfa_combine_kernel(SfaParams p, int H) {
  constexpr int CPT = DV / 64;  // columns per thread
  const int g = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int c0 = (threadIdx.x & 63) * CPT;
  const int S = p.splits;
  // the fused decode's call counter moves on once its kernel is complete
  if (p.epoch_word && g == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.epoch_word = epoch_after(*p.epoch_word);
  if (h >= H) return;
  // Splits go in groups of 4 whose log-sum-exps and partials are all loaded
  // before any is used (one memory round trip per group); the running
  // maximum rescales what earlier groups accumulated.
  float mx = -INFINITY, den = 0.f;
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c++) acc[c] = 0.f;
  for (int j0 = 0; j0 < S; j0 += 4) {
    float l[4];
    float v[4][CPT];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int j = min(j0 + u, S - 1);   // past the end: reloads the last split, masked below
      l[u] = (j0 + u < S) ? p.part_ml[((size_t)g * S + j) * H + h] : -INFINITY;
      if constexpr (BF16OUT) {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        static_assert(CPT == 8, "one 16-byte load of fp16 partials per thread");
        const f16x8 t = *(const f16x8*)((const _Float16*)p.part_o + (((size_t)g * S + j) * H + h) * DV + c0);
#pragma unroll
        for (int c = 0; c < 8; c++) v[u][c] = (float)t[c];
        continue;
      }
      const float* src = p.part_o + (((size_t)g * S + j) * H + h) * DV + c0;
      if constexpr (CPT % 4 == 0) {
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
          const f32x4 t = *(const f32x4*)(src + c);
          v[u][c] = t[0]; v[u][c + 1] = t[1]; v[u][c + 2] = t[2]; v[u][c + 3] = t[3];
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPT; c++) v[u][c] = src[c];
      }
    }
    const float mn = fmaxf(fmaxf(mx, fmaxf(l[0], l[1])), fmaxf(l[2], l[3]));
    if (mn == -INFINITY) continue;          // no selected row so far
    const float sc = exp2f(mx - mn);        // 0 while mx is still -inf
    den *= sc;
#pragma unroll
    for (int c = 0; c < CPT; c++) acc[c] *= sc;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float wj = (l[u] == -INFINITY) ? 0.f : exp2f(l[u] - mn);
      den += wj;
#pragma unroll
      for (int c = 0; c < CPT; c++) acc[c] += wj * v[u][c];
    }
    mx = mn;
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
// output columns.  With KV8 the rows are FP8 bytes, each multiplied by the
// fp32 scale of its tile of 128 elements as it is staged.
template <int H, int DQK, int DV, bool KV8>
__global__ __launch_bounds__(256) void sfa_f32_kernel(SfaParams p) {
  constexpr int NT = (DQK + 127) / 128;
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
      s_row[tid] = (pos >= 0) ? (bt[pos >> bv.page_shift] << bv.page_shift) + (pos & (P - 1)) : -1;
    }
    __syncthreads();
    for (int e = tid; e < TR * DQK; e += 256) {
      const int r = e / DQK, c = e % DQK;
      const int row = s_row[r];
      float x = 0.f;
      if (row >= 0) {
        if constexpr (KV8)
          x = __builtin_amdgcn_cvt_f32_fp8((int)((const unsigned char*)p.kv)[(size_t)row * DQK + c], 0) *
              p.kv_scale[(size_t)row * NT + c / 128];
        else
          x = ((const float*)p.kv)[(size_t)row * DQK + c];
      }
      s_kv[r][c] = x;
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

// (precise weights, head groups of 16 per wave, FP8 rows, waves): bf16 rows
// run 8 waves of 16 heads, FP8 rows 4 waves of 16 with two workgroups per token
int sfa_bf16_waves(const SfaParams& p) { return p.kv8 ? 4 : 8; }
const void* pick_sfa_bf16(const SfaParams& p) {
  if (p.kv8)
    return p.precise_weights ? (const void*)sfa_bf16_kernel<576, 512, true, 1, true>
                             : (const void*)sfa_bf16_kernel<576, 512, false, 1, true>;
  return p.precise_weights ? (const void*)sfa_bf16_kernel<576, 512, true, 1, false, 8>
                           : (const void*)sfa_bf16_kernel<576, 512, false, 1, false, 8>;
}

hipError_t launch_sfa(int dtype, int H, int Dqk, int Dv, const SfaParams& p, hipStream_t st) {
  if (p.bv.total_q == 0) return hipSuccess;
  if (dtype == kBF16 && H == 128 && Dqk == 576 && Dv == 512) {
    if (p.rows_per_split > kSfaMaxRows) return hipErrorInvalidValue;
    // heads per workgroup x workgroups per token must cover the 128 heads
    if (p.hsplit != (p.kv8 ? 2 : 1)) return hipErrorInvalidValue;
    if (p.kv8 && !p.kv_scale) return hipErrorInvalidValue;
    const void* kern = pick_sfa_bf16(p);
    const size_t lds = p.kv8 ? SfaKv8Geom<576, 512>::lds_bytes(p.rows_per_split)
                             : SfaBf16Geom<576, 512>::lds_bytes(p.rows_per_split);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int chunk = (p.bv.total_q + 7) / 8;
    const dim3 grid(8 * chunk, p.hsplit, p.splits);
    void* args[] = {(void*)&p};
    e = hipLaunchKernel(kern, grid, dim3(64 * sfa_bf16_waves(p)), args, lds, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  if (dtype == kF32 && H == 8 && Dqk == 80 && Dv == 64) {
    if (p.kv8 && !p.kv_scale) return hipErrorInvalidValue;
    if (p.kv8)
      hipLaunchKernelGGL((sfa_f32_kernel<8, 80, 64, true>), dim3(p.bv.total_q, 1, p.splits), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((sfa_f32_kernel<8, 80, 64, false>), dim3(p.bv.total_q, 1, p.splits), dim3(256), 0, st, p);
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
