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
constexpr int kTileRows = 32;
constexpr int kHeadsPerWG = 64;
constexpr int kLog2e_x = 0;  // (unused marker)

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

template <int DQK, int DV>
__global__ __launch_bounds__(kSfaThreads, 1) void sfa_bf16_kernel(SfaParams p) {
  constexpr int PITCH = DQK * 2 + 16;           // bytes per LDS row (padded)
  constexpr int KSTEPS = DQK / 32;               // QK^T K-steps (18)
  constexpr int VTILES = DV / 16;                // PV M-tiles (32)
  constexpr int CHUNKS = DQK * 2 / 16;           // 16-byte chunks per row (72)
  constexpr int LOADS = (kTileRows * CHUNKS + kSfaThreads - 1) / kSfaThreads;  // 9
  extern __shared__ __attribute__((aligned(16))) unsigned char sfa_smem[];
  unsigned char* buf0 = sfa_smem;
  unsigned char* buf1 = sfa_smem + kTileRows * PITCH;
  int32_t* s_rows = (int32_t*)(sfa_smem + 2 * kTileRows * PITCH);   // [rows_per_split]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x;                      // query token
  const int hg = blockIdx.y;                     // head group of 64
  const int split = blockIdx.z;
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  const int b = find_seq(bv, g);
  const int* bt = bv.block_table + (size_t)b * bv.max_pages;
  const int slot0 = split * p.rows_per_split;
  const int nslots = max(0, min(p.topk - slot0, p.rows_per_split));
  const int32_t* idx = p.idx + (size_t)g * p.topk + slot0;

  // physical rows of this range (-1 for empty slots)
  for (int r = tid; r < nslots; r += kSfaThreads) {
    const int pos = idx[r];
    s_rows[r] = (pos >= 0) ? bt[pos / P] * P + (pos % P) : -1;
  }
  __syncthreads();
  int fallback = -1;  // a valid row to read in place of empty slots
  for (int r = 0; r < nslots && fallback < 0; r++) fallback = s_rows[r];

  // q^T as the B operand of S^T = KV q^T: lane l holds head 16*wave + l%16,
  // dims 32*kk + 8*(l/16) .. +7 for K-step kk.
  const int head = hg * kHeadsPerWG + 16 * wave + (lane & 15);
  const int grp = lane >> 4;
  bf16x8 qb[KSTEPS];
  {
    const bf16x8* qs = (const bf16x8*)((const uint16_t*)p.q + ((size_t)g * (gridDim.y * kHeadsPerWG) + head) * DQK);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk++) qb[kk] = qs[4 * kk + grp];
  }

  f32x4 o[VTILES];
#pragma unroll
  for (int i = 0; i < VTILES; i++) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (nslots + kTileRows - 1) / kTileRows;
  u32x4 stage[LOADS];
  auto gather = [&](int tile) {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kSfaThreads * i;
      if (c < kTileRows * CHUNKS) {
        const int r = c / CHUNKS, col = c % CHUNKS;
        const int slot = tile * kTileRows + r;
        int row = (slot < nslots) ? s_rows[slot] : -1;
        if (row < 0) row = fallback;
        stage[i] = ((const u32x4*)((const uint16_t*)p.kv + (size_t)row * DQK))[col];
      }
    }
  };
  auto put = [&](unsigned char* buf) {
#pragma unroll
    for (int i = 0; i < LOADS; i++) {
      const int c = tid + kSfaThreads * i;
      if (c < kTileRows * CHUNKS) {
        const int r = c / CHUNKS, col = c % CHUNKS;
        *(u32x4*)(buf + r * PITCH + col * 16) = stage[i];
      }
    }
  };

  if (ntiles > 0 && fallback >= 0) {
    gather(0);
    put(buf0);
  }
  __syncthreads();
  for (int tile = 0; tile < ntiles && fallback >= 0; tile++) {
    unsigned char* cur = (tile & 1) ? buf1 : buf0;
    unsigned char* nxt = (tile & 1) ? buf0 : buf1;
    if (tile + 1 < ntiles) gather(tile + 1);

    // ---- S^T = KV q^T : rows on M (two 16-row tiles), this wave's 16 heads on N
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* ra = cur + (lane & 15) * PITCH + grp * 16;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk++) {
      const bf16x8 a0 = *(const bf16x8*)(ra + kk * 64);
      const bf16x8 a1 = *(const bf16x8*)(ra + 16 * PITCH + kk * 64);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb[kk], s1, 0, 0, 0);
    }
    // ---- online softmax over this tile for head (lane & 15); this lane holds
    // rows 4*grp + i (s0) and 16 + 4*grp + i (s1)
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r0 = tile * kTileRows + 4 * grp + i, r1 = r0 + 16;
      z[i] = (r0 < nslots && s_rows[r0] >= 0) ? s0[i] * p.scale_log2 : -INFINITY;
      z[4 + i] = (r1 < nslots && s_rows[r1] >= 0) ? s1[i] * p.scale_log2 : -INFINITY;
    }
    float mt = z[0];
#pragma unroll
    for (int i = 1; i < 8; i++) mt = fmaxf(mt, z[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    float pv[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      pv[i] = none ? 0.f : exp2f(z[i] - m_new);
      psum += pv[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; i++) pb[i] = (__bf16)pv[i];
#pragma unroll
    for (int i = 0; i < VTILES; i++) o[i] *= alpha;

    // ---- O^T[v, head] += V^T[v, rows] P^T[rows, head]
    // ds_read_b64_tr_b16 within each 16-lane group: source lane s = 4j + r
    // reads row (4*grp + j) [+16], columns 16*mv + 4r .. +3; lane l then holds
    // column 16*mv + l%16 of those 4 rows.
    const int sl = lane & 15;
    const unsigned char* tb0 = cur + (4 * grp + (sl >> 2)) * PITCH + (sl & 3) * 8;
    const unsigned char* tb1 = tb0 + 16 * PITCH;
#pragma unroll
    for (int mv = 0; mv < VTILES; mv++) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb0 + mv * 32));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tb1 + mv * 32));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, o[mv], 0, 0, 0);
    }

    if (tile + 1 < ntiles) put(nxt);
    __syncthreads();
  }

  // ---- epilogue: full row sum for this head, then write
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int H = gridDim.y * kHeadsPerWG;
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  if (p.splits == 1) {
    uint16_t* out = (uint16_t*)p.out + ((size_t)g * H + head) * DV;
#pragma unroll
    for (int mv = 0; mv < VTILES; mv++) {
      const int v = 16 * mv + 4 * grp;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(o[mv][0] * inv) | ((uint32_t)f32_to_bf16(o[mv][1] * inv) << 16);
      pk.y = (uint32_t)f32_to_bf16(o[mv][2] * inv) | ((uint32_t)f32_to_bf16(o[mv][3] * inv) << 16);
      *(uint2*)(out + v) = pk;
    }
    if (p.lse && grp == 0)
      p.lse[(size_t)g * H + head] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  } else {
    float* po = p.part_o + (((size_t)g * p.splits + split) * H + head) * DV;
#pragma unroll
    for (int mv = 0; mv < VTILES; mv++) {
      const int v = 16 * mv + 4 * grp;
      *(f32x4*)(po + v) = o[mv] * inv;
    }
    if (grp == 0)
      p.part_ml[((size_t)g * p.splits + split) * H + head] = (l_run > 0.f) ? m_run + log2f(l_run) : -INFINITY;
  }
}

// Merge the per-range partials of one token: weights 2^(lse_j - lse).
template <int DV, bool BF16OUT>
__global__ __launch_bounds__(256) void sfa_combine_kernel(SfaParams p, int H) {
  const int g = blockIdx.x;
  const int S = p.splits;
  for (int e = threadIdx.x; e < H * (DV / 4); e += blockDim.x) {
    const int h = e / (DV / 4), v = 4 * (e % (DV / 4));
    float mx = -INFINITY;
    for (int j = 0; j < S; j++) mx = fmaxf(mx, p.part_ml[((size_t)g * S + j) * H + h]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int j = 0; j < S; j++) {
      const float l = p.part_ml[((size_t)g * S + j) * H + h];
      if (l == -INFINITY) continue;
      const float wj = exp2f(l - mx);
      den += wj;
      acc += wj * *(const f32x4*)(p.part_o + (((size_t)g * S + j) * H + h) * DV + v);
    }
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
    acc *= inv;
    if (BF16OUT) {
      uint16_t* out = (uint16_t*)p.out + ((size_t)g * H + h) * DV + v;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      *(uint2*)out = pk;
    } else {
      *(f32x4*)((float*)p.out + ((size_t)g * H + h) * DV + v) = acc;
    }
    if (p.lse && v == 0)
      p.lse[(size_t)g * H + h] = (den > 0.f) ? (mx + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
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
    const size_t lds = 2 * kTileRows * (576 * 2 + 16) + (size_t)p.rows_per_split * 4;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(p.bv.total_q, H / kHeadsPerWG, p.splits), dim3(kSfaThreads), lds, st, p);
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
    hipLaunchKernelGGL((sfa_combine_kernel<512, true>), dim3(p.bv.total_q), dim3(256), 0, st, p, H);
    return hipGetLastError();
  }
  if (dtype == kF32 && Dv == 64) {
    hipLaunchKernelGGL((sfa_combine_kernel<64, false>), dim3(p.bv.total_q), dim3(256), 0, st, p, H);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
