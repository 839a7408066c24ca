// Device-side checks of the batch contents, run only with DSA_DEBUG=1 before
// anything else of a call is enqueued: the lengths, query offsets, block-table
// entries (and index rows handed to the attention) are preconditions that the
// host checks cannot see, and a wrong one would otherwise send the kernels to
// rows outside the caches ("Inference Acceleration for Next-Gen Attention
// Architectures", section 3.2, on paged addressing).
#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "api_internal.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int kCheckThreads = 256;
constexpr int kMaxDevices = 64;
__device__ __align__(16) uint32_t check_flags[4];
std::mutex g_mu;
uint32_t* g_flags[kMaxDevices] = {};

__global__ void clear_flags_kernel(uint32_t* flags) { flags[0] = 0u; }

// Workgroup 0 checks the lengths, query offsets and block-table entries; every
// workgroup checks the index rows of every gridDim.x-th token.  Flag bits as
// in debug_check_batch.
__global__ __launch_bounds__(kCheckThreads) void check_batch_kernel(BatchView bv, int max_q_len, int max_seq_len,
                                                                    int num_pages, const int32_t* idx, int topk,
                                                                    uint32_t* flags) {
  __shared__ uint32_t s_f;
  if (threadIdx.x == 0) s_f = 0u;
  __syncthreads();
  uint32_t f = 0u;
  const int64_t cap = (int64_t)bv.max_pages * bv.page_size;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0 && (bv.cu_q[0] != 0 || bv.cu_q[bv.batch] != bv.total_q)) f |= 2u;
    for (int b = 0; b < bv.batch; b++) {
      const int L = bv.seq_lens[b];
      const int q0 = bv.cu_q[b], q1 = bv.cu_q[b + 1];
      if (threadIdx.x == 0) {
        if (L < 0 || L > max_seq_len || L > cap) f |= 1u;
        if (q1 < q0 || q1 - q0 > max_q_len || q1 - q0 > L) f |= 2u;
      }
      const int Lc = (int)min((int64_t)max(L, 0), cap);
      const int np = (Lc + bv.page_size - 1) >> bv.page_shift;
      const int32_t* row = bv.block_table + (size_t)b * bv.max_pages;
      for (int i = threadIdx.x; i < np; i += kCheckThreads) {
        const int e = row[i];
        if (e < 0 || e >= num_pages) f |= 4u;
      }
    }
  }
  // index rows handed to the attention: positions in [0, L) of the token's
  // sequence, or -1
  for (int t = blockIdx.x; idx && t < bv.total_q; t += gridDim.x) {
    int lo = 0, hi = bv.batch - 1;   // the sequence: largest b with cu_q[b] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (bv.cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int L = bv.seq_lens[lo];
    for (int s = threadIdx.x; s < topk; s += kCheckThreads) {
      const int v = idx[(size_t)t * topk + s];
      if (v < -1 || v >= L) f |= 8u;
    }
  }
  if (f) atomicOr(&s_f, f);
  __syncthreads();
  if (threadIdx.x == 0 && s_f) atomicOr(flags, s_f);
}

}  // namespace

dsa_status debug_check_batch(const dsa_batch* b, int num_pages, int page_size, const int32_t* idx, int topk,
                             hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return set_error(DSA_ERR_HIP, "hipGetDevice failed (debug checks)");
  uint32_t* flags = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_flags[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flags));
      if (e != hipSuccess || !p) return set_error(DSA_ERR_HIP, "hipGetSymbolAddress(check_flags) failed");
      g_flags[dev] = (uint32_t*)p;
    }
    flags = g_flags[dev];
  }
  BatchView bv{};
  bv.batch = b->batch;
  bv.seq_lens = b->seq_lens;
  bv.cu_q = b->cu_q;
  bv.block_table = b->block_table;
  bv.max_pages = b->max_pages_per_seq;
  bv.page_size = page_size;
  bv.page_shift = __builtin_ctz((unsigned)page_size);
  bv.total_q = b->total_q;
  const int grid = idx ? (int)std::min<int64_t>(1024, std::max<int64_t>(1, b->total_q)) : 1;
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(1), 0, st, flags);
  hipLaunchKernelGGL(check_batch_kernel, dim3(grid), dim3(kCheckThreads), 0, st, bv, b->max_q_len, b->max_seq_len,
                     num_pages, idx, topk, flags);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(DSA_ERR_HIP, "debug check launch failed");
  uint32_t f = 0;
  e = hipMemcpyAsync(&f, flags, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(DSA_ERR_HIP, "debug check read-back failed");
  if (!f) return DSA_OK;
  char msg[400];
  snprintf(msg, sizeof msg, "DSA_DEBUG: batch contents violate the preconditions (flags 0x%x):%s%s%s%s", f,
           (f & 1u) ? " a seq_lens entry is negative or above max_seq_len or max_pages_per_seq * page_size;" : "",
           (f & 2u) ? " cu_q does not run from 0 to total_q without decreasing, or a sequence has more query tokens than max_q_len or than keys;" : "",
           (f & 4u) ? " a block_table entry of a page in use is outside [0, num_pages);" : "",
           (f & 8u) ? " an index row holds a position outside [-1, seq_len);" : "");
  return set_error(DSA_ERR_INVALID_ARG, msg);
}

}  // namespace dsa
