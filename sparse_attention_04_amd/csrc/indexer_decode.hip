// Fused Lightning Indexer for decode (few query tokens per sequence, long
// contexts): per-head relevance scores q_h . k_s read straight from the paged
// K cache, the head-weighted sum over heads, the causal mask and an exact
// Top-K, without ever writing the score row to device memory.
//
// Method: "Deep Fusion of LI and SFA" (Day0 Inference Optimization on Ascend
// CANN, sec. 2) and the three-step fused indexer (Inference Acceleration for
// Next-Gen Attention Architectures, sec. 3.1).  The pages' design is a single
// on-chip operator; here one sequence's keys are spread over several
// workgroups so that the whole chip streams the cache, and the Top-K is an
// exact cross-workgroup radix select:
//
//   1. each workgroup scores its page range (MFMA for bf16 / fp8 / MXFP8,
//      VALU for small f32 shapes) and keeps the scores in LDS as
//      order-preserving 32-bit keys;
//   2. three 11/11/10-bit radix passes: local LDS histogram of the candidates
//      that still match the fixed prefix, added into a per-query histogram in
//      the workspace, a barrier among the sequence's workgroups, then every
//      workgroup reads the same histogram and fixes the next digit of the k-th
//      key (passes stop early once the boundary bin is taken whole);
//   3. if equal keys straddle the boundary, one more exchange of per-workgroup
//      tie counts hands the remaining slots to the smallest positions;
//   4. each workgroup appends its selected positions to the query's output row.
//   When the first pass's boundary bin holds at most kHandoffCap keys, steps
//   2-3 stop after that pass: every workgroup writes the keys above the bin
//   to the row and the keys in it to a list, and the sequence's last
//   workgroup chooses the rest of them on its own (exactly, equal keys to the
//   smaller positions), with no further barrier.
//
// All workgroups of a launch are co-resident (the grid is sized from the
// occupancy of the kernel), every wait is bounded (group_barrier), and the grid
// always drains.
#include "common.h"
#include "kernels.h"
#include "indexer_decode_body.h"

namespace dsa {

size_t indexer_ws_bytes(int nseq, int nq, int grid) {
  WsLayout L{nullptr, nseq, nq, (grid + 31) / 32 * 32};
  return L.total_words() * 4;
}

template <int DT, int H, int D, int MAXQ>
__global__ __launch_bounds__(kIdxThreads, 1) void indexer_decode_kernel(IndexerDecodeParams p) {
  extern __shared__ __align__(16) uint32_t smem[];
  indexer_decode_body<DT, H, D, MAXQ, false>(p, blockIdx.x, smem, 0u);
}

// ------------------------------------------------------------------ launch ---

// The workgroups of a sequence wait for each other, so the whole grid must be
// resident at once.  The host sizes the grid from the occupancy query (at most
// what the device holds at once), and kernels on one stream run one after
// another, so a plain launch is resident as a whole unless other work shares
// the device; then the bounded waits give up, the affected rows are poisoned
// and the error bit is set (the end of indexer_decode_body).  A cooperative launch
// would have the runtime guarantee residency, but it measured about 11 us of
// idle device time before and after each launch on this part (74 us kernel,
// 22 us of gaps per call).
template <int DT, int H, int D, int MAXQ>
static hipError_t launch_one(const IndexerDecodeParams& p, size_t lds, hipStream_t st) {
  auto kern = indexer_decode_kernel<DT, H, D, MAXQ>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kIdxThreads), lds, st, p);
  return hipGetLastError();
}

int indexer_decode_max_q() { return kMaxDecodeQ; }

size_t indexer_decode_lds_bytes(int dtype, int maxq, int chunk_cap, int stage_pages) {
  const size_t xchg = (dtype == kBF16 && maxq == 4) ? 2 * kXchgSlotWords : 0;
  // the last workgroup's choice among the handed-off boundary bins (one
  // query at a time) reuses the same LDS for two 2048-bin histograms
  const size_t handoff = 2 * (size_t)kRadixBins * 4;
  return std::max((xchg_offset_words(maxq, chunk_cap, stage_pages) + xchg) * 4, handoff);
}

hipError_t indexer_decode_occupancy(int dtype, int H, int D, int maxq, size_t lds, int* blocks_per_cu) {
  const void* k = nullptr;
#define DSA_PICK(DT_, H_, D_, Q_) \
  if (dtype == DT_ && H == H_ && D == D_ && maxq == Q_) k = (const void*)indexer_decode_kernel<DT_, H_, D_, Q_>;
  DSA_INDEXER_DECODE_SHAPES(DSA_PICK)
#undef DSA_PICK
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k, kIdxThreads, lds);
}

hipError_t launch_indexer_decode(int dtype, int H, int D, int maxq, const IndexerDecodeParams& p,
                                 hipStream_t st) {
  const size_t lds = indexer_decode_lds_bytes(dtype, maxq, p.chunk_cap, p.stage_pages);
#define DSA_PICK(DT_, H_, D_, Q_) \
  if (dtype == DT_ && H == H_ && D == D_ && maxq == Q_) return launch_one<DT_, H_, D_, Q_>(p, lds, st);
  DSA_INDEXER_DECODE_SHAPES(DSA_PICK)
#undef DSA_PICK
  return hipErrorInvalidValue;
}

}  // namespace dsa
