// Fused decode: the Lightning Indexer and the sparse attention over its
// selection in one launch, the pages' deep fusion of the two operators
// ("Deep Fusion of LI and SFA", Day0 Inference Optimization on Ascend CANN,
// sec. 2; the fused indexer's three steps followed by SFA in Inference
// Acceleration for Next-Gen Attention Architectures, sec. 3.1-3.2).
//
// Every workgroup first does its share of the decode indexer (one page range
// of one sequence, the sequence's cross-workgroup radix select, its selected
// positions), then at most one attention task (one token, all heads, one
// range of index slots), exactly as the two kernels do apart.  A task may
// start as soon as its own sequence's index rows are complete, not when the
// whole batch is: the sequence's last indexer workgroup out writes the call's
// epoch into the sequence's ready word after every row of the sequence is
// written (the rows go out as agent-scope stores, and each workgroup's stores
// complete before it takes its exit ticket), and a task waits for that word
// and reads the rows with agent-scope loads.  So the attention of the
// sequences that finish first overlaps the selection of the others, and the
// launch between the two stages is gone.  The split ranges are merged by the
// combine kernel afterwards, as in the unfused path.
//
// Workgroup w runs on XCD w % 8 (round-robin dispatch).  Both phases number
// the workgroups XCD by XCD (virtual index (w % 8) * G/8 + w / 8), so with
// as many tasks as workgroups a workgroup's tasks belong to the sequence it
// scored, and all slot ranges of a token share one XCD.
//
// The grid is one workgroup per CU, all co-resident (sized from the
// occupancy of this kernel): every wait in it is bounded, and a task whose
// sequence never became ready (a wait gave up) skips its rows, contributes an
// empty range (lse = -inf) and sets the error bit, so the grid always drains
// and no row of a previous call is ever read.  The ready word holds an epoch
// that differs from call to call, and the sequence's last task clears it; a
// word a late writer leaves behind therefore never matches a later call's
// epoch.  The epoch comes from a counter in the workspace header that every
// workgroup reads at its start and the kernel after this one (the combine,
// or epoch_bump_kernel when there is one range per token) advances, so all
// workgroups of a launch agree on it and every replay of a captured graph
// gets a new one, as separate calls do.
#include "common.h"
#include "kernels.h"
#include "indexer_decode_body.h"
#include "sfa_body.h"

namespace dsa {
namespace {

constexpr int kFusedH = 128, kFusedDqk = 576, kFusedDv = 512;

// A task whose sequence never became ready: an empty range.
__device__ void sfa_empty_range(const SfaParams& p, int g, int split) {
  if (p.splits == 1) {
    uint16_t* out = (uint16_t*)p.out + (size_t)g * kFusedH * kFusedDv;
    for (int i = threadIdx.x; i < kFusedH * kFusedDv; i += blockDim.x) out[i] = 0;
    for (int h = threadIdx.x; h < kFusedH && p.lse; h += blockDim.x) p.lse[(size_t)g * kFusedH + h] = -INFINITY;
  } else {
    _Float16* po = (_Float16*)p.part_o + ((size_t)g * p.splits + split) * kFusedH * kFusedDv;
    for (int i = threadIdx.x; i < kFusedH * kFusedDv; i += blockDim.x) po[i] = (_Float16)0.f;
    for (int h = threadIdx.x; h < kFusedH; h += blockDim.x)
      p.part_ml[((size_t)g * p.splits + split) * kFusedH + h] = -INFINITY;
  }
}

template <int DT, int MAXQ, bool LO>
__global__ __launch_bounds__(kIdxThreads, 1) void fused_decode_kernel(IndexerDecodeParams ip, SfaParams sp) {
  static_assert(kIdxThreads == 64 * 8, "both phases run 8 waves");
  extern __shared__ __align__(16) uint32_t smem[];
  const int G = gridDim.x;   // a multiple of 8
  const int w = blockIdx.x;
  const int vw = (w & 7) * (G >> 3) + (w >> 3);
  // issued first, used only when the rows are published or awaited
  const uint32_t epoch = epoch_after(load_relaxed_agent(ip.ws + kWsEpochWord));
  indexer_decode_body<DT, 64, 128, MAXQ, true>(ip, vw, smem, epoch);
  // the indexer's LDS is free once every wave is past it
  __syncthreads();

  // One attention task per workgroup at most (the host launches the fused
  // kernel only when the tasks fit the grid): task w is token
  // (w % 8) * chunk + (w / 8) / S, slot range (w / 8) % S.  What the task
  // needs after the attention is kept in LDS, not in registers, which the
  // attention's tile loop uses to the last one.
  const int S = sp.splits;
  const int chunk = (sp.bv.total_q + 7) >> 3;   // tokens per XCD
  const int r = w >> 3, split = r % S;
  const int g = (w & 7) * chunk + r / S;
  if (r / S >= chunk || g >= sp.bv.total_q) return;
  __shared__ int s_ok, s_b;
  // The task's q loads are issued before this wait (inside the attention
  // body), so they overlap it; no index slot is read before it ends.
  auto wait_ready = [&]() -> bool {
    if (threadIdx.x == 0) {
      WsLayout W{ip.ws, ip.ws_nseq, ip.ws_nq, ip.ws_grid_pad};
      const int b = find_seq(sp.bv, g);
      uint32_t spins = 0;
      int ok = 1;
      while (load_relaxed_agent(W.seq_ready(b)) != epoch) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > ip.ready_spin_limit) {
          atomic_add_agent(W.err(), kErrBarrierTimeout);
          ok = 0;
          break;
        }
      }
      s_ok = ok;
      s_b = b;
    }
    __syncthreads();
    return s_ok != 0;
  };
  if (!sfa_bf16_body<kFusedDqk, kFusedDv, LO, 1, false, 8, true>(sp, g, 0, split, false, (unsigned char*)smem,
                                                                 wait_ready))
    sfa_empty_range(sp, g, split);
  // the last task of the sequence clears its ready word and its counter
  __syncthreads();
  if (threadIdx.x == 0) {
    WsLayout W{ip.ws, ip.ws_nseq, ip.ws_nq, ip.ws_grid_pad};
    const int b = s_b;
    const int T = sp.bv.cu_q[b + 1] - sp.bv.cu_q[b];
    const uint32_t n = atomic_add_agent(W.seq_attn_exit(b), 1u);
    if (n == (uint32_t)(T * sp.splits - 1)) {
      store_relaxed_agent(W.seq_attn_exit(b), 0u);
      store_relaxed_agent(W.seq_ready(b), 0u);
    }
  }
}

#define DSA_FUSED_SHAPES(X) \
  X(kBF16, 1, true)         \
  X(kBF16, 1, false)        \
  X(kBF16, 4, true)         \
  X(kFP8, 1, true)          \
  X(kMX, 1, true)           \
  X(kFP8, 4, true)          \
  X(kMX, 4, true)

__global__ void epoch_bump_kernel(uint32_t* w) {
  if (threadIdx.x == 0) *w = epoch_after(*w);
}

const void* pick_fused(int dtype, int maxq, bool lo) {
#define DSA_PICK(DT_, Q_, LO_) \
  if (dtype == DT_ && maxq == Q_ && lo == LO_) return (const void*)fused_decode_kernel<DT_, Q_, LO_>;
  DSA_FUSED_SHAPES(DSA_PICK)
#undef DSA_PICK
  return nullptr;
}

}  // namespace

size_t fused_decode_sfa_lds_bytes(int rows_per_split) {
  return SfaBf16Geom<kFusedDqk, kFusedDv>::lds_bytes(rows_per_split);
}

int fused_decode_max_rows() { return kSfaMaxRows; }

bool fused_decode_supported(int dtype, int maxq, bool precise_weights) {
  return pick_fused(dtype, maxq, precise_weights) != nullptr;
}

hipError_t fused_decode_occupancy(int dtype, int maxq, bool precise_weights, size_t lds, int* blocks_per_cu) {
  const void* k = pick_fused(dtype, maxq, precise_weights);
  if (!k) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k, kIdxThreads, lds);
}

hipError_t launch_fused_epoch_bump(uint32_t* epoch_word, hipStream_t st) {
  hipLaunchKernelGGL(epoch_bump_kernel, dim3(1), dim3(64), 0, st, epoch_word);
  return hipGetLastError();
}

hipError_t launch_fused_decode(int dtype, int maxq, const IndexerDecodeParams& ip, const SfaParams& sp,
                               size_t lds, hipStream_t st) {
  const void* k = pick_fused(dtype, maxq, sp.precise_weights != 0);
  // one task per workgroup at most: 8 * ceil(total_q / 8) * splits <= grid
  const int64_t tasks = 8 * (int64_t)((sp.bv.total_q + 7) / 8) * sp.splits;
  if (!k || ip.grid % 8 != 0 || ip.seq_base != 0 || sp.hsplit != 1 || sp.kv8 ||
      sp.rows_per_split > kSfaMaxRows || tasks > ip.grid || !sp.epoch_word)
    return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  IndexerDecodeParams ipc = ip;
  SfaParams spc = sp;
  void* args[] = {(void*)&ipc, (void*)&spc};
  e = hipLaunchKernel(k, dim3(ip.grid), dim3(kIdxThreads), args, lds, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace dsa
