// dsa_fused_decode_noalloc: the fused decode step with its scratch memory in a
// static device array instead of a caller workspace, for callers that cannot
// allocate (code under graph capture, serving loops that forbid allocation).
//
// The array is a file-scope __device__ variable, so every GPU the library runs
// on holds its own copy from module load until the process ends.  Its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept; host code only ever passes that address on, never the
// array's name (a host-side stand-in that is not a device address).  The
// decode indexer's part of the scratch must be zero when a call starts, and
// each call leaves it zero; the first call on a device clears it once with a
// fill kernel, in stream order, for the case that the loader did not.
//
// All calls on one GPU share its array: two calls that may overlap on the same
// GPU (different streams, or different host threads without ordering) race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "api_internal.h"
#include "common.h"
#include "dsa.h"

namespace dsa {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
// The first 16 MiB hold the decode indexer's zero state, the rest the index
// rows and attention partials (placed at the array's end): a call whose state
// or scratch exceeds its part is refused, so no call ever finds another call's
// scratch where it keeps its state, whatever the order of their shapes.
constexpr size_t kStateBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};      // device address of `scratch`, per device
bool g_cleared[kMaxDevices] = {};   // first-call clear enqueued, per device

__global__ void clear_scratch_kernel(u32x4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

dsa_status scratch_for_current_device(void** out, hipStream_t st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(DSA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return set_error(DSA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return set_error(DSA_ERR_HIP, msg);
    }
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    hipLaunchKernelGGL(clear_scratch_kernel, dim3(1024), dim3(256), 0, st, (u32x4*)g_ptr[dev], kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return set_error(DSA_ERR_HIP, "scratch clear launch failed");
    g_cleared[dev] = true;
  }
  *out = g_ptr[dev];
  return DSA_OK;
}

}  // namespace

dsa_status noalloc_scratch_if_set_up(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(DSA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return DSA_OK;
  std::lock_guard<std::mutex> lock(g_mu);
  *out = g_ptr[dev];
  return DSA_OK;
}

}  // namespace dsa

extern "C" {

size_t dsa_noalloc_scratch_bytes(void) { return dsa::kScratchBytes; }

dsa_status dsa_fused_decode_noalloc(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa,
                                    void* out, float* lse, int32_t* idx_out, void* stream) {
  dsa::clear_error();
  // every argument check runs before anything is enqueued (the first call's
  // scratch clear included)
  dsa_status s = dsa::fused_decode_impl(b, ia, sa, out, lse, idx_out, nullptr, 0, stream, true);
  if (s != DSA_OK) return s;
  const size_t need = dsa_workspace_size(DSA_OP_FUSED_DECODE, b, ia, sa);
  const size_t state = dsa::fused_decode_state_bytes(b);
  if (state > dsa::kStateBytes || need - state > dsa::kScratchBytes - dsa::kStateBytes) {
    char msg[240];
    snprintf(msg, sizeof msg, "this call needs %zu bytes of state and %zu of scratch; the static scratch holds %zu and %zu",
             state, need - state, dsa::kStateBytes, dsa::kScratchBytes - dsa::kStateBytes);
    return dsa::set_error(DSA_ERR_UNSUPPORTED, msg);
  }
  void* ws = nullptr;
  s = dsa::scratch_for_current_device(&ws, (hipStream_t)stream);
  if (s != DSA_OK) return s;
  return dsa::fused_decode_impl(b, ia, sa, out, lse, idx_out, ws, dsa::kScratchBytes, stream, false);
}

}  // extern "C"
