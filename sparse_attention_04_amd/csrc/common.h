// Shared device/host definitions for the gfx950 DSA kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { kF32 = 0, kBF16 = 1, kFP8 = 2, kMX = 3 };

constexpr int kWave = 64;
constexpr int kRadixBins = 2048;      // 11-bit digits
constexpr int kMaxPasses = 3;         // 11 + 11 + 10 bits
constexpr uint32_t kSpinLimit = 1u << 20;

// Error bits written to the workspace header when a bounded wait gives up.
constexpr uint32_t kErrBarrierTimeout = 1u;

// The fused decode's ready-word epoch that follows call counter value c (never
// 0, the value of a cleared ready word).
__host__ __device__ __forceinline__ uint32_t epoch_after(uint32_t c) { return (c + 1u == 0u) ? 1u : c + 1u; }

// Order-preserving map float -> uint32 (larger float -> larger key).  -0.0 is
// canonicalised to +0.0 first so both zeros compare equal.  Key 0 is never
// produced for a finite input (the smallest, -inf, maps to 0x007FFFFF), so 0
// marks "not a candidate".
__device__ __forceinline__ uint32_t float_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even f32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_relaxed_agent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_relaxed_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup barrier that waits only for this wave's LDS traffic, not for its
// outstanding global loads (a plain __syncthreads() waits for every memory
// operation, which would drain a load pipeline at each barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void store_agent_i32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier among the `count` workgroups sharing `ctr` (all co-resident).  The
// round-th call returns once count*round arrivals are seen.
//
// Every datum exchanged across workgroups around this barrier is itself an
// agent-scope atomic (RMW, load or store), which the hardware performs at the
// device-coherent level; the barrier therefore only has to order them: each
// wave waits for its own outstanding memory operations to complete before the
// workgroup arrives, and readers issue their loads after observing the count.
// No cache write-back or invalidation is needed, which keeps a barrier round to
// a few microseconds.  The wait is bounded by `spin_limit` sleeps: on timeout
// the error bit is set in `err`, the sequence's `failed` flag is raised and the
// workgroup continues, so the grid always drains.
__device__ __forceinline__ void group_barrier(uint32_t* ctr, uint32_t target, uint32_t* err, uint32_t* failed,
                                              uint32_t spin_limit) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    atomic_add_agent(ctr, 1u);
    uint32_t spins = 0;
    while (load_relaxed_agent(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > spin_limit) {
        atomic_add_agent(err, kErrBarrierTimeout);
        atomic_add_agent(failed, 1u);
        break;
      }
    }
  }
  __syncthreads();
}

// Block-wide helpers (blockDim.x a multiple of 64, at most 1024).
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Launch-parameter blocks (host fills, kernels read by value).
struct BatchView {
  int32_t batch;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t page_size;       // a power of two
  int32_t page_shift;      // log2(page_size)
  int32_t total_q;
};

}  // namespace dsa
