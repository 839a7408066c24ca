// Internal entry points shared by the C ABI's translation units (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>

#include "dsa.h"

namespace dsa {

// dsa_fused_decode's argument checks and, unless validate_only, its launches
// with the given workspace (the thread-local error message is set on failure,
// not cleared first).  validate_only skips the workspace checks.
dsa_status fused_decode_impl(const dsa_batch* b, const dsa_indexer_args* ia, const dsa_sfa_args* sa,
                             void* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                             void* stream, bool validate_only);

// Bytes at the start of a dsa_fused_decode workspace that hold its zero state
// (the rest of what dsa_workspace_size reports is scratch, kept at the end).
size_t fused_decode_state_bytes(const dsa_batch* b);

// DSA_DEBUG=1: check the device-resident batch contents (lengths, query
// offsets, block-table entries below num_pages, and idx rows of `topk` when
// idx is non-NULL) on `st` and wait for the result; DSA_ERR_INVALID_ARG with
// a message when a precondition is violated.
dsa_status debug_check_batch(const dsa_batch* b, int num_pages, int page_size, const int32_t* idx, int topk,
                             hipStream_t st);

// The current device's static scratch of dsa_fused_decode_noalloc, or NULL in
// *out if no such call has set it up on this device yet.
dsa_status noalloc_scratch_if_set_up(void** out);

// Wait for `st`, then read and clear the sticky error bits in the first word
// of an indexer workspace: DSA_ERR_HIP with a message if any was set.
dsa_status take_error_bits(uint32_t* ws, hipStream_t st);

// Record `msg` as the thread's last error and return `st`; clear it.
dsa_status set_error(dsa_status st, const char* msg);
void clear_error();

}  // namespace dsa
