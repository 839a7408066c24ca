// Internal entry points shared by the C ABI's translation units (not part of the ABI).
#pragma once
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

// Record `msg` as the thread's last error and return `st`; clear it.
dsa_status set_error(dsa_status st, const char* msg);
void clear_error();

}  // namespace dsa
