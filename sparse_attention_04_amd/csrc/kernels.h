// Internal kernel entry points and launch parameter blocks (not part of the ABI).
#pragma once
#include "common.h"

namespace dsa {

constexpr int kMaxDecodeQ = 4;   // query tokens per sequence handled by the decode indexer

// (dtype, H, D, MAXQ) instantiations of the decode indexer.
#define DSA_INDEXER_DECODE_SHAPES(X) \
  X(kF32, 4, 32, 1)                  \
  X(kF32, 4, 32, 4)                  \
  X(kBF16, 64, 128, 1)               \
  X(kBF16, 64, 128, 4)               \
  X(kFP8, 64, 128, 1)                \
  X(kFP8, 64, 128, 4)                \
  X(kMX, 64, 128, 1)                 \
  X(kMX, 64, 128, 4)

struct IndexerDecodeParams {
  BatchView bv;            // (possibly a sub-range of) the batch
  const void* q;           // [total_q][H][D]
  const void* q_scale;     // fp8: f32 [total_q][H]; mx: u8 [total_q][H][D/32]
  const float* w;          // [total_q][H]
  const void* k_data;      // [num_pages][P][D]
  const void* k_scale;     // fp8: f32 [num_pages][P]; mx: u8 [num_pages][P][D/32]
  int32_t topk;
  int32_t* idx_out;        // [total_q][topk]
  uint32_t* ws;            // indexer workspace base
  int32_t ws_nseq, ws_nq, ws_grid_pad;  // workspace geometry (whole batch)
  int32_t seq_base;        // index of bv's first sequence in the whole batch
  int32_t grid;            // workgroups launched
  int32_t chunk_cap;       // LDS score slots per query (keys)
  int32_t stage_pages;     // LDS slots for the workgroup's block-table slice
  uint32_t spin_limit;     // sleeps before a cross-workgroup wait gives up
  uint32_t barrier_slack;  // added to every barrier target (0; a test sets it to force timeouts)
  uint32_t ready_spin_limit;  // fused kernel: sleeps before a task's wait for its rows gives up
  uint32_t publish_ready;  // fused kernel: 1; 0 only in a test that withholds the handoff
  int32_t cand_cap;        // boundary-bin candidates a sequence's last workgroup may select
                           // itself (pairs; 0 = always run the later radix passes)
};

// Candidate pairs the boundary-bin handoff may use per query: they live in the
// query's pass-1/2 histograms and tie counts, which a handed-off query never
// uses ((4096 + grid_pad) / 2 words with the host's grid pad of 2048).
constexpr int kHandoffCap = 3072;

// Word of the indexer workspace header that counts fused decode calls (the
// source of their ready-word epochs); word 0 holds the sticky error bits.
constexpr int kWsEpochWord = 8;

size_t indexer_ws_bytes(int nseq, int nq, int grid);
size_t indexer_decode_lds_bytes(int dtype, int maxq, int chunk_cap, int stage_pages);
hipError_t indexer_decode_occupancy(int dtype, int H, int D, int maxq, size_t lds, int* blocks_per_cu);
hipError_t launch_indexer_decode(int dtype, int H, int D, int maxq, const IndexerDecodeParams& p,
                                 hipStream_t st);

struct IndexerPrefillParams {
  BatchView bv;
  const void* q;           // [total_q][H][D] bf16 or e4m3 bytes
  const void* q_scale;     // fp8: f32 [total_q][H]; mx: u8 [total_q][H][D/32]
  const float* w;          // [total_q][H]
  const void* k_data;      // [num_pages][P][D] bf16 or e4m3 bytes
  const void* k_scale;     // fp8: f32 [num_pages][P]; mx: u8 [num_pages][P][D/32], 4-byte aligned
  int32_t topk;
  int32_t* idx_out;        // [total_q][topk]
  int32_t grid;            // workgroups launched (>= number of zigzag units)
};

size_t indexer_prefill_lds_bytes(int dtype);
int indexer_prefill_grid(int total_q, int batch);
int indexer_prefill_max_pages();
int indexer_prefill_max_topk();
hipError_t launch_indexer_prefill(int dtype, int H, int D, const IndexerPrefillParams& p, hipStream_t st);

// -------------------------------------------------------- indexer prolog ---

struct PrologParams {
  BatchView bv;
  int32_t total_q, d_model, H, D;
  const void* x;           // [total_q][d_model] bf16
  const void* w_q;         // [H*D][d_model] bf16
  const void* w_k;         // [D][d_model] bf16
  const void* w_w;         // [H][d_model] bf16
  const float* ln_gamma;   // [D]
  const float* ln_beta;    // [D]
  float ln_eps;
  void* q_bf16;            // [total_q][H*D] bf16: the projected q (q_out itself for bf16 output)
  void* q_out;             // fp8 / mx: [total_q][H][D] e4m3 bytes
  void* q_scale_out;       // fp8: f32 [total_q][H]; mx: u8 [total_q][H][D/32]
  float* w_out;            // [total_q][H]
  float* part;             // workspace: float32 partial sums, [n_parts][total_q][H*D + D + H] with
                           // several d_model ranges, else [1][total_q][D + H] (k and w columns)
  int32_t n_parts;         // set by the launcher: d_model ranges of the GEMM
  void* k_bf16_out;        // optional [total_q][D] bf16 normalised keys
  void* k_data;            // paged K cache [num_pages][P][D] (written at the new tokens' rows)
  void* k_scale;           // its scales (fp8: f32 [num_pages][P]; mx: u8 [num_pages][P][D/32])
};

int prolog_d_model_unit();
int prolog_n_parts(int total_q, int d_model);
size_t prolog_part_words(int total_q, int d_model, int H, int D);
hipError_t launch_prolog(int out_dtype, const PrologParams& p, hipStream_t st);

// ------------------------------------------------------------------- SFA ---

// (dtype, H_S, Dqk, Dv) instantiations of SFA.
#define DSA_SFA_SHAPES(X) \
  X(kF32, 8, 80, 64)      \
  X(kBF16, 128, 576, 512)

struct SfaParams {
  BatchView bv;
  const void* q;           // [total_q][H][Dqk]
  const void* kv;          // [num_pages][P][Dqk] in the q dtype, or e4m3 bytes with kv8
  const float* kv_scale;   // kv8: f32 [num_pages][P][ceil(Dqk / 128)], one per tile of 128
  int32_t kv8;             // rows are FP8 e4m3 with per-tile scales
  const int32_t* idx;      // [total_q][topk]
  int32_t topk;
  float scale_log2;        // softmax_scale * log2(e)
  int32_t splits;          // ranges of index slots per token
  int32_t hsplit;          // workgroups sharing one token's heads (bf16: 1 or 2; grid y)
  int32_t precise_weights; // bf16: also multiply in the bf16 rounding residuals of the weights
  int32_t rows_per_split;  // multiple of the row tile
  void* out;               // splits == 1: final [total_q][H][Dv] in q dtype
  float* lse;              // splits == 1: [total_q][H] (natural log) or null
  float* part_o;           // splits > 1: [total_q][splits][H][Dv], fp16 (bf16 kernel) or f32 (f32 kernel)
  float* part_ml;          // splits > 1: [total_q][splits][H] log2-sum-exp of each range
  unsigned long long* dbg; // optional: per-phase clock sums of workgroup 0, wave 0 (profiling)
  uint32_t* epoch_word;    // fused decode only: the call counter the combine advances, else null
};

hipError_t launch_sfa(int dtype, int H, int Dqk, int Dv, const SfaParams& p, hipStream_t st);

// ------------------------------------------------------------- fused decode ---
// The decode indexer and the bf16 SFA (H = 128, 576/512, bf16 rows) in one
// launch of one workgroup per CU; the combine follows as its own kernel.
bool fused_decode_supported(int dtype, int maxq, bool precise_weights);
size_t fused_decode_sfa_lds_bytes(int rows_per_split);
int fused_decode_max_rows();
hipError_t fused_decode_occupancy(int dtype, int maxq, bool precise_weights, size_t lds, int* blocks_per_cu);
hipError_t launch_fused_decode(int dtype, int maxq, const IndexerDecodeParams& ip, const SfaParams& sp,
                               size_t lds, hipStream_t st);
// Advances the call counter when no combine follows the fused kernel (one range per token).
hipError_t launch_fused_epoch_bump(uint32_t* epoch_word, hipStream_t st);
hipError_t launch_sfa_combine(int dtype, int H, int Dv, const SfaParams& p, hipStream_t st);

}  // namespace dsa
