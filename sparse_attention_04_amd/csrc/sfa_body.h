// Device side of the bf16 sparse attention: the work of one workgroup (one
// token, its heads, one range of index slots) as a function, shared by the
// SFA kernel and the fused decode kernel.  The method and the layouts are
// described in sfa.hip.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dsa {
namespace {

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


// One 16-byte-per-lane global->LDS load (64 lanes fill lds_base .. +1 KiB in
// lane order).  Issued through inline assembly so that the compiler's
// wait-count pass, which cannot tell these LDS writes apart from the LDS reads
// of other ring slots, does not drain every in-flight tile before each read;
// the kernel orders them itself with explicit vmcnt waits and barriers.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}

// The 4-byte form (64 lanes fill lds_base .. +255 in lane order).
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_base) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char*)p;
}

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima): gfx9 encoding.
#define DSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// LDS operand loads of the MFMA loops, issued through inline assembly so that
// the compiler neither hoists all of them at once (which would need more
// registers than a wave has) nor waits on them early.  Each result is used
// only after lds_wait<N>() has taken it as an operand, which orders the use
// after the wait; N counts the LDS loads issued after it (they complete in
// order).
// (The byte offset OFF is an immediate, so one address register serves a
// whole loop.)
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  bf16x8 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16_b64(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  s16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8& a, bf16x8& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(s16x4& a, s16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}

// bf16 SFA, H = 128, Dqk = 576, Dv = 512.
//
// A workgroup serves 16 * NW * HG heads of one token for one range of index
// slots, with NW waves of 16 * HG heads each (HG groups ht of 16).  Wave w
// keeps q^T for all 576 dims in registers (72 VGPRs per group) and the O^T
// accumulators for all 512 columns (128 per group).  Each K/V operand read
// from LDS feeds every head group of the wave.  Configurations:
//   * bf16 rows: NW = 8, HG = 1, two waves per SIMD, so one wave's products
//     overlap the other's barrier and tile waits; the operand reads in flight
//     are fewer to fit 256 registers per wave (NW = 4 with HG = 2, one wave
//     per SIMD, measured 8% slower in prefill and more in decode);
//   * FP8 rows: NW = 4, HG = 1 (two workgroups per token, grid y).
// All heads of a token in one workgroup bring a gathered row on chip once per
// token and range.
//
// Per tile of 32 index slots:
//   S^T[row, head] = KV[row, :] . q[head, :]     16x16x32 bf16 MFMAs, rows on M
//   softmax weights against a fixed reference (see below)
//   O^T[v, head] += V^T[v, row] P^T[row, head]   V^T read with ds_read_b64_tr_b16
// The weights leave the first product already in the B-operand layout of the
// second, rounded to bf16 (each within 2^-8 relative; the denominator sums
// the rounded weights, so the output stays a convex combination of rows).
// With LO the wave also multiplies in the rounding residuals (a second bf16
// part), so the weights enter to ~2^-16 relative; it
// costs the PV product twice the MFMAs and is used where the launch is bound
// by memory rather than by the matrix units (few query tokens).  Rows stream
// through a 4-deep ring of LDS tiles filled by direct global->LDS loads; slots
// holding -1 are masked.
constexpr int kSfaKv8Threads = 256;        // threads of the FP8-row configuration (4 waves)
constexpr int kSfaMaxRows = 2048;          // index slots per workgroup (LDS row table)
constexpr float kSfaRefMargin = 40.f;      // softmax reference above the first tile maximum (log2 units)

template <int DQK, int DV, int NW_ = 4>
struct SfaBf16Geom {
  static constexpr int ROWB = DQK * 2;               // bytes of one latent row (1152)
  static constexpr int PITCH = ROWB + 32;            // LDS bytes per row (74 chunks of 16 B)
  static constexpr int TR = 32;                      // rows per tile
  static constexpr int NW = NW_;                     // waves
  static constexpr int LOADS = (TR * PITCH + 1023) / 1024;  // 1-KiB loads per tile (37)
  static constexpr int LPW = (LOADS + NW - 1) / NW;  // loads of wave 0 per tile (10)
  static constexpr int TILE = LOADS * 1024;          // LDS bytes per tile buffer
  static constexpr int NBUF = 4;                     // tiles in flight
  static constexpr int NA = LOADS % NW;              // waves issuing LPW loads (the rest LPW - 1)
  static_assert(NA != 0, "some waves issue one load more than the others");
  static constexpr size_t lds_bytes(int rows) { return (size_t)NBUF * TILE + (size_t)rows * 4; }
};

// FP8 rows: a staging ring of NBUF tiles of TR raw rows (no pad: the rows are
// only read row-wise, by the dequantising pass) plus their scales, and two
// bf16 tiles in the layout above for the matrix products.
template <int DQK, int DV>
struct SfaKv8Geom {
  using B = SfaBf16Geom<DQK, DV>;
  static constexpr int TR = B::TR, NW = B::NW;
  static constexpr int NT = (DQK + 127) / 128;           // scale tiles per row (5)
  static constexpr int STG = TR * DQK;                   // staging bytes per tile (18432)
  static constexpr int RLOADS = STG / 1024;              // 1-KiB row loads per tile (18)
  static constexpr int SLOADS = (TR * NT * 4 + 255) / 256;  // 256-byte scale loads per tile (3)
  static constexpr int SBYTES = SLOADS * 256;            // LDS bytes of one tile's scales
  static constexpr int LOADS = RLOADS + SLOADS;          // 21
  static constexpr int LPW = (LOADS + NW - 1) / NW;      // loads of wave 0 per tile (6)
  static constexpr int NBUF = 4;                         // staged tiles in flight
  static_assert(STG % 1024 == 0 && DQK % 16 == 0, "row loads tile the staging buffer");
  static_assert(LOADS % NW == 1, "wave 0 issues one load more than the others");
  static_assert(kSfaKv8Threads % TR == 0, "whole threads per converted row");
  static constexpr int SCOPY = TR * NT * 4;              // scale table of one converted tile (640)
  static_assert(SCOPY % 16 == 0, "scale tables copy in 16-byte pieces");
  // [2 bf16 tiles][2 scale tables][NBUF staged tiles][NBUF staged scale tables][row table]
  static constexpr size_t tscale_off() { return 2 * (size_t)B::TILE; }
  static constexpr size_t stage_off() { return tscale_off() + 2 * (size_t)SCOPY; }
  static constexpr size_t scale_off() { return stage_off() + (size_t)NBUF * STG; }
  static constexpr size_t rows_off() { return scale_off() + (size_t)NBUF * SBYTES; }
  static constexpr size_t lds_bytes(int rows) { return rows_off() + (size_t)rows * 4; }
};

// Gate of a body whose index rows are always complete: nothing to wait for.
struct SfaNoGate {
  __device__ bool operator()() const { return true; }
};

// The work of one workgroup: token g, head group hy (workgroups sharing the
// token's heads), slot range `split`.  COHERENT: the index rows were written
// by other workgroups of the same launch (the fused decode kernel) and are
// read with agent-scope loads; gate() (called by every thread, after the q
// loads are issued and before any index slot is read) waits until they are
// complete, and when it returns false the body returns false at once, having
// read no slot.  prof_wg marks the workgroup whose first wave records phase
// clocks (DSA_SFA_PHASES builds).
template <int DQK, int DV, bool LO, int HG, bool KV8, int NWV = 4, bool COHERENT = false, typename Gate = SfaNoGate>
__device__ __forceinline__ bool sfa_bf16_body(const SfaParams& p, int g, int hy, int split, bool prof_wg,
                                              unsigned char* sfa_smem, Gate gate = Gate{}) {
  using G = SfaBf16Geom<DQK, DV, NWV>;
  using G8 = SfaKv8Geom<DQK, DV>;
  constexpr int ROWB = G::ROWB, PITCH = G::PITCH, TR = G::TR, TILE = G::TILE;
  constexpr int NBUF = KV8 ? G8::NBUF : G::NBUF;
  constexpr int NW = G::NW, LPW = KV8 ? G8::LPW : G::LPW;
  constexpr int NA = KV8 ? 1 : G::NA;        // waves issuing LPW loads per tile
  constexpr int NT = 64 * NW;                // threads
  constexpr int KS = DQK / 32;               // QK^T K-steps of 32 (18)
  constexpr int MV = DV / 16;                // PV M-tiles of 16 columns (32)
  static_assert(DQK % 32 == 0 && (!KV8 || DV % 128 == 0), "FP8 scale tiles cover whole K-steps and M-tiles");
  constexpr int H = 128;
  int32_t* s_rows = (int32_t*)(sfa_smem + (KV8 ? G8::rows_off() : (size_t)NBUF * TILE));  // [rows_per_split]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, l16 = lane & 15;
  // Optional phase clocks of the first workgroup's first wave, compiled in
  // only with DSA_SFA_PHASES (they cost registers the tile loop needs).
#ifdef DSA_SFA_PHASES
  const bool prof = p.dbg && prof_wg && tid == 0;
  unsigned long long ph[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  unsigned long long tprev = prof ? __builtin_amdgcn_s_memtime() : 0;
#define DSA_PHASE(i)                                             \
  if (prof) {                                                    \
    const unsigned long long tn = __builtin_amdgcn_s_memtime();  \
    ph[i] += tn - tprev;                                         \
    tprev = tn;                                                  \
  }
#else
#define DSA_PHASE(i)
#endif
  const BatchView& bv = p.bv;
  const int P = bv.page_size;
  const int slot0 = split * p.rows_per_split;
  const int nslots = max(0, min(p.topk - slot0, p.rows_per_split));
  const int32_t* idx = p.idx + (size_t)g * p.topk + slot0;
  // Loads that depend on the token only are issued first: this thread's first
  // index slot, and the cu_q entries the token's sequence is found from (with
  // COHERENT rows the slot is read only after the gate, below).
  auto idx_at = [&](int r) -> int {
    if constexpr (COHERENT) return (int)load_relaxed_agent((const uint32_t*)idx + r);
    return idx[r];
  };
  int pos0 = (!COHERENT && tid < nslots) ? idx_at(tid) : -1;
  const int cq = (1 + lane < bv.batch) ? bv.cu_q[1 + lane] : 0x7FFFFFFF;

  // q^T as the B operand of S^T = KV q^T (16x16x32): for head group ht, lane l
  // holds head head0 + 16*ht and dims 32*k + 8*(l/16) .. +7 of K-step k.  The
  // workgroup's 16 * NW * HG heads start at 16 * NW * HG * hy; wave w
  // holds HG groups of 16.  Loaded first, so that their latency overlaps the
  // row lookups (and, with COHERENT rows, the wait for them).
  const int head0 = 16 * NW * HG * hy + 16 * HG * wave + l16;
  bf16x8 qb[HG][KS];
#pragma unroll
  for (int ht = 0; ht < HG; ht++) {
    const bf16x8* qs = (const bf16x8*)((const uint16_t*)p.q + ((size_t)g * H + head0 + 16 * ht) * DQK);
#pragma unroll
    for (int k = 0; k < KS; k++) qb[ht][k] = qs[4 * k + grp];
  }
  if constexpr (COHERENT) {
    if (!gate()) return false;
    pos0 = (tid < nslots) ? idx_at(tid) : -1;
  }
  // the token's sequence: the number of b in [1, batch) with cu_q[b] <= g
  // (cu_q is non-decreasing), from the entries loaded above when the batch
  // fits one wave, else a binary search
  const int b = (bv.batch <= 65) ? __builtin_amdgcn_readfirstlane(__popcll(__ballot(cq <= g))) : find_seq(bv, g);
  const int* bt = bv.block_table + (size_t)b * bv.max_pages;
  for (int r = tid; r < nslots; r += NT) {
    const int pos = (r == tid) ? pos0 : idx_at(r);
    s_rows[r] = (pos >= 0) ? (bt[pos >> bv.page_shift] << bv.page_shift) + (pos & (P - 1)) : -1;
  }
  lds_barrier();
  int fallback = -1;
  for (int r = 0; r < nslots && fallback < 0; r++) fallback = s_rows[r];
  const int ntiles = (fallback >= 0) ? (nslots + TR - 1) / TR : 0;
  DSA_PHASE(0);

  // Row r of a tile sits at byte r * PITCH of its buffer.  With the 32-byte
  // pad both read patterns below (16 rows x 16 bytes per K-step, and the
  // transposing reads of 16 rows x 32 bytes) measured free of LDS bank
  // conflicts on this part.  Load c (< LOADS) of a tile fills bytes
  // 1024c .. +1023 of its buffer and is issued by wave c % NW (wave 0 issues
  // LPW loads, the others LPW - 1); lanes that land on a pad or past row 31
  // load chunk 0 of the tile's row 0.
  const int nld = (wave < NA) ? LPW : LPW - 1;
  // FP8 rows: load c (< G8::LOADS) of a tile is issued by wave c % NW.  Loads
  // below RLOADS fill staging bytes 1024c .. +1023 (rows are 16-byte
  // multiples, so a lane's 16 bytes never straddle two rows); the others fill
  // the tile's scale table s[t][r] (t < NT, r < TR) 64 floats at a time, lanes
  // past the table loading a row's first scale into the pad.
  auto issue8 = [&](int tile) {
    const int slot = tile % NBUF;
    const uint32_t stg = lds_addr(sfa_smem + G8::stage_off() + (size_t)slot * G8::STG);
    const uint32_t scl = lds_addr(sfa_smem + G8::scale_off() + (size_t)slot * G8::SBYTES);
    int lo = lane * 16;
    asm volatile("" : "+v"(lo));
    int rows[LPW];
    const unsigned char* src[LPW];
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      const int c = wave + NW * k;
      int r, col;
      if (c < G8::RLOADS) {
        const int off = c * 1024 + lo;
        r = off / DQK;
        col = off - r * DQK;
      } else {
        const int e = (c - G8::RLOADS) * 64 + lane;
        const bool real = e < TR * G8::NT;
        r = real ? e % TR : 0;
        col = real ? 4 * (e / TR) : 0;
      }
      const int slot_r = tile * TR + r;
      rows[k] = (slot_r < nslots && k < nld) ? s_rows[slot_r] : -1;
      const int row = (rows[k] < 0) ? fallback : rows[k];
      src[k] = (c < G8::RLOADS) ? (const unsigned char*)p.kv + (size_t)row * DQK + col
                                : (const unsigned char*)p.kv_scale + (size_t)row * (4 * G8::NT) + col;
    }
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      if (k < LPW - 1 || wave < NA) {
        const int c = wave + NW * k;
        if (c < G8::RLOADS)
          dma16(src[k], __builtin_amdgcn_readfirstlane(stg + c * 1024));
        else
          dma4(src[k], __builtin_amdgcn_readfirstlane(scl + (c - G8::RLOADS) * 256));
      }
    }
  };
  // Convert staged tile `tile` into bf16 buffer tile & 1: each thread turns
  // runs of 8 bytes of one row into 8 bf16 values (exact; scale 1), and the
  // tile's scale table moves next to the buffer (the staging slot is reloaded
  // before the tile's products run).
  auto convert8 = [&](int tile) {
    const int slot = tile % NBUF;
    const unsigned char* stg = sfa_smem + G8::stage_off() + (size_t)slot * G8::STG;
    unsigned char* dst = sfa_smem + (size_t)(tile & 1) * TILE;
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    // thread t takes row t / 8 and the 8-byte runs t % 8 + 8 j of it
    constexpr int TPR = kSfaKv8Threads / TR;                  // threads per row (8)
    static_assert((DQK / 8) % TPR == 0, "runs of a row split evenly");
    const int r = tid / TPR;
#pragma unroll
    for (int j = 0; j < (DQK / 8) / TPR; j++) {
      const int cu = tid % TPR + TPR * j;
      const uint2 raw = *(const uint2*)(stg + r * DQK + 8 * cu);
      const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false);
      const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true);
      const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false);
      const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true);
      const bf16x8 v = {a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
      *(bf16x8*)(dst + r * PITCH + 16 * cu) = v;
    }
    if (tid < G8::SCOPY / 16) {
      const u32x4 sv = *(const u32x4*)(sfa_smem + G8::scale_off() + (size_t)slot * G8::SBYTES + 16 * tid);
      *(u32x4*)(sfa_smem + G8::tscale_off() + (size_t)(tile & 1) * G8::SCOPY + 16 * tid) = sv;
    }
  };
  auto issue = [&](int tile) {
    unsigned char* buf = sfa_smem + (tile % NBUF) * TILE;
    // recomputed per tile (cheap ALU) rather than held in registers across
    // the loop: the lane's byte offset is hidden from loop-invariant hoisting
    int lo = lane * 16;
    asm volatile("" : "+v"(lo));
    int rows[LPW], cols[LPW];
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      const int off = (wave + NW * k) * 1024 + lo;
      const int r = off / PITCH, c = off - r * PITCH;
      const bool real = r < TR && c < ROWB;
      const int slot = tile * TR + (real ? r : 0);
      rows[k] = (slot < nslots && k < nld) ? s_rows[slot] : -1;
      cols[k] = real ? c : 0;
    }
#pragma unroll
    for (int k = 0; k < LPW; k++) {
      if (k < LPW - 1 || wave < NA) {
        const int row = (rows[k] < 0) ? fallback : rows[k];
        const unsigned char* src = (const unsigned char*)p.kv + (size_t)row * ROWB + cols[k];
        dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(buf + (wave + NW * k) * 1024)));
      }
    }
  };
  // Every compiler-visible load (q, the lookups) is complete before the first
  // tile loads are issued, so the compiler's own waits never count the
  // asm-issued tile loads, and the loop below starts as soon as its first
  // tile has landed.
  __builtin_amdgcn_s_waitcnt(0);
  // the first tiles' loads
  if constexpr (KV8) {
    for (int t = 0; t < NBUF && t < ntiles; t++) issue8(t);
  } else {
    for (int t = 0; t < NBUF - 1 && t < ntiles; t++) issue(t);
  }

  f32x4 o[HG][MV];
#pragma unroll
  for (int ht = 0; ht < HG; ht++)
#pragma unroll
    for (int i = 0; i < MV; i++) o[ht][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[HG], l_run[HG];
#pragma unroll
  for (int ht = 0; ht < HG; ht++) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }
  if constexpr (KV8) {
    // every wave's loads of the first tiles have landed
    __builtin_amdgcn_s_waitcnt(0);
    if (ntiles > 0) {
      lds_barrier();
      convert8(0);
    }
  }
  DSA_PHASE(1);

  for (int tile = 0; tile < ntiles; tile++) {
    // bf16: this wave's loads of the tile have landed; up to NBUF - 2 younger
    // tiles may still be in flight.  FP8: the same for the next tile, which
    // this iteration dequantises.
    const int ahead = KV8 ? tile + 1 : tile;
    if (ahead < ntiles) {
      const int later = min(NBUF - 2, ntiles - 1 - ahead);
      if (wave < NA) {
        if (later >= 2) DSA_WAIT_VMCNT(2 * LPW); else if (later == 1) DSA_WAIT_VMCNT(LPW); else DSA_WAIT_VMCNT(0);
      } else {
        if (later >= 2) DSA_WAIT_VMCNT(2 * (LPW - 1)); else if (later == 1) DSA_WAIT_VMCNT(LPW - 1); else DSA_WAIT_VMCNT(0);
      }
    }
    // rows of this tile that hold a selected position (bit r)
    const int rslot = tile * TR + (lane & 31);
    const uint32_t valid = (uint32_t)__ballot(lane < 32 && rslot < nslots && s_rows[rslot] >= 0);
    DSA_PHASE(2);
    // bf16: every wave's loads of this tile are in LDS, and every wave is done
    // with the previous tile, whose buffer the next load refills.  FP8: this
    // tile's bf16 values are written, the next tile's raw rows are in LDS,
    // and every wave is done with the previous tile's bf16 buffer (which the
    // next dequantisation overwrites) and with this tile's staging slot
    // (which the next load refills).
    lds_barrier();
    const unsigned char* cur;
    if constexpr (KV8) {
      if (tile + NBUF < ntiles) issue8(tile + NBUF);
      if (tile + 1 < ntiles) convert8(tile + 1);
      cur = sfa_smem + (size_t)(tile & 1) * TILE;
    } else {
      if (tile + NBUF - 1 < ntiles) issue(tile + NBUF - 1);
      cur = sfa_smem + (tile % NBUF) * TILE;
    }
    DSA_PHASE(3);

    // ---- S^T[row, head]: two 16-row M-tiles x two 16-head groups
    f32x4 s[2][HG];
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
      for (int ht = 0; ht < HG; ht++) s[rt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
    // FP8: scales of this lane's rows 16 rt + 4 grp + i (i < 4) for every
    // 128-column tile t, and the per-tile partial products (two sets, so a
    // tile's partial is folded in while the next tile's products run)
    constexpr int NTS = KV8 ? G8::NT : 1;
    f32x4 scv[NTS][2];
    f32x4 pa[KV8 ? 2 : 1][2][HG];
    if constexpr (KV8) {
      const float* ts = (const float*)(sfa_smem + G8::tscale_off() + (size_t)(tile & 1) * G8::SCOPY);
#pragma unroll
      for (int t = 0; t < NTS; t++)
#pragma unroll
        for (int rt = 0; rt < 2; rt++) scv[t][rt] = *(const f32x4*)(ts + t * TR + 16 * rt + 4 * grp);
    }
    auto fold = [&](auto T) {
      constexpr int t = decltype(T)::value;
#pragma unroll
      for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int ht = 0; ht < HG; ht++) s[rt][ht] += scv[t][rt] * pa[t & 1][rt][ht];
    };
    {
      // K-step k reads dims 32k + 8*grp .. +7 of rows l%16 and 16 + l%16;
      // QD steps are in flight at a time
      constexpr int QD = (NW == 8) ? 2 : 4;
      const uint32_t ra = lds_addr(cur) + l16 * PITCH + 16 * grp;
      bf16x8 a[QD][2];
      static_for<0, QD>([&](auto D) {
        constexpr int d = decltype(D)::value;
        a[d][0] = lds_read_b128<64 * d>(ra);
        a[d][1] = lds_read_b128<16 * PITCH + 64 * d>(ra);
      });
      static_for<0, KS>([&](auto K) {
        constexpr int k = decltype(K)::value;
        constexpr int sl = k % QD;
        lds_wait<2 * (k + QD <= KS ? QD - 1 : KS - 1 - k)>(a[sl][0], a[sl][1]);
        if constexpr (KV8) {
          // K-steps 4t .. 4t + 3 make up column tile t
          constexpr int par = (k / 4) & 1;
          constexpr f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ht = 0; ht < HG; ht++) {
            pa[par][0][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sl][0], qb[ht][k], (k % 4 == 0) ? zero : pa[par][0][ht], 0, 0, 0);
            pa[par][1][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sl][1], qb[ht][k], (k % 4 == 0) ? zero : pa[par][1][ht], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int ht = 0; ht < HG; ht++) {
            s[0][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sl][0], qb[ht][k], s[0][ht], 0, 0, 0);
            s[1][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[sl][1], qb[ht][k], s[1][ht], 0, 0, 0);
          }
        }
        if constexpr (k + QD < KS) {
          a[sl][0] = lds_read_b128<64 * (k + QD)>(ra);
          a[sl][1] = lds_read_b128<16 * PITCH + 64 * (k + QD)>(ra);
        }
        // the previous tile's partial, one K-step after its last product
        if constexpr (KV8 && k % 4 == 1 && k >= 5) fold(std::integral_constant<int, k / 4 - 1>{});
      });
      if constexpr (KV8) fold(std::integral_constant<int, (KS - 1) / 4>{});
    }
    DSA_PHASE(4);

    // ---- softmax weights for heads l%16 (+16 ht); this lane holds rows
    // 4*grp + i and 16 + 4*grp + i (i < 4) of each head group.
    // Reference m_ref: the first tile with a selected row sets it to its
    // maximum plus kSfaRefMargin (log2 units), so weights 2^(z - m_ref) are at
    // most 2^-40 and the usual case never rescales.  A later tile whose
    // maximum passes m_ref (a logit more than kSfaRefMargin above the first
    // maximum) moves m_ref to that maximum plus the margin and rescales the
    // accumulators by 2^(old - new) first, so no weight ever exceeds 1 and the
    // sums stay finite whatever the order of the index rows.  Terms more than
    // ~86 below the reference's maximum are flushed, negligible next to its own
    // weight.  The normalised result does not depend on m_ref.
    bf16x8 phi[HG], plo[HG];
    float pwv[KV8 ? HG : 1][8];   // FP8: the fp32 weights, scaled per V tile below
#pragma unroll
    for (int ht = 0; ht < HG; ht++) {
      float z[8];
      float mt = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int r = 16 * (e >> 2) + 4 * grp + (e & 3);
        const float v = s[e >> 2][ht][e & 3];
        z[e] = ((valid >> r) & 1u) ? v * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, z[e]);
      }
      // the head's maximum over the tile (its rows sit in the four lane groups)
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      if (m_run[ht] == -INFINITY) {
        m_run[ht] = mt + kSfaRefMargin;     // still -inf if no row of the tile is selected
      } else if (mt > m_run[ht]) {
        // rare: move the reference up and rescale what was accumulated
        const float m_new = mt + kSfaRefMargin;
        const float alpha = __builtin_amdgcn_exp2f(m_run[ht] - m_new);
        l_run[ht] *= alpha;
#pragma unroll
        for (int mv = 0; mv < MV; mv++) o[ht][mv] *= alpha;
        m_run[ht] = m_new;
      }
      const bool none = (m_run[ht] == -INFINITY);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float pw = none ? 0.f : __builtin_amdgcn_exp2f(z[e] - m_run[ht]);
        if constexpr (KV8) {
          pwv[ht][e] = pw;
          psum += pw;
          continue;
        }
        const __bf16 hi = (__bf16)pw;
        phi[ht][e] = hi;
        if constexpr (LO) {
          const __bf16 lo = (__bf16)(pw - (float)hi);
          plo[ht][e] = lo;
          // the denominator sums exactly what the PV product multiplies in
          psum += (float)hi + (float)lo;
        } else {
          psum += (float)hi;
        }
      }
      l_run[ht] += psum;
    }
    DSA_PHASE(5);

    // ---- O^T[v, head] += V^T[v, rows] P^T[rows, head]: 16 columns on M, heads
    // on N, K = the tile's 32 rows.  This lane's K-slots 8*grp .. +7 hold rows
    // 4*grp + j and 16 + 4*grp + j (j < 4), matching the weights.  V^T comes
    // from ds_read_b64_tr_b16: in each 16-lane group, source lane s = 4j + r
    // reads columns vbase + 4r .. +3 of row j of the group's 4 rows; lane i
    // then holds column vbase + i of those 4 rows.
    {
      // M-tile mv reads columns 16 mv .. +15 of rows r0 and 16 + r0; PD tiles
      // are in flight at a time
      constexpr int PD = (NW == 8) ? 4 : 6;
      const int r0 = 4 * grp + (l16 >> 2);
      const uint32_t rv = lds_addr(cur) + r0 * PITCH + 8 * (l16 & 3);
      s16x4 v[PD][2];
      static_for<0, PD>([&](auto D) {
        constexpr int d = decltype(D)::value;
        v[d][0] = lds_read_tr16_b64<32 * d>(rv);
        v[d][1] = lds_read_tr16_b64<16 * PITCH + 32 * d>(rv);
      });
      static_for<0, MV>([&](auto M) {
        constexpr int mv = decltype(M)::value;
        constexpr int sl = mv % PD;
        if constexpr (KV8 && mv % 8 == 0) {
          // V columns 128 tv .. +127: weight of row r times that row's scale
          constexpr int tv = mv / 8;
#pragma unroll
          for (int ht = 0; ht < HG; ht++)
#pragma unroll
            for (int e = 0; e < 8; e++) {
              const float w = pwv[ht][e] * scv[tv][e >> 2][e & 3];
              const __bf16 hi = (__bf16)w;
              phi[ht][e] = hi;
              if constexpr (LO) plo[ht][e] = (__bf16)(w - (float)hi);
            }
        }
        lds_wait<2 * (mv + PD <= MV ? PD - 1 : MV - 1 - mv)>(v[sl][0], v[sl][1]);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 av = {v[sl][0][0], v[sl][0][1], v[sl][0][2], v[sl][0][3],
                          v[sl][1][0], v[sl][1][1], v[sl][1][2], v[sl][1][3]};
        const bf16x8 am = __builtin_bit_cast(bf16x8, av);
#pragma unroll
        for (int ht = 0; ht < HG; ht++) {
          o[ht][mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, phi[ht], o[ht][mv], 0, 0, 0);
          if constexpr (LO) o[ht][mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, plo[ht], o[ht][mv], 0, 0, 0);
        }
        if constexpr (mv + PD < MV) {
          v[sl][0] = lds_read_tr16_b64<32 * (mv + PD)>(rv);
          v[sl][1] = lds_read_tr16_b64<16 * PITCH + 32 * (mv + PD)>(rv);
        }
      });
    }
    DSA_PHASE(6);
  }

  // ---- epilogue: o[ht][mv][i] holds head head0 + 16*ht, v = 16*mv + 4*grp + i
#pragma unroll
  for (int ht = 0; ht < HG; ht++) {
    float l = l_run[ht];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    const int head = head0 + 16 * ht;
    if (p.splits == 1) {
      uint16_t* out = (uint16_t*)p.out + ((size_t)g * H + head) * DV;
#pragma unroll
      for (int mv = 0; mv < MV; mv++) {
        const int v = 16 * mv + 4 * grp;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(o[ht][mv][0] * inv) | ((uint32_t)f32_to_bf16(o[ht][mv][1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16(o[ht][mv][2] * inv) | ((uint32_t)f32_to_bf16(o[ht][mv][3] * inv) << 16);
        *(uint2*)(out + v) = pk;
      }
      if (p.lse && grp == 0)
        p.lse[(size_t)g * H + head] = (l > 0.f) ? (m_run[ht] + log2f(l)) * 0.69314718055994531f : -INFINITY;
    } else {
      // normalised partials are convex combinations of V rows (|o| <= max|V|),
      // kept in fp16: within 2^-11 relative, half the bytes of f32
      typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
      _Float16* po = (_Float16*)p.part_o + (((size_t)g * p.splits + split) * H + head) * DV;
#pragma unroll
      for (int mv = 0; mv < MV; mv++) {
        const f32x4 v = o[ht][mv] * inv;
        *(f16x4*)(po + 16 * mv + 4 * grp) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      }
      if (grp == 0)
        p.part_ml[((size_t)g * p.splits + split) * H + head] = (l > 0.f) ? m_run[ht] + log2f(l) : -INFINITY;
    }
  }
  DSA_PHASE(7);
#ifdef DSA_SFA_PHASES
  if (prof)
    for (int i = 0; i < 8; i++) p.dbg[i] = ph[i];
#endif
#undef DSA_PHASE
  return true;
}

}  // namespace
}  // namespace dsa
