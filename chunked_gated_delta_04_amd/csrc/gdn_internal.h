// Host-side declarations shared by the launchers and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"

namespace gdn {

// Blocks written by the WY pass. Value-head blocks: blk = hv * NC + c, so the
// chunks of one chain are contiguous. Key-head blocks (the normalised q and k,
// which do not depend on the gates and so serve every value head of their key
// head): kblk = (hv / G) * NC + c. Every tile is stored in the chunk-major
// layout of kcm() with its contraction axis chunked.
struct PrepOut {
  uint16_t* W;   // value head: W [tok][k]
  uint16_t* Qn;  // key head: Q~ [tok][k]
  uint16_t* P;   // value head: P [i][j] (its 16 x 16 tiles above the diagonal
                 // are zero and are not stored)
  uint16_t* Kn;  // key head: K^T [k][tok]
  float* gL;     // value head: e^gamma_L, 1 per block
  float* gE;     // value head: e^gamma (64), then e^(gamma_L - gamma) and beta (64
                 // each, zero past the chunk's end), kGates = 192 per block
  uint16_t* T;   // value head: T [i][j] (forward scan and backward; its 16 x 16 tiles
                 // above the diagonal are zero and are not stored), then T^T [j][i]
                 // (backward only), 2 x 64 x 64 per block
  float* gB;     // value head, backward only: the cumulative decay gamma in base 2
                 // (64), then beta (64, zero past the chunk's end), kGatesB = 128 per
                 // block
  int G;         // value heads per key head
};

// Backward scratch per (value head, chunk) block, blk = hv * NC + c.
struct BwdBufs {
  uint16_t* dh;   // gradient of the chunk's end state, [v / 32][v % 32 / 8][k][v % 8]
  uint16_t* dD;   // dD [tok][v], chunk-major (64 x 128)
  uint16_t* dDT;  // dD^T [v][tok], chunk-major (128 x 64)
};

hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int NC, ChunkInfo* table,
                              int32_t* seq_first, hipStream_t stream);

// Whether the WY pass also writes what only the backward reads (T^T, the
// cumulative decay and beta), when the forward saves for a backward.
enum class PrepMode { kForward, kBoth };

hipError_t launch_chunk_prep(PrepMode mode, const ChunkInfo* table, int NC, int H, int HV,
                             float scale, const uint16_t* q, const uint16_t* k, const float* g,
                             const float* beta, const PrepOut& fwd_out, const PrepOut& bwd_out,
                             hipStream_t stream);

// Where the forward scan takes each chain's start state and leaves its end
// state. Direct: h0 / hT are [N, HV, V, K] (either NULL). Paged: h0 == hT is a
// pool [slots, HV, V, K] updated in place; sequence n uses slot idx[n] when
// 0 < idx[n] < slots (else it starts from zero and writes nothing), starting
// from the slot when init is NULL or init[n] != 0 and from zero otherwise.
// Transition: M receives each chain's transition product and hT its end state
// from a zero start (h0 unused).
struct StateRef {
  const float* h0;
  float* hT;
  const int32_t* idx;   // paged only
  const int32_t* init;  // paged only, nullable
  int slots;
  float* M;             // transition only
};

// What one forward-scan launch produces.
enum class ScanMode {
  kOut,         // o (and hT)
  kOutSave,     // o, the saved states and D for the backward (and hT)
  kSave,        // only the saved states and D (the recomputing backward)
  kTransition,  // M and the zero-start end state, no o
};

// (v: the value rows the scan forms U = T diag(beta) V from)
hipError_t launch_fwd_scan(ScanMode mode, const int32_t* seq_first, int N, int HV, int NC,
                           const ChunkInfo* table, const PrepOut& prep, const uint16_t* v,
                           const StateRef& st, uint16_t* o, uint16_t* saved,
                           hipStream_t stream);

hipError_t launch_bwd_dh_scan(const int32_t* seq_first, int N, int HV, int NC,
                              const ChunkInfo* table, const PrepOut& prep, const uint16_t* dO,
                              const float* dhT, float* dh0, const BwdBufs& bufs,
                              hipStream_t stream);

hipError_t launch_bwd_chunk(const ChunkInfo* table, int NC, int H, int HV, float scale,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const uint16_t* saved,
                            const uint16_t* Tmat, const float* gE, const float* gB,
                            const BwdBufs& bufs, const uint16_t* dO,
                            uint16_t* dq, uint16_t* dk,
                            uint16_t* dv, float* dg, float* dbeta, hipStream_t stream);

hipError_t launch_state_copy(const float* src, float* dst, size_t n, hipStream_t stream);

hipError_t launch_decode_step(int N, int H, int HV, float scale, const uint16_t* q,
                              const uint16_t* k, const uint16_t* v, const uint16_t* a,
                              const uint16_t* b, const float* A_log, const float* dt_bias,
                              float* pool, int slots, const int32_t* idx, uint16_t* o,
                              hipStream_t stream);

}  // namespace gdn
