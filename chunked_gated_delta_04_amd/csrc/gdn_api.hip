// C ABI of the gated delta rule library: argument checks, workspace layout,
// launch sequencing. Every argument error returns before anything is
// enqueued (the Cake page "[Cake 1/13] gdn", "Review items": extents are
// checked before any launch; RL-Kernel PR #469, "What": an active decode
// index out of range or repeated is an error).
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

#define GDN_API extern "C" __attribute__((visibility("default")))

using namespace gdn;

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kBlk64x128 = 64 * 128;  // bf16 elements of one (value head, chunk) tile
constexpr size_t kBlk64x64 = 64 * 64;
constexpr size_t kState = (size_t)kHead * kHead;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Layout {
  size_t table, seq_first, W, T, Qn, P, Kn, gL, gE, dh, dD, dDT, total;
};

// Chunk slots: the bound T/64 + N (sum of ceil(L_n / 64) <= T/64 + N), with or
// without a host copy of the boundaries, so that every size and layout - in
// particular the `saved` buffer a forward hands to a backward - depends on
// (N, T, H, HV) only; slots past the pack's chunks exit at once.
int64_t chunk_slots(const gdn_problem* p) { return (int64_t)p->T / kChunk + p->N; }

gdn_status check_problem(const gdn_problem* p, int64_t* nc) {
  if (!p) return GDN_ERR_NULL;
  if (p->N < 0 || p->T < 0 || p->H <= 0 || p->HV <= 0 || p->K <= 0 || p->V <= 0 ||
      p->chunk <= 0)
    return GDN_ERR_SHAPE;
  if (p->K != kHead || p->V != kHead || p->chunk != kChunk || p->HV % p->H != 0)
    return GDN_ERR_UNSUPPORTED;
  if (p->H > 65535) return GDN_ERR_SHAPE;  // grid.y of the per-chunk kernels
  if (p->N == 0 && p->T != 0) return GDN_ERR_SHAPE;
  if (p->T > 0 && !p->cu_seqlens) return GDN_ERR_NULL;
  if (p->cu_seqlens_host) {
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0 || cu[p->N] != p->T) return GDN_ERR_SEQLENS;
    for (int n = 0; n < p->N; ++n)
      if (cu[n + 1] < cu[n]) return GDN_ERR_SEQLENS;
  }
  const int64_t c = chunk_slots(p);
  if (c > (int64_t)INT32_MAX / 2 || (int64_t)p->N * p->HV > (int64_t)INT32_MAX / 64)
    return GDN_ERR_SHAPE;
  if (nc) *nc = c;
  return GDN_OK;
}

// Forward workspace: chunk table, then the forward scan's operands. Backward
// workspace: chunk table, then the scratch of the dh scan (its operands come
// from `saved`, written by the forward's WY pass).
Layout make_layout(const gdn_problem* p, int64_t NC, bool bwd) {
  Layout L;
  const size_t blocks = (size_t)p->HV * (size_t)NC;
  const size_t kblocks = (size_t)p->H * (size_t)NC;
  size_t off = 0;
  L.table = off;     off = align_up(off + sizeof(ChunkInfo) * (size_t)NC);
  L.seq_first = off; off = align_up(off + sizeof(int32_t) * (size_t)(p->N + 1));
  L.W = L.T = L.Qn = L.P = L.Kn = L.gL = L.gE = off;
  if (!bwd) {
    L.W = off;       off = align_up(off + 2 * kBlk64x128 * blocks);
    L.T = off;       off = align_up(off + 2 * 2 * kBlk64x64 * blocks);  // T (T^T's half unused)
    L.Qn = off;      off = align_up(off + 2 * kBlk64x128 * kblocks);
    L.P = off;       off = align_up(off + 2 * kBlk64x64 * blocks);
    L.Kn = off;      off = align_up(off + 2 * kBlk64x128 * kblocks);
    L.gL = off;      off = align_up(off + sizeof(float) * blocks);
    L.gE = off;      off = align_up(off + sizeof(float) * kGates * blocks);
  }
  L.dh = L.dD = L.dDT = off;
  if (bwd) {
    L.dh = off;      off = align_up(off + 2 * kState * blocks);
    L.dD = off;      off = align_up(off + 2 * kBlk64x128 * blocks);
    L.dDT = off;     off = align_up(off + 2 * kBlk64x128 * blocks);
  }
  L.total = off;
  return L;
}

PrepOut prep_views(char* ws, const Layout& L, const gdn_problem* p) {
  PrepOut o;
  o.W = reinterpret_cast<uint16_t*>(ws + L.W);
  o.T = reinterpret_cast<uint16_t*>(ws + L.T);
  o.Qn = reinterpret_cast<uint16_t*>(ws + L.Qn);
  o.P = reinterpret_cast<uint16_t*>(ws + L.P);
  o.Kn = reinterpret_cast<uint16_t*>(ws + L.Kn);
  o.gL = reinterpret_cast<float*>(ws + L.gL);
  o.gE = reinterpret_cast<float*>(ws + L.gE);
  o.gB = nullptr;
  o.G = p->HV / p->H;
  return o;
}

// `saved`: per (chunk, value head) the bf16 start state and D (kSavedBlock
// elements each); then the WY operands the forward scan reads and the
// backward reads again: per (value head, chunk) W [tok][k] (64 x 128) and
// P [i][j] (64 x 64), per (key head, chunk) Q~ [tok][k] and K^T [k][tok]
// (64 x 128 each); then per (value head, chunk) T and T^T (2 x 64 x 64, T
// read by both, T^T by the backward only); then in fp32 per (value head,
// chunk) e^gamma_L, the kGates gate factors (e^gamma, e^(gamma_L - gamma),
// beta), and the cumulative decay gamma (base 2) and beta (kGatesB).
// the gate factors start 16-byte aligned after the e^gamma_L values
size_t gates_offset(size_t blocks) { return (blocks + 3) / 4 * 4; }
size_t saved_bytes(const gdn_problem* p, int64_t NC) {
  const size_t blocks = (size_t)p->HV * (size_t)NC, kblocks = (size_t)p->H * (size_t)NC;
  return (blocks * ((size_t)kSavedBlock + kBlk64x128 + 3 * kBlk64x64) +
          kblocks * 2 * kBlk64x128) * 2 +
         (gates_offset(blocks) + blocks * (kGates + kGatesB)) * sizeof(float);
}
PrepOut saved_views(uint16_t* saved, const gdn_problem* p, int64_t NC) {
  const size_t blocks = (size_t)p->HV * (size_t)NC, kblocks = (size_t)p->H * (size_t)NC;
  PrepOut o;
  uint16_t* b = saved + blocks * (size_t)kSavedBlock;
  o.W = b;                              b += blocks * kBlk64x128;
  o.P = b;                              b += blocks * kBlk64x64;
  o.Qn = b;                             b += kblocks * kBlk64x128;
  o.Kn = b;                             b += kblocks * kBlk64x128;
  o.T = b;                              b += blocks * 2 * kBlk64x64;
  o.gL = reinterpret_cast<float*>(b);
  o.gE = o.gL + gates_offset(blocks);
  o.gB = o.gE + blocks * kGates;
  o.G = p->HV / p->H;
  return o;
}

// The forward's WY pass views when it saves for a backward: every operand the
// forward scan reads (W, T, P, Q~, K^T and the gate factors) goes to `saved`,
// which the backward reads again.
PrepOut forward_views_saving(PrepOut f, const PrepOut& sv) {
  f.W = sv.W;
  f.T = sv.T;
  f.P = sv.P;
  f.Qn = sv.Qn;
  f.Kn = sv.Kn;
  f.gL = sv.gL;
  f.gE = sv.gE;
  return f;
}

float effective_scale(const gdn_problem* p) {
  return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->K);
}

// Host copy of state-pool indices: every index in (0, slots) is active and
// must be distinct; an index >= slots is an error; <= 0 means "no slot".
gdn_status check_indices_host(int N, int slots, const int32_t* indices_host) {
  if (!indices_host) return GDN_OK;
  std::vector<int32_t> act;
  act.reserve(N);
  for (int n = 0; n < N; ++n) {
    const int32_t x = indices_host[n];
    if (x <= 0) continue;  // null block or negative: skipped, never an error
    if (x >= slots) return GDN_ERR_INDEX;
    act.push_back(x);
  }
  std::sort(act.begin(), act.end());
  if (std::adjacent_find(act.begin(), act.end()) != act.end()) return GDN_ERR_INDEX;
  return GDN_OK;
}

#define GDN_TRY(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return GDN_ERR_HIP;  \
  } while (0)

}  // namespace

GDN_API const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "a negative or inconsistent extent";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration (K = V = 128, chunk = 64, HV % H == 0)";
    case GDN_ERR_SEQLENS: return "cu_seqlens must start at 0, be non-decreasing and end at T";
    case GDN_ERR_INDEX: return "an active state index is out of range or repeated";
    case GDN_ERR_WORKSPACE: return "workspace missing or smaller than the size query";
    case GDN_ERR_HIP: return "a HIP launch failed";
    case GDN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case GDN_ERR_SCRATCH:
      return "the problem needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

GDN_API int64_t gdn_num_chunks(const gdn_problem* p) {
  int64_t nc = 0;
  return check_problem(p, &nc) == GDN_OK ? nc : 0;
}

GDN_API size_t gdn_chunk_saved_size(const gdn_problem* p) {
  int64_t nc = 0;
  if (check_problem(p, &nc) != GDN_OK) return 0;
  return saved_bytes(p, nc);
}

GDN_API size_t gdn_chunk_fwd_workspace_size(const gdn_problem* p) {
  int64_t nc = 0;
  if (check_problem(p, &nc) != GDN_OK) return 0;
  return make_layout(p, nc, false).total;
}

GDN_API size_t gdn_chunk_bwd_workspace_size(const gdn_problem* p) {
  int64_t nc = 0;
  if (check_problem(p, &nc) != GDN_OK) return 0;
  return make_layout(p, nc, true).total;
}

// The recomputing backward holds the forward's operands (forward layout, at
// the workspace's start), the rebuilt `saved` after the larger of the two
// layouts, and the backward's scratch (backward layout, at the start again,
// once the forward's operands are consumed).
static size_t recompute_saved_offset(const gdn_problem* p, int64_t nc) {
  return align_up(std::max(make_layout(p, nc, true).total, make_layout(p, nc, false).total));
}

GDN_API size_t gdn_chunk_bwd_recompute_workspace_size(const gdn_problem* p) {
  int64_t nc = 0;
  if (check_problem(p, &nc) != GDN_OK) return 0;
  return recompute_saved_offset(p, nc) + gdn_chunk_saved_size(p);
}

// Records events[2 i] / events[2 i + 1] around stage i when events are given
// (a NULL handle is skipped).
struct StageClock {
  void* const* ev;
  int n;
  hipStream_t s;
  template <typename F>
  hipError_t run(F&& launch) {
    if (ev && ev[2 * n] && hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * n]), s) != hipSuccess)
      return hipErrorUnknown;
    hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (ev && ev[2 * n + 1] &&
        hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * n + 1]), s) != hipSuccess)
      return hipErrorUnknown;
    ++n;
    return hipSuccess;
  }
};

// Argument checks of the forward (everything but the workspace).
static gdn_status check_fwd_args(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const float* g, const float* beta,
                                 const StateRef& sr, const uint16_t* o, const uint16_t* saved,
                                 int64_t* NC) {
  gdn_status st = check_problem(p, NC);
  if (st != GDN_OK) return st;
  if (p->T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(sr.h0) ||
      !aligned16(sr.hT) || !aligned16(saved))
    return GDN_ERR_ALIGN;
  return GDN_OK;
}

// Argument checks of the paged forward beyond those of the forward.
static gdn_status check_paged_args(const gdn_problem* p, float* state_pool, int32_t slots,
                                   const int32_t* ssm_state_indices,
                                   const int32_t* indices_host) {
  const gdn_status ps = check_problem(p, nullptr);
  if (ps != GDN_OK) return ps;
  if (slots < 0) return GDN_ERR_SHAPE;
  if (p->N > 0 && (!state_pool || !ssm_state_indices)) return GDN_ERR_NULL;
  if (check_indices_host(p->N, slots, indices_host) != GDN_OK) return GDN_ERR_INDEX;
  return GDN_OK;
}

static int chunk_fwd_impl(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* g, const float* beta,
                          const StateRef& sr, bool paged, uint16_t* o, uint16_t* saved,
                          void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events, int* n_stages) {
  if (n_stages) *n_stages = 0;
  int64_t NC = 0;
  gdn_status st = check_fwd_args(p, q, k, v, g, beta, sr, o, saved, &NC);
  if (st != GDN_OK) return st;
  if (!aligned16(workspace)) return GDN_ERR_ALIGN;
  const Layout L = make_layout(p, NC, false);
  if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  StageClock clk{events, 0, s};
  if (p->N == 0) return GDN_OK;  // no sequences: nothing to read or write
  if (p->T == 0 && !paged) {  // no tokens: the state passes through
    if (sr.hT)
      GDN_TRY(clk.run([&] {
        return launch_state_copy(sr.h0, sr.hT, (size_t)p->N * p->HV * kState, s);
      }));
    if (n_stages) *n_stages = clk.n;
    return GDN_OK;
  }
  char* ws = static_cast<char*>(workspace);
  ChunkInfo* table = reinterpret_cast<ChunkInfo*>(ws + L.table);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + L.seq_first);
  const PrepOut bprep = saved ? saved_views(saved, p, NC) : PrepOut{};
  const PrepOut prep =
      saved ? forward_views_saving(prep_views(ws, L, p), bprep) : prep_views(ws, L, p);
  GDN_TRY(clk.run([&] {
    return launch_chunk_table(p->cu_seqlens, p->N, p->T, (int)NC, table, seq_first, s);
  }));
  if (NC > 0)
    GDN_TRY(clk.run([&] {
      return launch_chunk_prep(saved ? PrepMode::kBoth : PrepMode::kForward, table, (int)NC, p->H,
                               p->HV, effective_scale(p), q, k, g, beta, prep, bprep, s);
    }));
  GDN_TRY(clk.run([&] {
    return launch_fwd_scan(saved ? ScanMode::kOutSave : ScanMode::kOut, seq_first, p->N, p->HV,
                           (int)NC, table, prep, v, sr, o, saved, s);
  }));
  if (n_stages) *n_stages = clk.n;
  return GDN_OK;
}

GDN_API int gdn_chunk_fwd(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* g, const float* beta, const float* h0,
                          uint16_t* o, float* hT, uint16_t* saved, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const StateRef sr{h0, hT, nullptr, nullptr, 0};
  return chunk_fwd_impl(p, q, k, v, g, beta, sr, false, o, saved, workspace, workspace_bytes,
                        stream, nullptr, nullptr);
}

GDN_API int gdn_chunk_fwd_paged(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const float* g, const float* beta,
                                float* state_pool, int32_t slots,
                                const int32_t* ssm_state_indices,
                                const int32_t* has_initial_state, const int32_t* indices_host,
                                uint16_t* o, uint16_t* saved, void* workspace,
                                size_t workspace_bytes, void* stream) {
  const gdn_status ps = check_paged_args(p, state_pool, slots, ssm_state_indices, indices_host);
  if (ps != GDN_OK) return ps;
  const StateRef sr{state_pool, state_pool, ssm_state_indices, has_initial_state, slots};
  return chunk_fwd_impl(p, q, k, v, g, beta, sr, true, o, saved, workspace, workspace_bytes,
                        stream, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// The allocation-free paged prefill: the same kernels with their workspace in
// a file-scope device array instead of a caller's buffer. Each GPU holds its
// own copy of the array from the library's first use on it until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// the device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
namespace {
constexpr size_t kScratchBytes = (size_t)96 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's scratch array, looked up on first use.
static hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

GDN_API size_t gdn_chunk_fwd_paged_noalloc_max_bytes(void) { return kScratchBytes; }

GDN_API int gdn_chunk_fwd_paged_noalloc(const gdn_problem* p, const uint16_t* q,
                                        const uint16_t* k, const uint16_t* v, const float* g,
                                        const float* beta, float* state_pool, int32_t slots,
                                        const int32_t* ssm_state_indices,
                                        const int32_t* has_initial_state,
                                        const int32_t* indices_host, uint16_t* o,
                                        uint16_t* saved, void* stream) {
  // every argument check first, so that an argument error touches no device
  const gdn_status ps = check_paged_args(p, state_pool, slots, ssm_state_indices, indices_host);
  if (ps != GDN_OK) return ps;
  int64_t NC = 0;
  const StateRef sr{state_pool, state_pool, ssm_state_indices, has_initial_state, slots};
  const gdn_status fs = check_fwd_args(p, q, k, v, g, beta, sr, o, saved, &NC);
  if (fs != GDN_OK) return fs;
  if (make_layout(p, NC, false).total > kScratchBytes) return GDN_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_for_current_device(&ws) != hipSuccess) return GDN_ERR_HIP;
  return gdn_chunk_fwd_paged(p, q, k, v, g, beta, state_pool, slots, ssm_state_indices,
                             has_initial_state, indices_host, o, saved, ws, kScratchBytes, stream);
}

GDN_API int gdn_chunk_fwd_timed(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const float* g, const float* beta,
                                const float* h0, uint16_t* o, float* hT, uint16_t* saved,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events, int* n_stages) {
  if (!events || !n_stages) return GDN_ERR_NULL;
  const StateRef sr{h0, hT, nullptr, nullptr, 0};
  return chunk_fwd_impl(p, q, k, v, g, beta, sr, false, o, saved, workspace, workspace_bytes,
                        stream, events, n_stages);
}

GDN_API int gdn_chunk_transition(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const float* g, const float* beta, float* M,
                                 float* s_end, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int64_t NC = 0;
  const gdn_status st = check_problem(p, &NC);
  if (st != GDN_OK) return st;
  if (p->T > 0 && (!q || !k || !v || !g || !beta)) return GDN_ERR_NULL;
  if (p->N > 0 && (!M || !s_end)) return GDN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(M) || !aligned16(s_end) ||
      !aligned16(workspace))
    return GDN_ERR_ALIGN;
  const Layout L = make_layout(p, NC, false);
  if (!workspace || workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (p->N == 0) return GDN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  ChunkInfo* table = reinterpret_cast<ChunkInfo*>(ws + L.table);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + L.seq_first);
  const PrepOut prep = prep_views(ws, L, p);
  if (launch_chunk_table(p->cu_seqlens, p->N, p->T, (int)NC, table, seq_first, s) != hipSuccess)
    return GDN_ERR_HIP;
  if (NC > 0 && launch_chunk_prep(PrepMode::kForward, table, (int)NC, p->H, p->HV,
                                  effective_scale(p), q, k, g, beta, prep, PrepOut{}, s) !=
                    hipSuccess)
    return GDN_ERR_HIP;
  StateRef sr{};
  sr.hT = s_end;
  sr.M = M;
  if (launch_fwd_scan(ScanMode::kTransition, seq_first, p->N, p->HV, (int)NC, table, prep, v, sr,
                      nullptr, nullptr, s) != hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}

// The backward; with recompute_h0 != nullptr (the recomputing form) it first
// reruns the forward scan from that start state to rebuild the saved states
// and D in the workspace, after the backward's own buffers.
static int chunk_bwd_impl(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* g, const float* beta,
                          const uint16_t* saved, const uint16_t* dO, const float* dhT,
                          uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, float* dbeta,
                          float* dh0, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* events, int* n_stages, bool recompute = false,
                          const float* recompute_h0 = nullptr) {
  if (n_stages) *n_stages = 0;
  int64_t NC = 0;
  gdn_status st = check_problem(p, &NC);
  if (st != GDN_OK) return st;
  if (p->T > 0 && (!q || !k || !v || !g || !beta || (!saved && !recompute) || !dO || !dq ||
                   !dk || !dv || !dg || !dbeta))
    return GDN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(saved) ||
      !aligned16(dO) || !aligned16(dhT) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dh0) || !aligned16(workspace) || !aligned16(recompute_h0))
    return GDN_ERR_ALIGN;
  const Layout L = make_layout(p, NC, true);
  const size_t need = recompute ? gdn_chunk_bwd_recompute_workspace_size(p) : L.total;
  if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  StageClock clk{events, 0, s};
  if (p->T == 0) {  // no tokens: the state cotangent passes through
    if (dh0)
      GDN_TRY(clk.run([&] { return launch_state_copy(dhT, dh0, (size_t)p->N * p->HV * kState, s); }));
    if (n_stages) *n_stages = clk.n;
    return GDN_OK;
  }
  char* ws = static_cast<char*>(workspace);
  ChunkInfo* table = reinterpret_cast<ChunkInfo*>(ws + L.table);
  int32_t* seq_first = reinterpret_cast<int32_t*>(ws + L.seq_first);
  BwdBufs bufs;
  bufs.dh = reinterpret_cast<uint16_t*>(ws + L.dh);
  bufs.dD = reinterpret_cast<uint16_t*>(ws + L.dD);
  bufs.dDT = reinterpret_cast<uint16_t*>(ws + L.dDT);
  const float scale = effective_scale(p);
  GDN_TRY(clk.run([&] {
    return launch_chunk_table(p->cu_seqlens, p->N, p->T, (int)NC, table, seq_first, s);
  }));
  if (recompute) {
    // the forward's WY pass (saving) and a save-only scan rebuild `saved`
    // after both workspace layouts; a saving WY pass writes all its operands
    // there, so the backward's scratch at the workspace's start is free
    uint16_t* rebuilt = reinterpret_cast<uint16_t*>(ws + recompute_saved_offset(p, NC));
    const PrepOut rv = saved_views(rebuilt, p, NC);
    const PrepOut fprep = forward_views_saving(prep_views(ws, make_layout(p, NC, false), p), rv);
    GDN_TRY(clk.run([&] {
      return launch_chunk_prep(PrepMode::kBoth, table, (int)NC, p->H, p->HV, scale, q, k, g,
                               beta, fprep, rv, s);
    }));
    StateRef sr{};
    sr.h0 = recompute_h0;
    GDN_TRY(clk.run([&] {
      return launch_fwd_scan(ScanMode::kSave, seq_first, p->N, p->HV, (int)NC, table, fprep, v, sr,
                             nullptr, rebuilt, s);
    }));
    saved = rebuilt;
  }
  // the WY operands were written by the forward, behind the states
  const PrepOut prep = saved_views(const_cast<uint16_t*>(saved), p, NC);
  GDN_TRY(clk.run([&] {
    return launch_bwd_dh_scan(seq_first, p->N, p->HV, (int)NC, table, prep, dO, dhT, dh0, bufs, s);
  }));
  GDN_TRY(clk.run([&] {
    return launch_bwd_chunk(table, (int)NC, p->H, p->HV, scale, q, k, v, g, beta, saved, prep.T,
                            prep.gE, prep.gB, bufs, dO, dq, dk, dv, dg, dbeta, s);
  }));
  if (n_stages) *n_stages = clk.n;
  return GDN_OK;
}

GDN_API int gdn_chunk_bwd(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, const float* g, const float* beta,
                          const uint16_t* saved, const uint16_t* dO, const float* dhT,
                          uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, float* dbeta,
                          float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(p, q, k, v, g, beta, saved, dO, dhT, dq, dk, dv, dg, dbeta, dh0, workspace,
                        workspace_bytes, stream, nullptr, nullptr);
}

GDN_API int gdn_chunk_bwd_recompute(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                    const uint16_t* v, const float* g, const float* beta,
                                    const float* h0, const uint16_t* dO, const float* dhT,
                                    uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg,
                                    float* dbeta, float* dh0, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return chunk_bwd_impl(p, q, k, v, g, beta, nullptr, dO, dhT, dq, dk, dv, dg, dbeta, dh0,
                        workspace, workspace_bytes, stream, nullptr, nullptr, true, h0);
}

GDN_API int gdn_chunk_bwd_timed(const gdn_problem* p, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const float* g, const float* beta,
                                const uint16_t* saved, const uint16_t* dO, const float* dhT,
                                uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg,
                                float* dbeta, float* dh0, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* events,
                                int* n_stages) {
  if (!events || !n_stages) return GDN_ERR_NULL;
  return chunk_bwd_impl(p, q, k, v, g, beta, saved, dO, dhT, dq, dk, dv, dg, dbeta, dh0, workspace,
                        workspace_bytes, stream, events, n_stages);
}

GDN_API const char* gdn_stage_name(int op, int stage) {
  static const char* fwd[] = {"chunk_table", "chunk_prep", "fwd_scan"};
  static const char* bwd[] = {"chunk_table", "bwd_dh_scan", "bwd_chunk"};
  if (op == 0 && stage >= 0 && stage < 3) return fwd[stage];
  if (op == 1 && stage >= 0 && stage < 3) return bwd[stage];
  return "";
}

GDN_API int gdn_recurrent_step(int32_t N, int32_t H, int32_t HV, int32_t K, int32_t V, float scale,
                               const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* a, const uint16_t* b, const float* A_log,
                               const float* dt_bias, float* state_pool, int32_t slots,
                               const int32_t* ssm_state_indices, const int32_t* indices_host,
                               uint16_t* o, void* stream) {
  if (N < 0 || H <= 0 || HV <= 0 || K <= 0 || V <= 0 || slots < 0) return GDN_ERR_SHAPE;
  if (K != kHead || V != kHead || HV % H != 0) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)N * HV > (int64_t)INT32_MAX) return GDN_ERR_SHAPE;
  if (N == 0) return GDN_OK;
  if (!q || !k || !v || !a || !b || !A_log || !state_pool || !ssm_state_indices || !o)
    return GDN_ERR_NULL;
  if (!aligned16(state_pool) || !aligned16(o) || ((uintptr_t)q & 3u) || ((uintptr_t)k & 3u))
    return GDN_ERR_ALIGN;
  if (check_indices_host(N, slots, indices_host) != GDN_OK) return GDN_ERR_INDEX;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)K);
  if (launch_decode_step(N, H, HV, sc, q, k, v, a, b, A_log, dt_bias, state_pool, slots,
                         ssm_state_indices, o, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return GDN_ERR_HIP;
  return GDN_OK;
}
