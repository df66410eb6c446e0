/*
 * gdn.h - C ABI of the gated delta rule library for MI355X (gfx950).
 *
 * The library computes the chunked gated delta rule, forward and backward,
 * and its one-token recurrent decode step, on one GPU, with hand-written HIP
 * kernels. Per sequence and value head the state S is a V x K fp32 matrix:
 *
 *   S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t,
 *
 * where q and k are first divided by sqrt(sum(x*x) + 1e-6) in fp32, q is then
 * multiplied by `scale` (K^-1/2 by default) and k is never scaled, and value
 * head hv reads key head hv / (HV / H). Sources:
 *   - the recurrence, the norm, the scale, the head grouping and the decode
 *     gating: RL-Kernel PR #469 "[WS1][CUDA][Qwen3-Next] C6: GDN decode-step
 *     goldens and recurrent/conv state contract", "What" section and the
 *     agent note on where the kernel and the HF model disagree;
 *   - the chunk contract (chunk 64, K = V = 128, bf16 q/k/v, fp32 g/beta,
 *     varlen packing by cu_seqlens, in-kernel L2 norm, a call without tokens
 *     passes the state through, extents checked before any launch):
 *     "[Cake 1/13] gdn" (miles-ext-kernels PR #1), "API and flags" and
 *     "Review items";
 *   - the precision and determinism contract (fp32 running state across
 *     chunks, per-chunk state stored bf16, no device atomics, repeated runs
 *     bit-identical): "cake_gdn: deterministic chunked GDN training kernels"
 *     (miles PR #3597), "Summary".
 *
 * Conventions for every entry point
 *   - bf16 tensors are passed as uint16_t pointers holding bf16 bit patterns;
 *     fp32 as float; indices as int32_t. All tensors are dense, row-major,
 *     in the layouts stated per argument. Pointers are device pointers unless
 *     the name ends in _host.
 *   - `stream` is a hipStream_t (NULL: the null stream). Work is enqueued on
 *     it and the call returns without synchronising.
 *   - The caller owns every buffer. The library allocates nothing, frees
 *     nothing and keeps no state between calls; calls on different streams
 *     with disjoint buffers may run concurrently.
 *   - Every argument error is returned before anything is enqueued. A launch
 *     failure returns GDN_ERR_HIP; the outputs are then undefined.
 *   - Tensor and workspace pointers must be 16-byte aligned (the decode q and
 *     k rows 4-byte aligned), else GDN_ERR_ALIGN. Token tensors may be NULL
 *     when T = 0.
 *   - No kernel uses atomics: identical inputs, shapes and device give
 *     bit-identical outputs.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                         */
  GDN_ERR_SHAPE = 2,       /* a negative or inconsistent extent                  */
  GDN_ERR_UNSUPPORTED = 3, /* K or V != 128, chunk != 64, HV % H != 0            */
  GDN_ERR_SEQLENS = 4,     /* cu_seqlens_host not 0 .. T and non-decreasing      */
  GDN_ERR_INDEX = 5,       /* an active state-pool index >= slots, or repeated   */
  GDN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the size query      */
  GDN_ERR_HIP = 7,         /* a HIP launch failed                                */
  GDN_ERR_ALIGN = 8,       /* a tensor or workspace pointer not 16-byte aligned  */
  GDN_ERR_SCRATCH = 9      /* too large for the allocation-free entry point      */
} gdn_status;

/* Human-readable text of a status code; never NULL. */
const char* gdn_status_string(int status);

/* Problem description of one chunk call (forward or backward).
 *   N      number of sequences packed along the token axis (N >= 0)
 *   T      total tokens (T >= 0)
 *   H      key heads of q and k; HV value heads of v, o, g, beta (HV % H == 0)
 *   K, V   head dims, both 128
 *   chunk  64
 *   scale  multiplier of q after its norm; <= 0 selects K^-1/2
 *   cu_seqlens       device int32 [N+1]: sequence n owns tokens
 *                    [cu[n], cu[n+1]). Read by the kernels, never copied to
 *                    the host (no device-to-host synchronisation).
 *   cu_seqlens_host  optional host copy of the same boundaries. When given,
 *                    it is validated (0 = cu[0] <= ... <= cu[N] = T) before
 *                    any launch. Device boundaries that are not monotone or
 *                    leave [0, T] are clamped, never dereferenced out of
 *                    range.
 * Chunks restart at every sequence start; the last chunk of a sequence may be
 * shorter than 64. Chunks are numbered sequence by sequence in token order;
 * chunk c of the pack is the slot index used by the saved buffer. */
typedef struct {
  int32_t N, T, H, HV, K, V, chunk;
  float scale;
  const int32_t* cu_seqlens;
  const int32_t* cu_seqlens_host;
} gdn_problem;

/* Number of chunk slots the chunk calls index: the bound T/64 + N on the sum
 * of ceil(L_n / 64), whether or not cu_seqlens_host is given, so that every
 * size query below depends on (N, T, H, HV) only and a `saved` buffer written
 * by a forward always has the layout its backward expects. Slots past the
 * pack's chunks are skipped by the kernels. 0 on a bad problem. */
int64_t gdn_num_chunks(const gdn_problem* p);

/* Bytes of the `saved` buffer that gdn_chunk_fwd fills for gdn_chunk_bwd
 * (0 on a bad problem). */
size_t gdn_chunk_saved_size(const gdn_problem* p);

/* Workspace bytes needed by gdn_chunk_fwd / gdn_chunk_bwd for this problem
 * (0 on a bad problem). The workspace is caller-allocated device memory,
 * 256-byte aligned, used only during the call, and need not be zeroed. */
size_t gdn_chunk_fwd_workspace_size(const gdn_problem* p);
size_t gdn_chunk_bwd_workspace_size(const gdn_problem* p);
/* Workspace bytes of gdn_chunk_bwd_recompute: the backward's workspace plus
 * room for the per-chunk states it rebuilds (gdn_chunk_saved_size). */
size_t gdn_chunk_bwd_recompute_workspace_size(const gdn_problem* p);

/* Chunked forward.
 *   q, k      bf16 [T, H, K]
 *   v         bf16 [T, HV, V]
 *   g         fp32 [T, HV]  log-decay (exp(g) multiplies the state)
 *   beta      fp32 [T, HV]  write strength (already passed through a sigmoid)
 *   h0        fp32 [N, HV, V, K] initial states, or NULL for zero states
 *   o         bf16 [T, HV, V] output (written)
 *   hT        fp32 [N, HV, V, K] final states, or NULL to skip
 *   saved     gdn_chunk_saved_size(p) bytes kept for gdn_chunk_bwd, or NULL
 *             when no backward follows. For chunk slot c and value head hv
 *             the block at element offset (c * HV + hv) * (K*V + 64*V) holds
 *             the chunk's start state (the fp32 running state rounded to
 *             nearest-even bf16) and then the chunk's 64 x V corrected
 *             values D = U - W h in bf16 (rows past the chunk's end are
 *             zero); after all those blocks come the chunk quantities the
 *             backward contracts with (W, P, T in bf16 per value head and
 *             chunk; the normalised q and k in bf16 per key head and chunk;
 *             e^gamma_L, the per-token factors e^gamma, e^(gamma_L - gamma)
 *             and beta, and the cumulative decay gamma with beta again, in
 *             fp32 per value head and chunk), written by the same WY pass
 *             that feeds the forward scan so that the backward does not form
 *             them again. All in tile orders internal to this library: only
 *             gdn_chunk_bwd of the same build reads them.
 * A sequence of length 0 gets hT = h0 (or 0). T = 0 is valid: nothing is
 * read from the token tensors and hT = h0 (or 0).
 * Errors: GDN_ERR_NULL (p, or q, k, v, g, beta, o, cu_seqlens when T > 0),
 * GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS,
 * GDN_ERR_WORKSPACE, GDN_ERR_ALIGN, GDN_ERR_HIP. */
int gdn_chunk_fwd(const gdn_problem* p,
                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const float* g, const float* beta, const float* h0,
                  uint16_t* o, float* hT, uint16_t* saved,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Chunked forward (prefill) whose start and end states live in a state pool,
 * updated in place: the paged prefill of a serving stack, sharing the pool
 * [slots, HV, V, K] of gdn_recurrent_step, without gather / scatter copies.
 * The torchtitan PR #4389 page (the serving-path and paged-state continuity
 * sections) describes a serving path whose cache slots are advanced in place
 * and checks that a prefix resumed from its slot continues the sequence.
 * Same p, q, k, v, g, beta, o, saved and workspace as gdn_chunk_fwd, and:
 *   state_pool fp32 [slots, HV, V, K]
 *   ssm_state_indices int32 [N] (device): sequence n reads and writes block
 *             ssm_state_indices[n]. An index <= 0 (0 is the null block), or
 *             one >= slots, gives the sequence no block: it starts from a
 *             zero state and its end state is not written anywhere.
 *   has_initial_state int32 [N] (device) or NULL: a sequence with a block
 *             starts from the block's contents when the flag is nonzero (a
 *             resumed prefix) and from zero when it is 0 (a fresh prompt);
 *             NULL resumes every sequence. Its end state replaces the block.
 *   indices_host optional host copy of the indices, validated as for
 *             gdn_recurrent_step (GDN_ERR_INDEX); without it the caller
 *             guarantees that active indices are distinct.
 * A sequence of length 0 leaves a resumed block unchanged and zeroes a fresh
 * one. Every other block of the pool is neither read nor written. The results
 * (o, the end states, saved) equal gdn_chunk_fwd with h0 / hT gathered from
 * and scattered to the pool, bit for bit.
 * Errors: those of gdn_chunk_fwd, GDN_ERR_NULL for state_pool or
 * ssm_state_indices when N > 0, GDN_ERR_SHAPE for slots < 0, GDN_ERR_INDEX. */
int gdn_chunk_fwd_paged(const gdn_problem* p,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta,
                        float* state_pool, int32_t slots,
                        const int32_t* ssm_state_indices, const int32_t* has_initial_state,
                        const int32_t* indices_host,
                        uint16_t* o, uint16_t* saved,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The paged prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, results and errors as
 * gdn_chunk_fwd_paged minus `workspace` / `workspace_bytes`: the kernels use a
 * scratch array inside the library instead, of
 * gdn_chunk_fwd_paged_noalloc_max_bytes() bytes (96 MiB) per GPU, held from
 * the first call on a GPU until the process ends. A problem whose
 * gdn_chunk_fwd_workspace_size exceeds that returns GDN_ERR_SCRATCH before any
 * launch (for example 16 value / 8 key heads fit 8 x 512 tokens; the limit
 * scales with (T / 64 + N) x (HV x 40.5 KiB + H x 32 KiB)). The call allocates
 * nothing (no hipMalloc, no allocating library routine); its first call on a
 * GPU looks the array's device address up once. Every call on one GPU shares
 * that GPU's array: calls that may overlap on one GPU (different streams,
 * different host threads) race and must be serialised by the caller. Nothing
 * in the array needs to start at zero. */
size_t gdn_chunk_fwd_paged_noalloc_max_bytes(void);
int gdn_chunk_fwd_paged_noalloc(const gdn_problem* p,
                                const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* g, const float* beta,
                                float* state_pool, int32_t slots,
                                const int32_t* ssm_state_indices,
                                const int32_t* has_initial_state,
                                const int32_t* indices_host,
                                uint16_t* o, uint16_t* saved, void* stream);

/* Chunked backward of gdn_chunk_fwd (same p, q, k, v, g, beta).
 *   saved     as written by gdn_chunk_fwd for the same problem and inputs
 *   dO        bf16 [T, HV, V] cotangent of o
 *   dhT       fp32 [N, HV, V, K] cotangent of hT, or NULL for zero
 *   dq, dk    bf16 [T, H, K]; dv bf16 [T, HV, V]; dg, dbeta fp32 [T, HV]
 *   dh0       fp32 [N, HV, V, K] cotangent of h0, or NULL to skip
 * The value heads of one key head are summed into dq, dk in a fixed order.
 * No atomics: repeated calls on identical inputs give identical bits. */
int gdn_chunk_bwd(const gdn_problem* p,
                  const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const float* g, const float* beta,
                  const uint16_t* saved, const uint16_t* dO, const float* dhT,
                  uint16_t* dq, uint16_t* dk, uint16_t* dv,
                  float* dg, float* dbeta, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Backward that recomputes the per-chunk states instead of reading them from
 * a `saved` buffer (the recompute-state form of the Cake page "[Cake 1/13]
 * gdn", miles-ext-kernels PR #1, variant routing and its recompute-state
 * switch): the forward then needs no `saved` buffer at all. Same arguments as
 * gdn_chunk_bwd with `saved` replaced by
 *   h0        fp32 [N, HV, V, K] the forward's initial states, or NULL (zero)
 * and a workspace of gdn_chunk_bwd_recompute_workspace_size(p) bytes. It
 * reruns the forward's WY pass and state scan (without the output) into the
 * workspace, then runs the backward; the gradients equal those of
 * gdn_chunk_fwd(saved) + gdn_chunk_bwd bit for bit.
 * Errors: as gdn_chunk_bwd. */
int gdn_chunk_bwd_recompute(const gdn_problem* p,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const float* h0,
                            const uint16_t* dO, const float* dhT,
                            uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            float* dg, float* dbeta, float* dh0,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Local transition of each sequence of the pack: the piece of a context-
 * parallel forward that one GPU computes on its share of a long sequence
 * (the maxtext page "Qwen3.5-397B RL trainer on 128 v7x", the commit adding
 * the gdn_cp_m_scan forward transition product: the product of the chunk
 * transitions e^gamma_L I - K_bwd^T W, and the end state from a zero start).
 * For every start state S_0 [V, K] the sequence's end state is
 *   S_end = S_0 M + s
 * with
 *   M         fp32 [N, HV, K, K] (row j, column k: M[n][hv][j][k])
 *   s         fp32 [N, HV, V, K] the end state from S_0 = 0
 * both written, never read. A length-0 sequence gets M = I and s = 0. Same
 * p, q, k, v, g, beta and workspace (gdn_chunk_fwd_workspace_size) as
 * gdn_chunk_fwd; no output o is produced. A rank of a context-parallel run
 * combines the (M, s) of the ranks before it into its start state and then
 * calls gdn_chunk_fwd from that state; the backward mirrors it with
 * gdn_chunk_bwd, whose dh0 is linear in dhT (dh0 = dhT M^T + dh0 at dhT = 0).
 * Errors: GDN_ERR_NULL (p, q, k, v, g, beta when T > 0, M and s when N > 0),
 * GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS,
 * GDN_ERR_WORKSPACE, GDN_ERR_ALIGN, GDN_ERR_HIP. */
int gdn_chunk_transition(const gdn_problem* p,
                         const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const float* g, const float* beta,
                         float* M, float* s,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing, for measurement tools. Same as gdn_chunk_fwd /
 * gdn_chunk_bwd, plus `events`: 2 * GDN_MAX_STAGES hipEvent_t handles created
 * by the caller (hipEventCreate). The library records events[2 i] before and
 * events[2 i + 1] after launching stage i on `stream` and stores the number of
 * stages it launched in *n_stages; gdn_stage_name(op, i) names stage i
 * (op 0: forward, 1: backward; "" past the last stage). A NULL handle in
 * `events` is not recorded, so that a caller can time one stage without
 * markers between the others. Results are the same bits as the untimed calls.
 * GDN_ERR_NULL if events or n_stages is NULL. */
#define GDN_MAX_STAGES 8
int gdn_chunk_fwd_timed(const gdn_problem* p,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta, const float* h0,
                        uint16_t* o, float* hT, uint16_t* saved,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const* events, int* n_stages);
int gdn_chunk_bwd_timed(const gdn_problem* p,
                        const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* g, const float* beta,
                        const uint16_t* saved, const uint16_t* dO, const float* dhT,
                        uint16_t* dq, uint16_t* dk, uint16_t* dv,
                        float* dg, float* dbeta, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const* events, int* n_stages);
const char* gdn_stage_name(int op, int stage);

/* One recurrent decode step, in place on a state pool.
 *   N rows (requests), one token each; H, HV, K = V = 128 as above.
 *   q, k      bf16 [N, H, K];  v bf16 [N, HV, V]
 *   a, b      bf16 [N, HV]: beta = sigmoid(b) and
 *             g = -exp(A_log) * softplus(a + dt_bias), in fp32, with
 *             softplus(x) = x for x > 20 and log(1 + e^x) otherwise
 *   A_log     fp32 [HV];  dt_bias fp32 [HV] or NULL for zero
 *   state_pool fp32 [slots, HV, V, K], updated in place
 *   ssm_state_indices int32 [N] (device): row n updates block
 *             ssm_state_indices[n]. An index <= 0 (0 is the null block) skips
 *             the row: its o row is written as zeros and no state block is
 *             read or written. The kernel also skips an index >= slots
 *             instead of dereferencing it.
 *   indices_host optional host copy of the indices: when given, an active
 *             index >= slots or an active index used by two rows returns
 *             GDN_ERR_INDEX before any launch. Without it the caller
 *             guarantees that active indices are distinct.
 *   o         bf16 [N, HV, V] (written)
 * Each (row, value head) is computed alone, so a row's output and state do
 * not depend on the other rows of the batch.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_INDEX,
 * GDN_ERR_ALIGN, GDN_ERR_HIP. N = 0 is valid and enqueues nothing. */
int gdn_recurrent_step(int32_t N, int32_t H, int32_t HV, int32_t K, int32_t V, float scale,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint16_t* a, const uint16_t* b,
                       const float* A_log, const float* dt_bias,
                       float* state_pool, int32_t slots,
                       const int32_t* ssm_state_indices, const int32_t* indices_host,
                       uint16_t* o, void* stream);

/* ---------------------------------------------------------------------------
 * Causal short convolution (the depthwise convolution in front of the gated
 * delta rule). Per channel c of C, for the tokens of each sequence preceded by
 * its W - 1 carried inputs xe (the conv state, zero when none is given):
 *   pre_t = bias[c] + sum_{i<W} weight[c][i] * xe[t - (W - 1) + i]
 *   y_t   = silu(pre_t) = pre_t / (1 + e^-pre_t)   (activation 1) or pre_t (0)
 * accumulated in fp32 from the bf16 inputs, y rounded to bf16. The state of a
 * sequence is its last W - 1 inputs, [C, W - 1] in bf16. Definitions: the
 * goldens page ("[WS1][CUDA][Qwen3-Next] C6: GDN decode-step goldens and
 * recurrent/conv state contract", RL-Kernel PR #469, "What": the conv update
 * golden with bias and SiLU, the state [num_blocks, dim, W - 1], the null
 * block 0 and the error on a negative index); the cake_gdn page (miles PR
 * #3597) for a conv weight gradient without atomics; the torchtitan PR #4389
 * page for the paged convolution prefill.
 * Layouts: x, y, dy, dx bf16 [T, C] (row-major, token rows); weight bf16
 * [C, W]; bias bf16 [C] or NULL; states bf16 [N or slots, C, W - 1].
 * Supported: 2 <= W <= 4, C a multiple of 4 (GDN_ERR_UNSUPPORTED otherwise).
 * Token tensors must be 8-byte aligned (GDN_ERR_ALIGN). */
typedef struct {
  int32_t N;            /* sequences                                         */
  int32_t T;            /* total tokens                                      */
  int32_t C;            /* channels                                          */
  int32_t W;            /* filter width                                      */
  int32_t activation;   /* 0 none, 1 SiLU                                    */
  const int32_t* cu_seqlens;       /* device [N + 1]                         */
  const int32_t* cu_seqlens_host;  /* optional host copy, validated          */
} gdn_conv_problem;

/* Varlen forward. state_in [N, C, W - 1] or NULL (zero start); state_out
 * [N, C, W - 1] or NULL (not written): each sequence's last W - 1 inputs,
 * reaching into state_in when the sequence is shorter than W - 1.
 * Errors: GDN_ERR_NULL (p, weight; x, y, cu_seqlens when T > 0),
 * GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_SEQLENS, GDN_ERR_ALIGN,
 * GDN_ERR_HIP. */
int gdn_conv_fwd(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                 const uint16_t* bias, const uint16_t* state_in, uint16_t* y,
                 uint16_t* state_out, void* stream);

/* Paged forward: the carried inputs come from, and the end states go back to,
 * blocks of state_pool [slots, C, W - 1] (in place). Sequence n uses block
 * indices[n] (device int32 [N]); index 0 is the null block: zero start,
 * nothing written. has_initial_state (device int32 [N], nullable: all
 * resume) selects a resumed (nonzero) or fresh (0, zero start) sequence.
 * indices_host, optional: validated (GDN_ERR_INDEX for a negative index, one
 * >= slots, or an active index used twice); without it the caller guarantees
 * that, and a bad index is treated as the null block. Results equal
 * gdn_conv_fwd with the states gathered and scattered, bit for bit.
 * Errors: as gdn_conv_fwd, GDN_ERR_NULL for state_pool or indices when
 * N > 0, GDN_ERR_SHAPE for slots < 0, GDN_ERR_INDEX. */
int gdn_conv_fwd_paged(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                       const uint16_t* bias, uint16_t* state_pool, int32_t slots,
                       const int32_t* indices, const int32_t* has_initial_state,
                       const int32_t* indices_host, uint16_t* y, void* stream);

/* Workspace bytes of gdn_conv_bwd (0 on a bad problem). */
size_t gdn_conv_bwd_workspace_size(const gdn_conv_problem* p);

/* Backward of gdn_conv_fwd (same p, x, weight, bias, state_in):
 *   dy        bf16 [T, C] cotangent of y
 *   dx        bf16 [T, C]
 *   dweight   fp32 [C, W]
 *   dbias     fp32 [C] or NULL
 *   dstate_in fp32 [N, C, W - 1] cotangent of state_in, or NULL
 * The weight and bias gradients are sums over all tokens taken in a fixed
 * order (per-tile partial sums, then two ordered passes): no atomics, the
 * same bits on every call. Workspace: gdn_conv_bwd_workspace_size bytes,
 * 16-byte aligned. Errors: as gdn_conv_fwd, GDN_ERR_NULL for dweight (and dy,
 * dx when T > 0), GDN_ERR_WORKSPACE. */
int gdn_conv_bwd(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                 const uint16_t* bias, const uint16_t* state_in, const uint16_t* dy,
                 uint16_t* dx, float* dweight, float* dbias, float* dstate_in,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Decode update: one token per row. x [N, C] bf16; row n uses block
 * indices[n] of state_pool [slots, C, W - 1] (device int32 [N]): y_n from
 * the block's W - 1 inputs and x_n, then the block shifts by one input (x_n
 * enters last), in place. Index 0 (the null block): zero output row, no
 * block touched. indices_host as for gdn_conv_fwd_paged. N = 0 is valid.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_INDEX,
 * GDN_ERR_ALIGN, GDN_ERR_HIP. */
int gdn_conv_update(int32_t N, int32_t C, int32_t W, int32_t activation, const uint16_t* x,
                    const uint16_t* weight, const uint16_t* bias, uint16_t* state_pool,
                    int32_t slots, const int32_t* indices, const int32_t* indices_host,
                    uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
