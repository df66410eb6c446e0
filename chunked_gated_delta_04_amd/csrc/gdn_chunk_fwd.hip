// Forward state scan with the fused output of the chunked gated delta rule.
//
// Per chunk, with h = S^T the K x V start state (fp32, kept in registers):
//   U  = T diag(beta) V              (no state needed: formed here from the
//                                     WY pass's T and the raw value rows)
//   D  = U - W h                     corrected values of the chunk
//   O  = Q_g h + P D                 inter-chunk plus intra-chunk output
//   h <- e^gamma_L h + K_bwd^T D     state at the next chunk's start
// where Q_g = diag(e^gamma) Q~ and K_bwd = diag(e^(gamma_L - gamma)) K^: the
// scan reads the key head's Q~ and K^ (shared by its value heads) and applies
// the per-token decays in fp32, to the rows of Q~ h and to the rows of D.
// (the chunk form of the recurrence; the scan and the output are the
// forward stages named on the cake_gdn page, miles PR #3597, "What the
// commits add"; the start state of every chunk is stored in bf16 for the
// backward while the running state stays fp32, as its "Summary" requires).
// For the backward each chunk also saves D, so that the gradient kernel
// never has to rebuild it from the other layout of the state.
//
// The columns of the state (value dims) evolve independently, so one chain
// (sequence, value head) is split into 128/VB value blocks, each its own
// workgroup: with VB = 32 a 4 x 4096 pack at 32 value heads launches 512
// workgroups. Block b runs on XCD b % 8; the value blocks of one chain get
// the same b % 8 so they share that XCD's L2 for the chunk operands they all
// read. All operands come straight from global memory in MFMA fragment
// layout (16 bytes per lane per operand); only S (bf16), D and the block's
// value rows (scaled by beta, contracted over the chunk's tokens, so read as
// columns with transposing reads) pass through LDS.
//
// Transition mode (one GPU's share of a context-parallel forward): the end
// state is affine in the start state, h_end = M_h h_0 + s, and the chunk map
// is h -> (e^gamma_L I - K_bwd^T W) h + K_bwd^T U (the chunk transition of the
// maxtext page "Qwen3.5-397B RL trainer on 128 v7x", its gdn_cp_m_scan
// commit). M_h is the same scan run on a K x K "state" that starts at the
// identity with U = 0, and s the ordinary scan from zero; the launch runs both
// as 2 x 128/VB value blocks per chain and writes M_h transposed, i.e. the
// matrix M with S_end = S_0 M + s in the S = h^T layout of the states.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <bool kSave, bool kOut, bool kTrans>
__global__ __launch_bounds__(256) void fwd_scan_kernel(
    const int32_t* __restrict__ seq_first, int N, int HV, int NC,
    const ChunkInfo* __restrict__ table, PrepOut prep, const uint16_t* __restrict__ v,
    StateRef st,
    uint16_t* __restrict__ o, uint16_t* __restrict__ saved) {
  constexpr int VB = kScanVB;
  constexpr int NVB = kHead / VB;  // value blocks per head
  constexpr int VT = VB / 16;      // 16-wide value tiles per block
  constexpr int SP = 136;          // LDS pitch of S rows (bf16)
  constexpr int DP = 72;           // LDS pitch of D^T rows (bf16)
  constexpr int VP = VB + 8;       // LDS pitch of the beta-scaled value rows (bf16)

  constexpr int NVBL = kTrans ? 2 * NVB : NVB;  // blocks per chain
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int vb = slot % NVB;
  const bool mblk = kTrans && slot % NVBL < NVB;  // a block of M's columns
  // the value heads of one key head (consecutive chains) share an XCD too,
  // so the key head's Q~ and K^ tiles they all read come from one L2
  const int m = slot / NVBL, G = prep.G;
  const int chain = ((m / G) * 8 + xcd) * G + m % G;
  if (chain >= N * HV) return;
  const int seq = chain / HV, hv = chain - seq * HV;
  const int v0 = vb * VB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;

  __shared__ __align__(16) uint16_t Ss[VB * SP];  // S[v][k] of the chunk start (bf16)
  __shared__ __align__(16) uint16_t Ds[VB * DP];  // D^T[v][tok] (bf16)
  __shared__ __align__(16) uint16_t Es[VB * DP];  // (diag(e^(gamma_L - gamma)) D)^T (bf16)
  __shared__ __align__(16) uint16_t Vs[kChunk * VP];  // diag(beta) V [tok][v - v0] (bf16)

  // start and end state of this chain (the paged form reads and writes one
  // pool slot in place: each thread reads its own elements before the scan
  // and writes the same elements after it)
  const float* h0 = st.h0;
  float* hT = st.hT;
  size_t state_base = ((size_t)seq * HV + hv) * kHead * kHead;
  if (st.idx) {
    const int sl = st.idx[seq];
    const bool live = sl > 0 && sl < st.slots;
    state_base = live ? ((size_t)sl * HV + hv) * kHead * kHead : 0;
    h0 = live && (!st.init || st.init[seq] != 0) ? st.h0 : nullptr;
    hT = live ? st.hT : nullptr;
  }

  // h[dt][vt][r] = h[k = 16 (2 wave + dt) + 4 kq + r][v = v0 + 16 vt + li]
  f32x4 h[2][VT];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      const int kk = 16 * (2 * wave + dt) + 4 * kq;
      const int vv = v0 + 16 * vt + li;
      if constexpr (kTrans) {
        h[dt][vt] = zero4();
        if (mblk) {
#pragma unroll
          for (int r = 0; r < 4; ++r) h[dt][vt][r] = kk + r == vv ? 1.f : 0.f;
        }
      } else if (h0) {
        const float4 x = *reinterpret_cast<const float4*>(h0 + state_base + (size_t)vv * kHead + kk);
        h[dt][vt] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        h[dt][vt] = zero4();
      }
    }

  // The chunks of one sequence are consecutive 64-token pieces, so a chunk's
  // first token and length follow from the sequence's bounds without a table
  // read on the chain's critical path.
  const int c_begin = seq_first[seq], c_end = seq_first[seq + 1];
  int bos = 0, eos = 0;
  if (c_begin < c_end) {
    const ChunkInfo first = table[c_begin], lastc = table[c_end - 1];
    bos = first.t0;
    eos = lastc.t0 + lastc.len;
  }

  // Operands of one chunk in MFMA fragment layout. Two sets alternate: the
  // next chunk's set is requested before the current chunk computes. Every
  // chunk issues the same number of loads and stores, with no branch around
  // any of them, so the wait for a set counts exactly the memory operations
  // issued after it and never waits for a store to finish.
  struct Ops {
    uint4 vr;    // value row piece: token tid / 4, columns v0 + 8 (tid % 4) .. + 7
    float bt;    // beta of that token
    bf16x8 wa[4], qa[4], pa[2], ka[2][2], ta[2];
    float gl;
    float eg;    // e^gamma of token 16 wave + li (output rows)
    float4 ebw;  // e^(gamma_L - gamma) of tokens 16 wave + 4 kq .. + 3 (D rows)
    uint32_t pf;  // L2 warm-up word of a later chunk (see touch_line)
  };
  // This workgroup's share of a chunk's operand lines for the L2 warm-up: the
  // value head's W lines (128), the stored lines of T and P (40 each), its gate
  // factors (6) and value rows (128), split over its value blocks, and the key
  // head's Q~ and K^T lines (256) over the workgroups of all its value heads.
  // Lanes past the share all touch its first line (one request per wave
  // instruction, the lanes' addresses being the same).
  const int vshare = (kTrans ? 2 * NVB : NVB);
  const int vpos = kTrans ? slot % NVBL : vb;
  const int vlines = (342 + vshare - 1) / vshare;
  const int kshares = NVBL * prep.G, kpos = (hv % prep.G) * NVBL + vpos;
  const int klines = (256 + kshares - 1) / kshares;
  auto warm_line = [&](int c) -> const void* {
    const size_t blk = (size_t)hv * NC + c;
    const size_t kblk = (size_t)(hv / prep.G) * NC + c;
    int i = tid < vlines + klines ? tid : 0;
    if (i < vlines) {
      const int l = min(vpos * vlines + i, 341);
      if (l < 128) return prep.W + blk * 8192 + l * kLineElems16;
      if (l < 168) return prep.T + blk * 8192 + lower_tile_line(l - 128) * kLineElems16;
      if (l < 208) return kOut ? (const void*)(prep.P + blk * 4096 + lower_tile_line(l - 168) * kLineElems16)
                               : (const void*)(prep.W + blk * 8192);
      if (l < 214) return prep.gE + blk * kGates + (l - 208) * kLineElems32;
      // value rows: token (l - 214) / 2, half (l - 214) % 2 of its 256 bytes
      const int t0 = bos + (c - c_begin) * kChunk, len = min(kChunk, eos - t0);
      const int tok = (l - 214) >> 1;
      return v + ((size_t)(t0 + (tok < len ? tok : 0)) * HV + hv) * kHead + 64 * ((l - 214) & 1);
    }
    const int l = min(kpos * klines + (i - vlines), 255);
    if (l < 128) return kOut ? (const void*)(prep.Qn + kblk * 8192 + l * kLineElems16)
                             : (const void*)(prep.Kn + kblk * 8192);
    return prep.Kn + kblk * 8192 + (l - 128) * kLineElems16;
  };
  uint32_t sink = 0;
  // pc: the chunk whose lines the set's L2 warm-up word touches
  auto load_ops = [&](int c, Ops& x, int pc) {
    const size_t blk = (size_t)hv * NC + c;
    const size_t kblk = (size_t)(hv / prep.G) * NC + c;
    const uint16_t* Wb = prep.W + blk * 8192;
    const uint16_t* Qb = prep.Qn + kblk * 8192;  // Q~ [tok][k]
    const uint16_t* Pb = prep.P + blk * 4096;
    const uint16_t* Kb = prep.Kn + kblk * 8192;  // K^T [k][tok]
    // The value row pieces and beta first: the step waits for them before its
    // first barrier, for the rest only after it. Value rows at or past the
    // chunk's end read as zeros, and so do all of them in a block of M's
    // columns (U = 0 there).
    {
      const int t0 = bos + (c - c_begin) * kChunk;
      const int n = mblk ? 0 : min(kChunk, eos - t0);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(v) + ((size_t)t0 * HV + hv) * kHead, 0, n * HV * kHead * 2,
          kBufferWord3);
      x.vr = load_b128(rv, ((tid >> 2) * HV * kHead + v0 + 8 * (tid & 3)) * 2);
      // beta from the block's gate factors (64 consecutive floats), not from the
      // input, whose betas of one value head are a line apart
      x.bt = prep.gE[blk * kGates + 2 * kChunk + (tid >> 2)];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      x.wa[s] = ld8(Wb + kcm(16 * wave + li, 32 * s + 8 * kq, 64));
      if constexpr (kOut) x.qa[s] = ld8(Qb + kcm(16 * wave + li, 32 * s + 8 * kq, 64));
    }
    if constexpr (kOut) {
      // P's tiles above the diagonal are not stored: those pieces come from
      // past the end of a range-checked buffer, as zeros
      const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(Pb), 0, kChunk * kChunk * 2, kBufferWord3);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        x.pa[s] = ld8_buf(rp, 2 * s + (kq >> 1) <= wave ? kcm(16 * wave + li, 32 * s + 8 * kq, 64) * 2
                                                       : kChunk * kChunk * 2);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        x.ka[dt][s] = ld8(Kb + kcm(16 * (2 * wave + dt) + li, 32 * s + 8 * kq, 128));
    {
      // T [i][j]: the tiles above the diagonal are not stored and read as zeros
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(prep.T + blk * 8192), 0, kChunk * kChunk * 2, kBufferWord3);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        x.ta[s] = ld8_buf(rt, 2 * s + (kq >> 1) <= wave ? kcm(16 * wave + li, 32 * s + 8 * kq, 64) * 2
                                                       : kChunk * kChunk * 2);
    }
    x.gl = prep.gL[blk];
    const float* ge = prep.gE + blk * kGates;
    if constexpr (kOut) x.eg = ge[16 * wave + li];
    x.ebw = *reinterpret_cast<const float4*>(ge + kChunk + 16 * wave + 4 * kq);
    x.pf = touch_line(warm_line(pc));
  };

  auto step = [&](int c, const Ops& cur, int cn, Ops& nxt) {
    const int t0 = bos + (c - c_begin) * kChunk;
    const int len = min(kChunk, eos - t0);
    // the warm-up word nxt carries was requested two steps ago
    sink ^= nxt.pf;
    // 1. chunk-start state -> LDS (bf16), and the value rows scaled by beta
    {
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(&cur.vr);
      uint4 y;
      uint32_t* yw = reinterpret_cast<uint32_t*>(&y);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        yw[e] = pk2(bf2f(vw[e] & 0xffffu) * cur.bt, bf2f(vw[e] >> 16) * cur.bt);
      *reinterpret_cast<uint4*>(&Vs[(tid >> 2) * VP + 8 * (tid & 3)]) = y;
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int kk = 16 * (2 * wave + dt) + 4 * kq;
        const int vl = 16 * vt + li;
        *reinterpret_cast<uint2*>(&Ss[vl * SP + kk]) =
            pack4_bf16(h[dt][vt][0], h[dt][vt][1], h[dt][vt][2], h[dt][vt][3]);
      }
    __syncthreads();
    // the next set's requests, issued by all waves together right after the
    // barrier (waves that issue them together share the lines they fetch),
    // and the L2 warm-up of the chunk two steps ahead
    load_ops(cn, nxt, min(cn + 1, c_end - 1));
    uint16_t* sv = saved + blk_saved(c, hv, HV);
    if constexpr (kSave) {
      // h = S^T as [v / 32][v % 32 / 8][k][v % 8]: chunk e = 64 q + lane holds
      // h[k = e % 128][8 (e / 128) ..], read as columns of Ss with transposed
      // reads; consecutive lanes write consecutive chunks
#pragma unroll
      for (int i = 0; i < VB / 16; ++i) {
        const int q = wave + 4 * i;
        const uint4 x = lds_col8(Ss, SP, 8 * (q >> 1), 64 * (q & 1) + 16 * kq, lane);
        *reinterpret_cast<uint4*>(sv + v0 * kHead + 8 * (64 * q + lane)) = x;
      }
    }

    // 2. D = U - W h with U = T (diag(beta) V); wave w owns tokens
    //    16 w .. 16 w + 15 (T is lower triangular: tokens j > 16 w + 15
    //    contribute nothing to U there). The state part of
    //    the output, (S Q~^T) diag(e^gamma), needs no D: it is formed here from
    //    the same S fragments, ahead of the barrier that D needs.
    f32x4 oq[VT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      bf16x8 sb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) sb[s] = ld8(&Ss[(16 * vt + li) * SP + 32 * s + 8 * kq]);
      // two independent partial sums, so the MFMAs do not wait on each other
      f32x4 a0 = mfma(cur.wa[0], sb[0], zero4());
      f32x4 a1 = mfma(cur.wa[1], sb[1], zero4());
      if constexpr (kOut) {
        f32x4 q0 = mfma(sb[0], cur.qa[0], zero4());
        f32x4 q1 = mfma(sb[1], cur.qa[1], zero4());
        q0 = mfma(sb[2], cur.qa[2], q0);
        q1 = mfma(sb[3], cur.qa[3], q1);
        oq[vt] = (q0 + q1) * cur.eg;  // [v = 16 vt + 4 kq + r][t = 16 w + li]
      }
      a0 = mfma(cur.wa[2], sb[2], a0);
      a1 = mfma(cur.wa[3], sb[3], a1);
      const f32x4 acc = a0 + a1;
      // acc[r] = (W h)[t = 16 w + 4 kq + r][v = 16 vt + li], and u[r] = U there
      f32x4 u = mfma(cur.ta[0], __builtin_bit_cast(bf16x8, lds_col8(Vs, VP, 8 * kq, 16 * vt, lane)),
                     zero4());
      if (wave >= 2)
        u = mfma(cur.ta[1], __builtin_bit_cast(bf16x8, lds_col8(Vs, VP, 32 + 8 * kq, 16 * vt, lane)), u);
      const float d0 = u[0] - acc[0], d1 = u[1] - acc[1];
      const float d2 = u[2] - acc[2], d3 = u[3] - acc[3];
      const int ds = (16 * vt + li) * DP + 16 * wave + 4 * kq;
      *reinterpret_cast<uint2*>(&Ds[ds]) = pack4_bf16(d0, d1, d2, d3);
      *reinterpret_cast<uint2*>(&Es[ds]) = pack4_bf16(cur.ebw.x * d0, cur.ebw.y * d1,
                                                      cur.ebw.z * d2, cur.ebw.w * d3);
    }
    __syncthreads();
    if constexpr (kSave) {
      // D [tok][v] in the chunk-major tile layout: wave w writes the chunks of
      // value columns v0 + 8 w .. + 7, lane = token, read as columns of D^T
      if (wave < VB / 8)
        *reinterpret_cast<uint4*>(sv + kSavedH + kcm(lane, v0 + 8 * wave, kChunk)) =
            lds_col8(Ds, DP, 8 * wave, 16 * kq, lane);
    }

    // 3. O^T = (S Q~^T) diag(e^gamma) + D^T P^T, the first term from step 2;
    //    wave w owns tokens 16 w .. 16 w + 15 (lane li: token 16 w + li, so
    //    e^gamma is one factor). Rows at
    //    or past the chunk length fall outside the store's buffer range, which
    //    drops them.
    if constexpr (kOut) {
      const int tl = 16 * wave + li;
      const __amdgpu_buffer_rsrc_t orng =
          __builtin_amdgcn_make_buffer_rsrc(o + ((size_t)t0 * HV + hv) * kHead, 0,
                                            len * HV * kHead * 2, kBufferWord3);
      uint2 pk[VT];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        bf16x8 db[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) db[s] = ld8(&Ds[(16 * vt + li) * DP + 32 * s + 8 * kq]);
        // P is lower triangular: tokens j > 16 w + 15 contribute nothing
        f32x4 acc = mfma(db[0], cur.pa[0], oq[vt]);
        if (wave >= 2) acc = mfma(db[1], cur.pa[1], acc);
        // acc[r] = O[t = t0 + 16 w + li][v = v0 + 16 vt + 4 kq + r]
        pk[vt] = pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
      }
      // Lanes 16 kq + li and 16 (kq ^ 1) + li swap one of their two pieces: an
      // even kq keeps its vt = 0 piece and takes its partner's, an odd kq
      // keeps its vt = 1 piece and takes its partner's, so that each lane holds
      // 8 consecutive columns of its token's row and a wave's 16 rows x 64
      // bytes go out in one 16-byte store (one request per row, not two).
      static_assert(VT == 2, "two 16-column value tiles per block");
      const bool ev = (kq & 1) == 0;
      const uint2 send = ev ? pk[1] : pk[0];
      const uint2 recv = make_uint2(__shfl_xor(send.x, 16, 64), __shfl_xor(send.y, 16, 64));
      const uint4 x = ev ? make_uint4(pk[0].x, pk[0].y, recv.x, recv.y)
                         : make_uint4(recv.x, recv.y, pk[1].x, pk[1].y);
      const int col = ev ? 4 * kq : 16 + 4 * (kq - 1);
      store_b128(x, orng, (tl * HV * kHead + v0 + col) * 2);
    }

    // 4. h <- e^gamma_L h + K^T (diag(e^(gamma_L - gamma)) D); wave w owns key
    //    rows 32 w .. 32 w + 31
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        f32x4 acc = h[dt][vt] * cur.gl;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc = mfma(cur.ka[dt][s], ld8(&Es[(16 * vt + li) * DP + 32 * s + 8 * kq]), acc);
        h[dt][vt] = acc;
      }
    // No barrier here: no wave reads Ss or Vs after the barrier above, and
    // Ds, Es are rewritten only after the next chunk's first barrier, which
    // every wave reaches after its reads of them.
  };

  if (c_begin < c_end) {
    // the request past the last chunk re-reads the last chunk: one extra set
    // per chain keeps the memory operations of every chunk the same
    const int last = c_end - 1;
    Ops A, B;
    B.pf = 0;
    load_ops(c_begin, A, min(c_begin + 1, last));
    for (int c = c_begin;; c += 2) {
      step(c, A, min(c + 1, last), B);
      if (c + 1 > last) break;
      step(c + 1, B, min(c + 2, last), A);
      if (c + 2 > last) break;
    }
  }

  consume(sink);
  if constexpr (kTrans) hT = mblk ? st.M : st.hT;
  if (hT) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int kk = 16 * (2 * wave + dt) + 4 * kq;
        const int vv = v0 + 16 * vt + li;
        *reinterpret_cast<float4*>(hT + state_base + (size_t)vv * kHead + kk) =
            make_float4(h[dt][vt][0], h[dt][vt][1], h[dt][vt][2], h[dt][vt][3]);
      }
  }
}

__global__ __launch_bounds__(256) void state_copy_kernel(const float* __restrict__ src,
                                                         float* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_fwd_scan(ScanMode mode, const int32_t* seq_first, int N, int HV, int NC,
                           const ChunkInfo* table, const PrepOut& prep, const uint16_t* v,
                           const StateRef& st, uint16_t* o, uint16_t* saved,
                           hipStream_t stream) {
  const long chains = (long)N * HV;
  const long per_chain = (kHead / kScanVB) * (mode == ScanMode::kTransition ? 2 : 1);
  const long group = 8L * prep.G;  // chains per cycle over the XCDs (whole key heads)
  const dim3 grid((unsigned)((chains + group - 1) / group * group * per_chain));
  switch (mode) {
    case ScanMode::kOut:
      hipLaunchKernelGGL((fwd_scan_kernel<false, true, false>), grid, dim3(256), 0, stream,
                         seq_first, N, HV, NC, table, prep, v, st, o, saved);
      break;
    case ScanMode::kOutSave:
      hipLaunchKernelGGL((fwd_scan_kernel<true, true, false>), grid, dim3(256), 0, stream,
                         seq_first, N, HV, NC, table, prep, v, st, o, saved);
      break;
    case ScanMode::kSave:
      hipLaunchKernelGGL((fwd_scan_kernel<true, false, false>), grid, dim3(256), 0, stream,
                         seq_first, N, HV, NC, table, prep, v, st, o, saved);
      break;
    case ScanMode::kTransition:
      hipLaunchKernelGGL((fwd_scan_kernel<false, false, true>), grid, dim3(256), 0, stream,
                         seq_first, N, HV, NC, table, prep, v, st, o, saved);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_state_copy(const float* src, float* dst, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     src, dst, n);
  return hipGetLastError();
}

}  // namespace gdn
