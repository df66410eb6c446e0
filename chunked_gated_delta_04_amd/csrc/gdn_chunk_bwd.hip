// Backward of the chunked gated delta rule: reverse state-gradient scan and
// the per-chunk gradient pass. Their per-chunk operands (W, P, T, T^T,
// e^gamma_L and the per-token decays per value head; Q~ and K^T per key head)
// are the ones the forward's WY pass wrote behind the saved states
// (gdn_chunk_prep.hip), so no WY pass runs here.
//
// Chunk form (see gdn_chunk_prep.hip): D = U - W h, O = Q_g h + P D,
// h' = e^gamma_L h + K_bwd^T D, with U = T diag(beta) V,
// W = T diag(beta e^gamma) K^, T = (I + A)^-1. Given dO and dh' (the
// gradient of the chunk's end state):
//   dD   = P^T dO + K_bwd dh'
//   dh   = e^gamma_L dh' + Q_g^T dO - W^T dD          (reverse scan)
// which is the reverse recurrence written on the maxtext page ("Qwen3.5-397B
// RL trainer on 128 v7x", the gdn_cp_dh_scan commit) and the dhu stage the
// cake_gdn page (miles PR #3597) names; then, per chunk and in parallel,
//   dP   = dO D^T (i >= j)        dq~ += e^gamma dO h^T + (dP o Gamma) K^
//   dk^ += (dP o Gamma)^T Q~ + e^(gamma_L - gamma) D dh'^T
//        + diag(beta e^gamma) T^T dW + M K^ + M^T K^
//   dW   = -dD h^T,  dV = diag(beta) T^T dD
//   dT   = dD (beta V)^T + dW (beta e^gamma K^)^T,  dA = -T^T dT T^T (i > j)
//   M_ij = dA_ij beta_i e^(gamma_i - gamma_j)
// and the gate gradients dbeta, dgamma (then dg = reverse cumsum of dgamma in
// the chunk), the dqkwg and WY-pullback stages of the same page. The value
// heads of one key head are summed into dq^, dk^ in a fixed order inside one
// workgroup, then the L2-norm backward dx = (dx^ - x^ (x^ . dx^)) / |x| and
// the scale are applied. Nothing uses atomics; every sum has one owner and a
// fixed order, so results repeat bit for bit.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {
constexpr int KP = 136;  // LDS pitch (bf16) of [64][128] tiles

// Sum over the 16 lanes of a 16-lane group (lanes sharing kq), complete in
// the group's first lane only: DPP row shifts (VALU work in a fixed order)
// instead of four LDS swizzles.
__device__ __forceinline__ float sum16_lane0(float x) { return row_sum_first_lane(x); }
}  // namespace

// ---------------------------------------------------------------------------
// Reverse scan: dh (K x VB slice) in registers, chunks in reverse order.
// Writes per (chunk, value head): dh' as [k][v], dD as [tok][v] and [v][tok].
// The decays of Q_g = diag(e^gamma) Q~ and K_bwd = diag(e^(gamma_L - gamma)) K^
// are applied in fp32: to the dO rows for Q_g^T dO = Q~^T (diag(e^gamma) dO)
// and to the rows of K^ dh' for K_bwd dh'.
// As in the forward scan, two operand sets alternate and every chunk issues
// the same loads and stores with no branch around them, so waiting for a set
// never waits for a store; dO rows past the chunk's end come from a
// range-checked buffer load, which returns zeros there.
__global__ __launch_bounds__(256) void bwd_dh_scan_kernel(
    const int32_t* __restrict__ seq_first, int N, int HV, int NC,
    const ChunkInfo* __restrict__ table, PrepOut prep, const uint16_t* __restrict__ dO,
    const float* __restrict__ dhT, float* __restrict__ dh0, BwdBufs bufs) {
  constexpr int VB = kScanVB;
  constexpr int NVB = kHead / VB;
  constexpr int VT = VB / 16;
  constexpr int SP = 136;
  constexpr int DP = 72;
  constexpr int SPT = VB / 8;  // 16-byte dO segments per token row of the block
  static_assert(kChunk * SPT <= 256 && VB * 8 <= 256, "at most one 16-byte segment per thread");

  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int vb = slot % NVB;
  const int m = slot / NVB, G = prep.G;  // a key head's value heads on one XCD
  const int chain = ((m / G) * 8 + xcd) * G + m % G;
  if (chain >= N * HV) return;
  const int seq = chain / HV, hv = chain - seq * HV;
  const int v0 = vb * VB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;

  __shared__ __align__(16) uint16_t Hs[VB * SP];  // dh as [v][k]
  constexpr int OP = 40;  // LDS pitch of the dO rows (bf16)
  __shared__ __align__(16) uint16_t Ot[kChunk * OP];  // dO [tok][v - v0]
  __shared__ __align__(16) uint16_t Og[kChunk * OP];  // diag(e^gamma) dO [tok][v - v0]
  __shared__ __align__(16) uint16_t Es[VB * DP];  // dD^T [v][tok]
  // The chunk operands each wave contracts, in the forward's layouts (P [i][j],
  // K^T [k][tok], Q~ [tok][k], W [tok][k], all chunk-major): per wave
  // kOpBlocks column groups of 64 rows x 16 bytes, loaded into registers a
  // chunk ahead, written to the wave's own region at the start of the chunk
  // and read back transposed (lds_col8_cm). Only the wave that writes a
  // region reads it, so no barrier orders them.
  constexpr int kOpBlocks = 14, kOpStride = 512;
  __shared__ __align__(16) uint16_t Lop[4 * kOpBlocks * kOpStride];

  f32x4 dh[2][VT];
  const size_t state_base = ((size_t)seq * HV + hv) * kHead * kHead;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      const int kk = 16 * (2 * wave + dt) + 4 * kq;
      const int vv = v0 + 16 * vt + li;
      if (dhT) {
        const float4 x = *reinterpret_cast<const float4*>(dhT + state_base + (size_t)vv * kHead + kk);
        dh[dt][vt] = f32x4{x.x, x.y, x.z, x.w};
      } else {
        dh[dt][vt] = zero4();
      }
    }

  struct Ops {
    u32v4 op[kOpBlocks];  // row `lane` of each column group (see load_ops)
    uint4 dO;
    float gl;
    float eg;    // e^gamma of token ot (the dO row this thread stages)
    float4 ebw;  // e^(gamma_L - gamma) of tokens 16 wave + 4 kq .. + 3 (dD rows)
    uint32_t pf;  // L2 warm-up word of a later chunk (see touch_line)
  };
  const int ot = tid / SPT, osg = tid % SPT;  // dO segment of this thread (ot < 64 holds one)
  // chunk bounds from the sequence's bounds (consecutive 64-token chunks)
  const int c_begin = seq_first[seq], c_end = seq_first[seq + 1];
  int bos = 0, eos = 0;
  if (c_begin < c_end) {
    const ChunkInfo first = table[c_begin], lastc = table[c_end - 1];
    bos = first.t0;
    eos = lastc.t0 + lastc.len;
  }
  // This workgroup's share of a chunk's operand lines for the L2 warm-up: the
  // value head's W, P, gate-factor and dO lines (324) split over its value
  // blocks, the key head's Q~ and K^T lines (256) over the workgroups of all its
  // value heads. Lanes past the share all touch its first line (one request per
  // wave instruction, the lanes' addresses being the same); dO rows
  // past the chunk's end touch its last row.
  const int vlines = (324 + NVB - 1) / NVB;
  const int kshares = NVB * prep.G, kpos = (hv % prep.G) * NVB + vb;
  const int klines = (256 + kshares - 1) / kshares;
  auto warm_line = [&](int c) -> const void* {
    const size_t blk = (size_t)hv * NC + c;
    const size_t kblk = (size_t)(hv / prep.G) * NC + c;
    const int i = tid < vlines + klines ? tid : 0;
    if (i < vlines) {
      const int l = min(vb * vlines + i, 323);
      if (l < 128) return prep.W + blk * 8192 + l * kLineElems16;
      if (l < 192) return prep.P + blk * 4096 + (l - 128) * kLineElems16;
      if (l < 196) return prep.gE + blk * kGates + (l - 192) * kLineElems32;
      const int t0 = bos + (c - c_begin) * kChunk;
      const int r = min((l - 196) >> 1, eos - t0 - 1);
      return dO + ((size_t)(t0 + r) * HV + hv) * kHead + ((l - 196) & 1) * kLineElems16;
    }
    const int l = min(kpos * klines + (i - vlines), 255);
    if (l < 128) return prep.Qn + kblk * 8192 + l * kLineElems16;
    return prep.Kn + kblk * 8192 + (l - 128) * kLineElems16;
  };
  uint32_t sink = 0;
  // pc: the chunk whose lines the set's L2 warm-up word touches. Wave w takes
  // the column groups it contracts: P's columns 16 w .. 16 w + 15 (groups
  // 2 w, 2 w + 1; pieces 0, 1), K^T's token columns 16 w .. (groups 2 w,
  // 2 w + 1, each as key rows 0-63 and 64-127; pieces 2-5), and the key
  // columns 32 w .. 32 w + 31 of Q~ and W (groups 4 w .. ; pieces 6-9 and
  // 10-13). Each piece is one 1 KiB request: lane l holds the 16 bytes of row l.
  auto load_ops = [&](int c, Ops& x, int pc) {
    const size_t blk = (size_t)hv * NC + c;
    const size_t kblk = (size_t)(hv / prep.G) * NC + c;
    const uint16_t* Pb = prep.P + blk * 4096;     // P [i][j]
    const uint16_t* Kb = prep.Kn + kblk * 8192;   // K^T [k][tok]
    const uint16_t* Qb = prep.Qn + kblk * 8192;   // Q~ [tok][k]
    const uint16_t* Wb = prep.W + blk * 8192;     // W [tok][k]
#pragma unroll
    for (int g = 0; g < 2; ++g)
      x.op[g] = *reinterpret_cast<const u32v4*>(Pb + (2 * wave + g) * 512 + 8 * lane);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        x.op[2 + 2 * g + hh] =
            *reinterpret_cast<const u32v4*>(Kb + (2 * wave + g) * 1024 + hh * 512 + 8 * lane);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      x.op[6 + g] = *reinterpret_cast<const u32v4*>(Qb + (4 * wave + g) * 512 + 8 * lane);
      x.op[10 + g] = *reinterpret_cast<const u32v4*>(Wb + (4 * wave + g) * 512 + 8 * lane);
    }
    x.gl = prep.gL[blk];
    const float* ge = prep.gE + blk * kGates;
    x.eg = ge[ot & (kChunk - 1)];
    x.ebw = *reinterpret_cast<const float4*>(ge + kChunk + 16 * wave + 4 * kq);
    const int t0 = bos + (c - c_begin) * kChunk;
    const int len = min(kChunk, eos - t0);
    const __amdgpu_buffer_rsrc_t rng = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(dO) + ((size_t)t0 * HV + hv) * kHead, 0, len * HV * kHead * 2,
        kBufferWord3);
    x.dO = load_b128(rng, (ot * HV * kHead + v0 + 8 * osg) * 2);
    x.pf = touch_line(warm_line(pc));
  };

  auto step = [&](int c, const Ops& cur) {
    const size_t blk = (size_t)hv * NC + c;
    uint16_t* const R = Lop + wave * (kOpBlocks * kOpStride);
    // the wave's operand pieces into its own region (the previous chunk's
    // transposed reads of it have completed: their MFMAs consumed them)
#pragma unroll
    for (int i = 0; i < kOpBlocks; ++i)
      *reinterpret_cast<u32v4*>(R + i * kOpStride + 8 * lane) = cur.op[i];
    // 1. dh -> LDS; stage dO^T for this value block
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int kk = 16 * (2 * wave + dt) + 4 * kq;
        *reinterpret_cast<uint2*>(&Hs[(16 * vt + li) * SP + kk]) =
            pack4_bf16(dh[dt][vt][0], dh[dt][vt][1], dh[dt][vt][2], dh[dt][vt][3]);
      }
    if (ot < kChunk) {
      *reinterpret_cast<uint4*>(&Ot[ot * OP + 8 * osg]) = cur.dO;
      const uint32_t* xw = reinterpret_cast<const uint32_t*>(&cur.dO);
      const float e = cur.eg;
      *reinterpret_cast<uint4*>(&Og[ot * OP + 8 * osg]) =
          make_uint4(pk2(e * bf2f(xw[0] & 0xffffu), e * bf2f(xw[0] >> 16)),
                     pk2(e * bf2f(xw[1] & 0xffffu), e * bf2f(xw[1] >> 16)),
                     pk2(e * bf2f(xw[2] & 0xffffu), e * bf2f(xw[2] >> 16)),
                     pk2(e * bf2f(xw[3] & 0xffffu), e * bf2f(xw[3] >> 16)));
    }
    __syncthreads();
    // dh' (gradient of this chunk's end state) as [v / 32][v % 32 / 8][k][v % 8],
    // read as columns of Hs with transposed reads (chunk e = 64 q + lane)
    {
      uint16_t* dhb = bufs.dh + blk * (kHead * kHead) + v0 * kHead;
#pragma unroll
      for (int i = 0; i < VB / 16; ++i) {
        const int q = wave + 4 * i;
        *reinterpret_cast<uint4*>(dhb + 8 * (64 * q + lane)) =
            lds_col8(Hs, SP, 8 * (q >> 1), 64 * (q & 1) + 16 * kq, lane);
      }
    }

    // dO as operand fragments (contraction over tokens), read as columns of
    // the dO rows: ob[vt][s] = dO[32 s + 8 kq .. + 7][16 vt + li]
    bf16x8 ob[VT][2];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        ob[vt][s] = __builtin_bit_cast(bf16x8, lds_col8(Ot, OP, 32 * s + 8 * kq, 16 * vt, lane));

    // 2. dD = P^T dO + diag(e^(gamma_L - gamma)) K^ dh; wave w owns tokens
    //    16 w .. 16 w + 15. Operands: pa[s] = P[32 s + 8 kq ..][16 w + li]
    //    (P^T's rows), zero where that 16 x 16 tile of P lies above its
    //    diagonal (those tiles are not stored); ka[s] = K^[16 w + li][32 s + 8 kq ..]
    bf16x8 pa[2], ka[4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 x = lds_col8_cm(R, R + kOpStride, 32 * s + 8 * kq, lane);
      pa[s] = __builtin_bit_cast(bf16x8, 2 * s + (kq >> 1) >= wave ? x : make_uint4(0u, 0u, 0u, 0u));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      ka[s] = __builtin_bit_cast(bf16x8, lds_col8_cm(R + (2 + (s >> 1)) * kOpStride,
                                                     R + (4 + (s >> 1)) * kOpStride,
                                                     (32 * s + 8 * kq) & 63, lane));
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      bf16x8 hb4[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) hb4[s] = ld8(&Hs[(16 * vt + li) * SP + 32 * s + 8 * kq]);
      // two independent partial sums, so the MFMAs do not wait on each other
      f32x4 a0 = mfma(ka[0], hb4[0], zero4());
      f32x4 a1 = mfma(ka[1], hb4[1], zero4());
      f32x4 ap = mfma(pa[1], ob[vt][1], zero4());
      a0 = mfma(ka[2], hb4[2], a0);
      a1 = mfma(ka[3], hb4[3], a1);
      if (wave < 2) ap = mfma(pa[0], ob[vt][0], ap);
      const f32x4 ak = a0 + a1;
      const f32x4 acc = f32x4{ak[0] * cur.ebw.x, ak[1] * cur.ebw.y, ak[2] * cur.ebw.z,
                              ak[3] * cur.ebw.w} + ap;
      // acc[r] = dD[t = 16 w + 4 kq + r][v = 16 vt + li]
      *reinterpret_cast<uint2*>(&Es[(16 * vt + li) * DP + 16 * wave + 4 * kq]) =
          pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
    }
    // The part of step 3 that needs no dD, while the other waves finish theirs:
    // dh <- e^gamma_L dh + Q~^T (diag(e^gamma) dO) (dh was copied to LDS above)
    {
      // qa[dt][s] = Q~^T[16 (2 w + dt) + li][32 s + 8 kq ..], columns of Q~
      bf16x8 qa[2][2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          qa[dt][s] = __builtin_bit_cast(bf16x8, lds_col8_cm(R + (6 + 2 * dt) * kOpStride,
                                                             R + (7 + 2 * dt) * kOpStride,
                                                             32 * s + 8 * kq, lane));
      bf16x8 og[VT][2];
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          og[vt][s] = __builtin_bit_cast(bf16x8, lds_col8(Og, OP, 32 * s + 8 * kq, 16 * vt, lane));
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
          f32x4 acc = dh[dt][vt] * cur.gl;
#pragma unroll
          for (int s = 0; s < 2; ++s) acc = mfma(qa[dt][s], og[vt][s], acc);
          dh[dt][vt] = acc;
        }
    }
    __syncthreads();
    // dD to global as [v][tok] (row copy) and [tok][v] (column gather), both in
    // the chunk-major tile layout: one 16-byte store each per thread
    {
      uint16_t* dDT = bufs.dDT + blk * 8192;
      uint16_t* dDr = bufs.dD + blk * 8192;
      const int sg = tid / VB, vl = tid % VB;
      if (tid < VB * 8)
        *reinterpret_cast<uint4*>(dDT + kcm(v0 + vl, 8 * sg, kHead)) =
            *reinterpret_cast<const uint4*>(&Es[vl * DP + 8 * sg]);
      if (wave < VB / 8)
        *reinterpret_cast<uint4*>(dDr + kcm(lane, v0 + 8 * wave, kChunk)) =
            lds_col8(Es, DP, 8 * wave, 16 * kq, lane);
    }

    // 3. dh <- (e^gamma_L dh + Q~^T (diag(e^gamma) dO), from above) - W^T dD;
    //    wave w owns key rows 32 w .. 32 w + 31;
    //    wa[dt][s] = W^T[16 (2 w + dt) + li][32 s + 8 kq ..], columns of W
    bf16x8 wa[2][2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        wa[dt][s] = __builtin_bit_cast(bf16x8, lds_col8_cm(R + (10 + 2 * dt) * kOpStride,
                                                           R + (11 + 2 * dt) * kOpStride,
                                                           32 * s + 8 * kq, lane));
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        f32x4 acw = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acw = mfma(wa[dt][s], ld8(&Es[(16 * vt + li) * DP + 32 * s + 8 * kq]), acw);
        dh[dt][vt] = dh[dt][vt] - acw;
      }
    // No barrier here: Hs, Ot and Og are last read before the barrier above,
    // and Es is rewritten only after the next chunk's first barrier, which
    // every wave reaches after its reads of it.
  };

  if (c_begin < c_end) {
    // chunks run from the last to the first; the request past the first chunk
    // re-reads the first one
    const int first = c_begin;
    Ops A, B;
    B.pf = 0;
    load_ops(c_end - 1, A, max(c_end - 2, first));
    for (int c = c_end - 1;; c -= 2) {
      sink ^= B.pf;  // requested two sets ago
      load_ops(max(c - 1, first), B, max(c - 2, first));
      step(c, A);
      if (c - 1 < first) break;
      sink ^= A.pf;
      load_ops(max(c - 2, first), A, max(c - 3, first));
      step(c - 1, B);
      if (c - 2 < first) break;
    }
  }
  consume(sink);

  if (dh0) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int kk = 16 * (2 * wave + dt) + 4 * kq;
        const int vv = v0 + 16 * vt + li;
        *reinterpret_cast<float4*>(dh0 + state_base + (size_t)vv * kHead + kk) =
            make_float4(dh[dt][vt][0], dh[dt][vt][1], dh[dt][vt][2], dh[dt][vt][3]);
      }
  }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients: one 512-thread workgroup per CU (its LDS leaves room
// for no second one), each taking the items (chunk, key head) c H + h in
// steps of the grid size; the value heads of an item run in order. Wave w owns
// token tile tw = w & 3 (tokens 16 tw .. 16 tw + 15) and column half
// kh = w >> 2 (key or value columns 64 kh .. 64 kh + 63) of every
// token-indexed result. Matrices that are contracted over the chunk's tokens
// are kept in LDS as bf16 rows (tiles of 64 x 64 also transposed); their
// columns come from transposing LDS reads, so every MFMA operand is one or two
// LDS reads. The state h and its gradient dh' are copied straight from HBM
// into LDS - for an item's first value head, together with its raw q and k
// rows, while the previous item finishes (norm backward, output stores); for
// the next value head as soon as the current one is done with them - and each
// phase's other operands are requested a phase ahead, so the workgroup, alone
// on its CU, does not stall on memory at every phase.
// Per-token and per-column partial sums go to LDS slots owned by one wave each
// and are added once per value head in a fixed order.
namespace {
constexpr int BP = 72;  // LDS pitch (bf16) of [64][64] tiles

struct BwdLds {
  uint16_t Ks[64 * KP];                     // k^ rows
  uint16_t Qs[64 * KP];                     // q~ rows (columns of both come from
                                            // transpose reads)
  union {                                   // time-shared regions
    uint16_t Z[64 * KP];                    //   Z = T^T dD [tok][v]
    uint16_t V[64 * KP];                    //   V rows of the chunk
    uint16_t dT[64 * BP];                   //   dT [i][m]
    uint16_t dq[64 * KP];                   //   dq rows before they are stored
  } rz;
  float gam[64], bet[64], eg[64], ebw[64];
  float inv_k[64], inv_q[64];  // 1 / |k|, 1 / |q| per token
  float rowF[2][64], colF[8][64];           // F = dP o P
  float rowG[2][64], rowB2[2][64];          // row terms of the key-column passes
  float rowB[2][64];                        // dbeta of U
  float rowE[2][64], colE[8][64], rowB3[2][64];  // E = dA o A, dbeta of A
  float gl_part[8], hd_part[8];
  float dot_q[2][64], dot_k[2][64];         // (dot_q also holds an even value head's
                                            // dg, dbeta until its odd partner's)
};

// Column c0 + lane % 16 of a [64][KP] row tile: rows r0 .. r0 + 7 as an MFMA
// operand, or rows r0 .. r0 + 3 in fp32 (r0 may differ between lane groups).
__device__ __forceinline__ bf16x8 col8(const uint16_t* tile, int r0, int c0, int lane) {
  return __builtin_bit_cast(bf16x8, lds_col8(tile, KP, r0, c0, lane));
}
__device__ __forceinline__ float4 col4_bf16(const uint16_t* tile, int r0, int c0, int lane) {
  const int j = lane & 15;
  const uint2 u = lds_tr16(tile + (r0 + (j >> 2)) * KP + c0 + 4 * (j & 3));
  return make_float4(bf2f(u.x & 0xffffu), bf2f(u.x >> 16), bf2f(u.y & 0xffffu), bf2f(u.y >> 16));
}
__device__ __forceinline__ float dot8u(const uint4& a, const uint4& b) {  // bf16 pairs
  const uint32_t* x = reinterpret_cast<const uint32_t*>(&a);
  const uint32_t* y = reinterpret_cast<const uint32_t*>(&b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    s += bf2f(x[e] & 0xffffu) * bf2f(y[e] & 0xffffu) + bf2f(x[e] >> 16) * bf2f(y[e] >> 16);
  return s;
}
}  // namespace

template <bool kPair>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(
    const ChunkInfo* __restrict__ table, int NC, int H, int HV, float scale,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const uint16_t* __restrict__ saved,
    const uint16_t* __restrict__ Tmat, const float* __restrict__ gE,
    const float* __restrict__ gB, BwdBufs bufs, const uint16_t* __restrict__ dO,
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta) {
  __shared__ __align__(16) BwdLds S;
  // h and dh' in the layout both have in global memory ([v / 8][k][v % 8]),
  // filled by direct global-to-LDS copies; arrays of their own, so that those
  // copies are not taken to alias the tiles in S.
  __shared__ __align__(16) uint16_t Hs[kHead * kHead];
  __shared__ __align__(16) uint16_t Gs[kHead * kHead];
  // The [64][64] tiles dP o Gamma and its transpose (then T, T^T; then M, M^T)
  // and the dW / Y1^T region: arrays of their own as well, because between
  // two items they receive the next item's raw q and k rows by direct copies.
  __shared__ __align__(16) uint16_t PP[2 * 64 * BP];
  __shared__ __align__(16) uint16_t RW[64 * KP];
  uint16_t* const Pm = PP;
  uint16_t* const PmT = PP + 64 * BP;
  uint16_t* const dWs = RW;   // dW [tok][k], pitch KP
  uint16_t* const Y1T = RW;   // (dT T^T)^T [j][i], pitch BP
  uint16_t* const Qraw = PP;  // raw q rows [tok][k], pitch 128
  uint16_t* const Kraw = RW;  // raw k rows [tok][k], pitch 128

  const int G = HV / H;
  const int NI = NC * H;  // items: (chunk c, key head h) is item c H + h

  // h and dh' of chunk c_, value head hv_ straight into LDS (Hs, Gs): each
  // wave copies 1 KiB per request, lane l the 16 bytes at offset 16 l.
  auto copy_states = [&](int c_, int hv_, int wave, int lane) {
    const uint16_t* hb_ = saved + blk_saved(c_, hv_, HV);
    const uint16_t* dhb_ = bufs.dh + ((size_t)hv_ * NC + c_) * (kHead * kHead);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e0 = 512 * i + 64 * wave;  // first 16-byte chunk of the copy
      __builtin_amdgcn_global_load_lds(hb_ + 8 * (e0 + lane),
                                       (__attribute__((address_space(3))) void*)(Hs + 8 * e0),
                                       16, 0, kNonTemporal);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e0 = 512 * i + 64 * wave;
      __builtin_amdgcn_global_load_lds(dhb_ + 8 * (e0 + lane),
                                       (__attribute__((address_space(3))) void*)(Gs + 8 * e0),
                                       16, 0, kNonTemporal);
    }
  };

  // What item it_ needs before its first value head, copied straight into
  // LDS: h and dh' of its first value head (Hs, Gs) and its raw q and k rows
  // (Qraw, Kraw; wave copy i of wave w covers rows 8 w + 4 i .. + 3, lane l
  // the 16 bytes of row + l / 16 at column 8 (l % 16); rows past the chunk's
  // end repeat its last row and are masked where they are read). Issued for
  // the workgroup's first item on entry and for its next item as soon as the
  // current one is done with those regions, so that the copies overlap the
  // current item's norm backward and output stores.
  auto prefetch = [&](int it_) {
    if (it_ >= NI) return;
    const int c_ = it_ / H, h_ = it_ - c_ * H;
    const ChunkInfo cn = table[c_];
    if (cn.seq < 0) return;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6, lane = tid & 63;
    copy_states(c_, h_ * G, wave, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r0 = 8 * wave + 4 * i;
      const int r = min(r0 + (lane >> 4), cn.len - 1);
      const size_t off = ((size_t)(cn.t0 + r) * H + h_) * kHead + 8 * (lane & 15);
      __builtin_amdgcn_global_load_lds(q + off,
                                       (__attribute__((address_space(3))) void*)(Qraw + 128 * r0),
                                       16, 0, kNonTemporal);
      __builtin_amdgcn_global_load_lds(k + off,
                                       (__attribute__((address_space(3))) void*)(Kraw + 128 * r0),
                                       16, 0, kNonTemporal);
    }
  };

  prefetch(blockIdx.x);
  for (int it = blockIdx.x; it < NI; it += gridDim.x) {
    const int c = it / H, h = it - c * H;
    const ChunkInfo ci = table[c];
    // the chunk slots past the pack's chunks are the last ones, so every later
    // item of this workgroup is past them too
    if (ci.seq < 0) break;
    const int t0 = ci.t0, L = ci.len;

    // every wave's copies for this item have landed
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    lds_barrier();

    // ---- q, k rows (copied into Qraw, Kraw): L2 norm; k^ and q~ as rows (Ks,
    //      Qs). 16 threads per row.
    {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));  // (opaque: nothing here is hoisted out of the item loop)
      const int sg = tid & 15;
      uint4 kr[2], qr[2];
      float sk[2], sq[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = (tid >> 4) + 32 * j;
        const uint32_t m = r < L ? 0xffffffffu : 0u;  // rows past the chunk's end: zeros
        const uint4 kx = *reinterpret_cast<const uint4*>(&Kraw[128 * r + 8 * sg]);
        const uint4 qx = *reinterpret_cast<const uint4*>(&Qraw[128 * r + 8 * sg]);
        kr[j] = make_uint4(kx.x & m, kx.y & m, kx.z & m, kx.w & m);
        qr[j] = make_uint4(qx.x & m, qx.y & m, qx.z & m, qx.w & m);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qr[j]);
        sk[j] = 0.f;
        sq[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = bf2f(kw[e] & 0xffffu), a1 = bf2f(kw[e] >> 16);
          const float b0 = bf2f(qw[e] & 0xffffu), b1 = bf2f(qw[e] >> 16);
          sk[j] += a0 * a0 + a1 * a1;
          sq[j] += b0 * b0 + b1 * b1;
        }
        sk[j] = group_sum<16>(sk[j]);
        sq[j] = group_sum<16>(sq[j]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = (tid >> 4) + 32 * j;
        const float ik = 1.f / sqrtf(sk[j] + kNormEps), iq = 1.f / sqrtf(sq[j] + kNormEps);
        const float iqs = iq * scale;
        if (sg == 0) {
          S.inv_k[r] = ik;
          S.inv_q[r] = iq;
        }
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qr[j]);
        uint4 ko, qo;
        uint32_t* kow = reinterpret_cast<uint32_t*>(&ko);
        uint32_t* qow = reinterpret_cast<uint32_t*>(&qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kow[e] = pk2(bf2f(kw[e] & 0xffffu) * ik, bf2f(kw[e] >> 16) * ik);
          qow[e] = pk2(bf2f(qw[e] & 0xffffu) * iqs, bf2f(qw[e] >> 16) * iqs);
        }
        *reinterpret_cast<uint4*>(&S.Ks[r * KP + sg * 8]) = ko;
        *reinterpret_cast<uint4*>(&S.Qs[r * KP + sg * 8]) = qo;
      }
    }
    lds_barrier();

    // Gate gradients of value head hv_ (the item's jv-th): fixed-order sums of
    // the partial slots, then dg = reverse cumsum of dgamma inside the chunk
    // (wave 0), and dbeta (wave 1), each wave storing one of the two. Run at the
    // top of the next value head (or after the last one): the slots and gamma
    // are rewritten only after the next gate barrier, which both waves reach
    // after this, and the work overlaps the other waves' requests. Each store
    // reaches 64 lines (a token's line holds every value head's value) and a
    // wave's later loads wait for its stores, so the two go to different waves,
    // and with kPair (an even number of value heads per key head, dg and dbeta
    // 8-byte aligned) an even head's values wait in LDS for its odd partner's,
    // so that one store writes both. t: the lane, from an opaque
    // copy of the thread index (see the value-head loop), so that none of the
    // addresses below is hoisted out of the loop.
    auto put = [&](float* dst, float* stash, int hv_, int jv, int t, float x) {
      if (kPair && (jv & 1) == 0) {
        stash[t] = x;
      } else if (t < L) {
        float* p = dst + (size_t)(t0 + t) * HV + hv_;
        if (kPair)
          *reinterpret_cast<float2*>(p - 1) = make_float2(stash[t], x);
        else
          *p = x;
      }
    };
    auto db_out = [&](int hv_, int jv, int t) {
      const float dbt = (S.rowB[0][t] + S.rowB[1][t]) + (S.rowB2[0][t] + S.rowB2[1][t]) +
                        (S.rowB3[0][t] + S.rowB3[1][t]);
      put(dbeta, S.dot_q[1], hv_, jv, t, dbt);
    };
    auto dg_out = [&](int hv_, int jv, int t) {
      const int w0 = 4 * ((t >> 4) & 1);  // the waves whose column tiles hold t
      float dgm = (S.rowF[0][t] + S.rowF[1][t]) + (S.rowG[0][t] + S.rowG[1][t]) +
                  (S.rowE[0][t] + S.rowE[1][t]);
#pragma unroll
      for (int w = 0; w < 4; ++w) dgm -= S.colF[w0 + w][t] + S.colE[w0 + w][t];
      float x = t < L ? dgm : 0.f;
      if (t == L - 1) {
        float glsum = 0.f, hdsum = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          glsum += S.gl_part[w];
          hdsum += S.hd_part[w];
        }
        x += glsum + exp2_fast(S.gam[L - 1]) * hdsum;
      }
      x = wave_suffix_sum(x, t);
      put(dg, S.dot_q[0], hv_, jv, t, x);
    };

    // dq~, dk^ over the value heads: [j][r] = d[16 tw + 4 kq + r][16 (4 kh + j) + li]
    f32x4 adq[4], adk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      adq[j] = zero4();
      adk[j] = zero4();
    }

    const size_t rs = (size_t)HV * kHead;  // token stride of dO, v, dv


    for (int jg = 0; jg < G; ++jg) {
      // Re-derive the thread coordinates each iteration from an opaque copy, so
      // the many LDS addresses built from them are not hoisted out of the loop
      // (they would not fit in the register budget of two waves per SIMD).
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63, wave = tid >> 6;
      const int tw = wave & 3, kh = wave >> 2;
      const int li = lane & 15, kq = lane >> 4;
      const int trow = 16 * tw + li;
      const bool trow_ok = trow < L;
      const int hv = h * G + jg;
      const size_t blk = (size_t)hv * NC + c;
      // (chunk-major tiles: see kcm; states: [v / 32][v % 32 / 8][k][v % 8])
      const uint16_t* hb = saved + blk_saved(c, hv, HV);  // h
      const uint16_t* Db = hb + kSavedH;                   // D [tok][v], chunk-major
      const uint16_t* dDb = bufs.dD + blk * 8192;          // dD [tok][v], chunk-major
      const uint16_t* dDTb = bufs.dDT + blk * 8192;        // dD^T [v][tok], chunk-major
      const uint16_t* Tg = Tmat + blk * 8192;              // T, then T^T, chunk-major
      // Token rows of dO and v through range-checked buffer loads: rows at or
      // past the chunk's end read as zeros, with no branch around the load.
      const __amdgpu_buffer_rsrc_t rdO = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(dO) + ((size_t)t0 * HV + hv) * kHead, 0, L * (int)rs * 2, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(v) + ((size_t)t0 * HV + hv) * kHead, 0, L * (int)rs * 2, kBufferWord3);

      // ---- gate requests first (every wave; wave 0 uses them), so that their
      //      wait does not cover the operand requests below: gamma (base 2),
      //      beta, e^gamma and e^(gamma_L - gamma) of each token as the forward's
      //      WY pass formed them, four contiguous 256-byte rows
      const float gam_t = gB[blk * kGatesB + lane];
      const float bet_t = gB[blk * kGatesB + kChunk + lane];
      const float eg_t = gE[blk * kGates + lane];
      const float ebw_t = gE[blk * kGates + kChunk + lane];

      // ---- requests for the dP phase: the own rows of dO and q, the D rows of
      //      this wave's dP tiles. Operand pieces the wave does not use (tiles
      //      above the diagonal, token blocks before its own) are requested past
      //      the end of a range-checked buffer, which returns zeros and moves no
      //      data, so every wave issues the same requests with no branch.
      constexpr int kTileBytes = kChunk * kHead * 2, kTBytes = kChunk * kChunk * 2;
      const __amdgpu_buffer_rsrc_t rD = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(Db), 0, kTileBytes, kBufferWord3);
      bf16x8 oa[4], dfr[2][4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        oa[s] = ld8_buf(rdO, (trow * (int)rs + 32 * s + 8 * kq) * 2);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int jb = kh + 2 * q2;
          dfr[q2][s] = ld8_buf(rD, jb <= tw ? kcm(16 * jb + li, 32 * s + 8 * kq, kChunk) * 2 : kTileBytes);
        }
      }

      // requests for the Z phase: T^T rows of this wave's tokens, dD^T rows, v rows
      // (token blocks s with 32 s + 31 < 16 tw meet only zeros of T; T^T's
      // tiles below the diagonal are not stored, so those pieces are zeros
      // from past the end of the buffer too)
      const __amdgpu_buffer_rsrc_t rTT = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(Tg) + 4096, 0, kTBytes, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rDDT = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(dDTb), 0, kTileBytes, kBufferWord3);
      bf16x8 tt[2], ddt[4][2];
      uint2 vr[4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        tt[s] = ld8_buf(rTT, 2 * s + (kq >> 1) >= tw ? kcm(trow, 32 * s + 8 * kq, 64) * 2 : kTBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vt = 4 * kh + j;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          ddt[j][s] = ld8_buf(rDDT, 32 * s + 31 >= 16 * tw
                                        ? kcm(16 * vt + li, 32 * s + 8 * kq, kHead) * 2 : kTileBytes);
        vr[j] = load_b64(rv, (trow * (int)rs + 16 * vt + 4 * kq) * 2);
      }

      // ---- gates (wave 0, after the previous value head's gate gradients)
      if (wave == 0) {
        if (jg > 0) dg_out(hv - 1, jg - 1, lane);
        S.gam[lane] = gam_t;
        S.bet[lane] = bet_t;
        S.eg[lane] = eg_t;
        S.ebw[lane] = ebw_t;
      } else if (wave == 1) {
        if (jg > 0) db_out(hv - 1, jg - 1, lane);
      }
      lds_barrier();

      // ---- dP = dO D^T (i >= j) and P = Gamma o Q~K^T: Pm = dP o Gamma (+ transpose);
      //      F = dP o P row / column partial sums. Wave: row tile tw, col tiles kh, kh + 2.
      {
        float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int jb = kh + 2 * q2;
          const int j = 16 * jb + li;
          float pv[4] = {0.f, 0.f, 0.f, 0.f};
          if (jb <= tw) {
            // dP tile and the Q~ K^T tile at the same place (formed here, per
            // value head, rather than kept in registers across them)
            f32x4 dp = zero4(), qk = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              dp = mfma(oa[s], dfr[q2][s], dp);
              qk = mfma(ld8(&S.Qs[trow * KP + 32 * s + 8 * kq]),
                        ld8(&S.Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), qk);
            }
            float colp = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 16 * tw + 4 * kq + r;
              if (i >= j) {
                const float dpm = dp[r] * exp2_fast(S.gam[i] - S.gam[j]);
                const float f = dpm * qk[r];
                pv[r] = dpm;
                rowp[r] += f;
                colp += f;
              }
            }
            colp = sum_over_rows(colp);
            if (kq == 0) S.colF[wave][j] = colp;
          } else if (kq == 0) {
            S.colF[wave][j] = 0.f;  // every slot of the wave's column tiles is written
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) Pm[(16 * tw + 4 * kq + r) * BP + j] = f2bf(pv[r]);
          *reinterpret_cast<uint2*>(&PmT[j * BP + 16 * tw + 4 * kq]) =
              pack4_bf16(pv[0], pv[1], pv[2], pv[3]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rowp[r] = sum16_lane0(rowp[r]);
        if (li == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) S.rowF[kh][16 * tw + 4 * kq + r] = rowp[r];
        }
      }
      // ---- Z = T^T dD (written [tok][v]); dV = diag(beta) Z; dbeta of U.
      //      Wave: token columns of tile tw, value tiles 4 kh .. 4 kh + 3.
      //      First every request of this wave is waited for: the Z operands are
      //      the youngest, and the copies of h and dh', issued before them, are
      //      then in LDS too (for the other waves after the barrier below).
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      {
        float bp = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int vt = 4 * kh + j;
          f32x4 z = zero4();
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (32 * s + 31 >= 16 * tw)  // T[m][t] needs m >= t
              z = mfma(ddt[j][s], tt[s], z);
          // z[r] = Z[t = trow][v = 16 vt + 4 kq + r]
          const int vv = 16 * vt + 4 * kq;
          *reinterpret_cast<uint2*>(&S.rz.Z[trow * KP + vv]) = pack4_bf16(z[0], z[1], z[2], z[3]);
          if (trow_ok) {
            const uint2 u = vr[j];
            bp += bf2f(u.x & 0xffffu) * z[0] + bf2f(u.x >> 16) * z[1] +
                  bf2f(u.y & 0xffffu) * z[2] + bf2f(u.y >> 16) * z[3];
            const float bt = S.bet[trow];
            *reinterpret_cast<uint2*>(dv + ((size_t)(t0 + trow) * HV + hv) * kHead + vv) =
                pack4_bf16(bt * z[0], bt * z[1], bt * z[2], bt * z[3]);
          }
        }
        bp = sum_over_rows(bp);
        if (kq == 0) S.rowB[kh][trow] = bp;
      }
      // the own rows of dD (pass 2 and dT), requested as soon as the Z operands
      // are dead, so that passes 1a and 1b cover their wait
      bf16x8 ea[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        ea[s] = __builtin_bit_cast(bf16x8, ld16_nt(dDb + kcm(trow, 32 * s + 8 * kq, kChunk)));
      lds_barrier();

      // ---- key-column passes (columns 16 kt + li, kt = 4 kh .. 4 kh + 3), h from LDS:
      //      pass 1: x1 = dO h^T, x4 = Z h^T (= -T^T dW),
      //              y1 = (dP o Gamma) K^, y2 = (dP o Gamma)^T Q~
      //      pass 2: x3 = dD h^T (= -dW), stored for dT
      //      then dh' replaces h in LDS; pass 3: x2 = D dh'^T
      float gr[4] = {0.f, 0.f, 0.f, 0.f}, br[4] = {0.f, 0.f, 0.f, 0.f};
      {  // pass 1a: x1, y1 -> dq~
        bf16x8 pa[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) pa[s] = ld8(&Pm[trow * BP + 32 * s + 8 * kq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * (4 * kh + j) + li;
          f32x4 x1 = zero4(), y1 = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) x1 = mfma(oa[s], ld8(&Hs[kcm(kr, 32 * s + 8 * kq, kHead)]), x1);
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (32 * s <= 16 * tw + 15)  // (dP o Gamma)[t][j] needs j <= t
              y1 = mfma(pa[s], col8(S.Ks, 32 * s + 8 * kq, kr - li, lane), y1);
          const int tr = 16 * tw + 4 * kq;
          const float4 qv = col4_bf16(S.Qs, tr, kr - li, lane);
          const float qa_[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = S.eg[tr + r];
            adq[j][r] += e * x1[r] + y1[r];
            gr[r] += e * qa_[r] * x1[r];               // inter-chunk output decay
          }
        }
      }
      {  // pass 1b: x4, y2 -> dk^
        bf16x8 za[4], pta[2];
#pragma unroll
        for (int s = 0; s < 4; ++s) za[s] = ld8(&S.rz.Z[trow * KP + 32 * s + 8 * kq]);
#pragma unroll
        for (int s = 0; s < 2; ++s) pta[s] = ld8(&PmT[trow * BP + 32 * s + 8 * kq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * (4 * kh + j) + li;
          f32x4 x4 = zero4(), y2 = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) x4 = mfma(za[s], ld8(&Hs[kcm(kr, 32 * s + 8 * kq, kHead)]), x4);
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (32 * s + 31 >= 16 * tw)  // (dP o Gamma)[i][t] needs i >= t
              y2 = mfma(pta[s], col8(S.Qs, 32 * s + 8 * kq, kr - li, lane), y2);
          const int tr = 16 * tw + 4 * kq;
          const float4 kv = col4_bf16(S.Ks, tr, kr - li, lane);
          const float ka_[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = tr + r;
            const float e = S.eg[t], bt = S.bet[t];
            adk[j][r] += y2[r] - bt * e * x4[r];
            const float zk = -ka_[r] * x4[r];          // k^ . (T^T dW)
            br[r] += e * zk;
            gr[r] += bt * e * zk;
          }
        }
      }
      // Requests: the own rows of D (pass 3), then V and T, T^T, staged into
      // LDS once Z and the P tiles are dead.
      bf16x8 da[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        da[s] = __builtin_bit_cast(bf16x8, ld16_nt(Db + kcm(trow, 32 * s + 8 * kq, kChunk)));
      // (last reads of D, T and T^T in this kernel: non-temporal; the chunks of
      // the zero tiles, which are not stored, come from past the end of a
      // range-checked buffer as zeros: chunk tid is row tid % 64, columns
      // 8 (tid / 64) ..)
      const __amdgpu_buffer_rsrc_t rT = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(Tg), 0, 2 * kTBytes, kBufferWord3);
      const int tcb = tid >> 7, trb = (tid & 63) >> 4;  // column and row tile of the chunk
      const uint4 tst0 = load_b128_nt(rT, tcb <= trb ? 16 * tid : 2 * kTBytes);             // T
      const uint4 tst1 = load_b128_nt(rT, tcb >= trb ? kTBytes + 16 * tid : 2 * kTBytes);   // T^T
      {  // pass 2: x3 -> dW
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * (4 * kh + j) + li;
          f32x4 x3 = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) x3 = mfma(ea[s], ld8(&Hs[kcm(kr, 32 * s + 8 * kq, kHead)]), x3);
          const int tr = 16 * tw + 4 * kq;
#pragma unroll
          for (int r = 0; r < 4; ++r) dWs[(tr + r) * KP + kr] = f2bf(-x3[r]);
        }
      }
      {
        // <h, dh'> over the whole state
        float hd = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = tid + 512 * i;
          hd += dot8u(*reinterpret_cast<const uint4*>(&Hs[8 * e]),
                      *reinterpret_cast<const uint4*>(&Gs[8 * e]));
        }
        hd = wave_sum_uniform(hd);
        if (lane == 0) S.hd_part[wave] = hd;
      }
      {  // pass 3: x2 -> dk^
        float glp = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * (4 * kh + j) + li;
          f32x4 x2 = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s) x2 = mfma(da[s], ld8(&Gs[kcm(kr, 32 * s + 8 * kq, kHead)]), x2);
          const int tr = 16 * tw + 4 * kq;
          const float4 kv = col4_bf16(S.Ks, tr, kr - li, lane);
          const float ka_[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = tr + r;
            const float bw = S.ebw[t];
            adk[j][r] += bw * x2[r];
            const float dc = ka_[r] * x2[r];
            gr[r] -= bw * dc;                            // K_bwd decay, token side
            glp += bw * dc;                              // K_bwd decay, gamma_L side
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gr[r] = sum16_lane0(gr[r]);
          br[r] = sum16_lane0(br[r]);
        }
        if (li == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            S.rowG[kh][16 * tw + 4 * kq + r] = gr[r];
            S.rowB2[kh][16 * tw + 4 * kq + r] = br[r];
          }
        }
        glp = wave_sum_uniform(glp);
        if (lane == 0) S.gl_part[wave] = glp;
      }
      lds_barrier();  // every wave is done with Z, the P tiles, Hs and Gs, and dW is whole
      // V rows from the pieces the waves read for dbeta (together the whole tile)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(&S.rz.V[trow * KP + 16 * (4 * kh + j) + 4 * kq]) = vr[j];
      // T rows into Pm, T^T rows into PmT (chunk e = tid: row tid % 64, columns 8 (tid / 64) ..)
      *reinterpret_cast<uint4*>(&Pm[(tid & 63) * BP + (tid >> 6) * 8]) = tst0;
      *reinterpret_cast<uint4*>(&PmT[(tid & 63) * BP + (tid >> 6) * 8]) = tst1;
      // (after the stores above, which wait for their own requests only)
      if (jg + 1 < G) copy_states(c, hv + 1, wave, lane);
      lds_barrier();

      // ---- dT = dD (beta V)^T + dW (beta e^gamma K^)^T, strictly lower
      //      (wave: row tile tw, col tiles kh, kh + 2)
      {
        bf16x8 wa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) wa[s] = ld8(&dWs[trow * KP + 32 * s + 8 * kq]);
        f32x4 acc[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int mb = kh + 2 * q2;
          f32x4 a1 = zero4(), a2 = zero4();
          if (mb <= tw) {
            const int mrow = 16 * mb + li;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              a1 = mfma(ea[s], ld8(&S.rz.V[mrow * KP + 32 * s + 8 * kq]), a1);
              a2 = mfma(wa[s], ld8(&S.Ks[mrow * KP + 32 * s + 8 * kq]), a2);
            }
          }
          const int m = 16 * mb + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * tw + 4 * kq + r;
            acc[q2][r] = i > m ? S.bet[m] * (a1[r] + S.eg[m] * a2[r]) : 0.f;
          }
        }
        lds_barrier();  // every wave has read V and dW
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int m = 16 * (kh + 2 * q2) + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) S.rz.dT[(16 * tw + 4 * kq + r) * BP + m] = f2bf(acc[q2][r]);
        }
      }
      lds_barrier();

      // ---- Y1 = dT T^T (i > j), stored transposed. Also the own rows of T^T
      //      for dA, read here so that the barrier below orders them before M
      //      overwrites the tile.
      bf16x8 tta[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) tta[s] = ld8(&PmT[trow * BP + 32 * s + 8 * kq]);
      {
        bf16x8 ta[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) ta[s] = ld8(&S.rz.dT[trow * BP + 32 * s + 8 * kq]);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int jb = kh + 2 * q2;
          f32x4 acc = zero4();
          if (jb <= tw) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
              acc = mfma(ta[s], ld8(&Pm[(16 * jb + li) * BP + 32 * s + 8 * kq]), acc);
          }
          const int j = 16 * jb + li;
          float y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = (16 * tw + 4 * kq + r) > j ? acc[r] : 0.f;
          *reinterpret_cast<uint2*>(&Y1T[j * BP + 16 * tw + 4 * kq]) =
              pack4_bf16(y[0], y[1], y[2], y[3]);
        }
      }
      lds_barrier();

      // ---- dA = -T^T Y1 (i > j); M = dA o beta_i Gamma -> Pm, PmT; E = dA o A sums; dbeta of A
      {
        float re[4] = {0.f, 0.f, 0.f, 0.f}, rb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const int jb = kh + 2 * q2;
          const int j = 16 * jb + li;
          float mv[4] = {0.f, 0.f, 0.f, 0.f};
          if (jb <= tw) {
            f32x4 acc = zero4(), kk = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s)
              if (32 * s + 31 >= 16 * tw)
                acc = mfma(tta[s], ld8(&Y1T[(16 * jb + li) * BP + 32 * s + 8 * kq]), acc);
#pragma unroll
            for (int s = 0; s < 4; ++s)
              kk = mfma(ld8(&S.Ks[trow * KP + 32 * s + 8 * kq]),
                        ld8(&S.Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), kk);
            float colp = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 16 * tw + 4 * kq + r;
              if (i > j) {
                const float da_ = -acc[r];
                const float dec = exp2_fast(S.gam[i] - S.gam[j]);
                const float m_ = da_ * S.bet[i] * dec;
                const float e_ = m_ * kk[r];
                mv[r] = m_;
                rb[r] += da_ * dec * kk[r];
                re[r] += e_;
                colp += e_;
              }
            }
            colp = sum_over_rows(colp);
            if (kq == 0) S.colE[wave][j] = colp;
          } else if (kq == 0) {
            S.colE[wave][j] = 0.f;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) Pm[(16 * tw + 4 * kq + r) * BP + j] = f2bf(mv[r]);
          *reinterpret_cast<uint2*>(&PmT[j * BP + 16 * tw + 4 * kq]) =
              pack4_bf16(mv[0], mv[1], mv[2], mv[3]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          re[r] = sum16_lane0(re[r]);
          rb[r] = sum16_lane0(rb[r]);
        }
        if (li == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            S.rowE[kh][16 * tw + 4 * kq + r] = re[r];
            S.rowB3[kh][16 * tw + 4 * kq + r] = rb[r];
          }
        }
      }
      lds_barrier();

      // ---- dk^ += M K^ + M^T K^
      {
        bf16x8 ma[2], mta[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          ma[s] = ld8(&Pm[trow * BP + 32 * s + 8 * kq]);
          mta[s] = ld8(&PmT[trow * BP + 32 * s + 8 * kq]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = 16 * (4 * kh + j) + li;
          f32x4 acc = adk[j];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 kc = col8(S.Ks, 32 * s + 8 * kq, kr - li, lane);
            if (32 * s <= 16 * tw + 15) acc = mfma(ma[s], kc, acc);
            if (32 * s + 31 >= 16 * tw) acc = mfma(mta[s], kc, acc);
          }
          adk[j] = acc;
        }
      }
      // No barrier here: up to its first barrier the next value head writes
      // only the gates (wave 0), which nothing after the barrier above reads;
      // its later writes follow that first barrier, which every wave reaches
      // after the reads above.
    }

    {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      if ((tid >> 6) == 0) dg_out(h * G + G - 1, G - 1, tid & 63);
      else if ((tid >> 6) == 1) db_out(h * G + G - 1, G - 1, tid & 63);
    }

    // every wave is done with Hs, Gs, the P tiles and the dW / Y1^T region:
    // the next item's copies go out now
    lds_barrier();
    prefetch(it + (int)gridDim.x);

    // ---- L2-norm backward and scale: x^ . dx^ over all 128 columns (two halves).
    //      x^ are the normalised rows every product above used (Ks; Qs holds
    //      q~ = scale q^), so the raw rows are not read again. (LDS barriers
    //      only, so that nothing here waits for the copies just issued.)
    {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63, wave = tid >> 6;
      const int tw = wave & 3, kh = wave >> 2;
      const int li = lane & 15, kq = lane >> 4;
      float dq_[4] = {0.f, 0.f, 0.f, 0.f}, dk_[4] = {0.f, 0.f, 0.f, 0.f};
      float qh[4][4], kh_[4][4];  // q^, k^ of the thread's 16 elements
      const float inv_scale = 1.f / scale;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tw + 4 * kq + r;
          const int kc = 16 * (4 * kh + j) + li;
          // (rows past the chunk's end hold zeros)
          const float qs = bf2f(S.Qs[t * KP + kc]), kv = bf2f(S.Ks[t * KP + kc]);
          qh[j][r] = qs * inv_scale;
          kh_[j][r] = kv;
          dq_[r] += qs * adq[j][r];
          dk_[r] += kv * adk[j][r];
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dq_[r] = sum16_lane0(dq_[r]);
        dk_[r] = sum16_lane0(dk_[r]);
      }
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          S.dot_q[kh][16 * tw + 4 * kq + r] = dq_[r];
          S.dot_k[kh][16 * tw + 4 * kq + r] = dk_[r];
        }
      }
      lds_barrier();
      // (every LDS read of this step before its first write: in that order the
      // compiler places no wait for the copies just issued inside the step)
      float dotq[4], dotk[4], iq[4], ik[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tw + 4 * kq + r;
        dotq[r] = S.dot_q[0][t] + S.dot_q[1][t];
        dotk[r] = S.dot_k[0][t] + S.dot_k[1][t];
        iq[r] = S.inv_q[t];
        ik[r] = S.inv_k[t];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tw + 4 * kq + r;
          const int kc = 16 * (4 * kh + j) + li;
          const float dqh = scale * adq[j][r];
          S.rz.dq[t * KP + kc] = f2bf((dqh - qh[j][r] * dotq[r]) * iq[r]);
          S.Ks[t * KP + kc] = f2bf((adk[j][r] - kh_[j][r] * dotk[r]) * ik[r]);
        }
    }
    lds_barrier();
    {
      // rows tid / 16 and tid / 16 + 32, columns 8 (tid % 16) ..
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int sg = tid & 15;
      uint4 xq[2], xk[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = (tid >> 4) + 32 * j;
        xq[j] = *reinterpret_cast<const uint4*>(&S.rz.dq[t * KP + sg * 8]);
        xk[j] = *reinterpret_cast<const uint4*>(&S.Ks[t * KP + sg * 8]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = (tid >> 4) + 32 * j;
        if (t < L) {
          const size_t off = ((size_t)(t0 + t) * H + h) * kHead + sg * 8;
          *reinterpret_cast<uint4*>(dq + off) = xq[j];
          *reinterpret_cast<uint4*>(dk + off) = xk[j];
        }
      }
    }
  }
}

hipError_t launch_bwd_dh_scan(const int32_t* seq_first, int N, int HV, int NC,
                              const ChunkInfo* table, const PrepOut& prep, const uint16_t* dO,
                              const float* dhT, float* dh0, const BwdBufs& bufs,
                              hipStream_t stream) {
  const long chains = (long)N * HV;
  const long group = 8L * prep.G;
  const long blocks = (chains + group - 1) / group * group * (kHead / kScanVB);
  hipLaunchKernelGGL(bwd_dh_scan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, seq_first,
                     N, HV, NC, table, prep, dO, dhT, dh0, bufs);
  return hipGetLastError();
}

hipError_t launch_bwd_chunk(const ChunkInfo* table, int NC, int H, int HV, float scale,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const uint16_t* saved,
                            const uint16_t* Tmat, const float* gE, const float* gB,
                            const BwdBufs& bufs, const uint16_t* dO,
                            uint16_t* dq, uint16_t* dk, uint16_t* dv, float* dg, float* dbeta,
                            hipStream_t stream) {
  // one workgroup per CU (its LDS allows no second one), each looping over
  // the items c H + h, c H + h + grid, ...
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long items = (long)NC * H;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::max(1L, std::min(items, (long)cus));
  // dg and dbeta of two value heads of a key head in one 8-byte store
  const bool pair = (HV / H) % 2 == 0 && (reinterpret_cast<uintptr_t>(dg) & 7) == 0 &&
                    (reinterpret_cast<uintptr_t>(dbeta) & 7) == 0;
  if (pair)
    hipLaunchKernelGGL(bwd_chunk_kernel<true>, dim3(grid), dim3(512), 0, stream, table, NC, H, HV,
                       scale, q, k, v, g, beta, saved, Tmat, gE, gB, bufs, dO, dq, dk, dv, dg, dbeta);
  else
    hipLaunchKernelGGL(bwd_chunk_kernel<false>, dim3(grid), dim3(512), 0, stream, table, NC, H, HV,
                       scale, q, k, v, g, beta, saved, Tmat, gE, gB, bufs, dO, dq, dk, dv, dg, dbeta);
  return hipGetLastError();
}

}  // namespace gdn
