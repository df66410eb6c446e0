// Backward of the chunked gated delta rule: reverse state-gradient scan and
// the per-chunk gradient pass.
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
constexpr int TP = 72;   // LDS pitch (bf16) of [128][64] tiles
constexpr int FP = 68;   // LDS pitch (fp32) of [64][64] tiles

__device__ __forceinline__ void lower_tile(int t, int& ib, int& jb) {
  ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
  jb = t - (ib * (ib + 1)) / 2;
}

__device__ __forceinline__ bf16x8 ld8_or0(const uint16_t* p, bool ok) {
  if (ok) return ld8(p);
  return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

// sum over the 16 lanes of a 16-lane group (lanes sharing kq)
__device__ __forceinline__ float sum16(float x) { return group_sum<16>(x); }
}  // namespace

// ---------------------------------------------------------------------------
// Reverse scan: dh (K x VB slice) in registers, chunks in reverse order.
// Writes per (chunk, value head): dh' as [k][v], dD as [tok][v] and [v][tok].
template <int VB>
__global__ __launch_bounds__(256) void bwd_dh_scan_kernel(
    const int32_t* __restrict__ seq_first, int N, int HV, int NC,
    const ChunkInfo* __restrict__ table, PrepOut prep, const uint16_t* __restrict__ dO,
    const float* __restrict__ dhT, float* __restrict__ dh0, BwdBufs bufs) {
  constexpr int NVB = kHead / VB;
  constexpr int VT = VB / 16;
  constexpr int SP = 136;
  constexpr int DP = 72;

  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int vb = slot % NVB;
  const int chain = (slot / NVB) * 8 + xcd;
  if (chain >= N * HV) return;
  const int seq = chain / HV, hv = chain - seq * HV;
  const int v0 = vb * VB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;

  __shared__ __align__(16) uint16_t Hs[VB * SP];  // dh as [v][k]
  __shared__ __align__(16) uint16_t Os[VB * DP];  // dO^T [v][tok]
  __shared__ __align__(16) uint16_t Es[VB * DP];  // dD^T [v][tok]

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

  const int c_begin = seq_first[seq], c_end = seq_first[seq + 1];
  for (int c = c_end - 1; c >= c_begin; --c) {
    const ChunkInfo ci = table[c];
    const size_t blk = (size_t)hv * NC + c;

    // 1. dh -> LDS; stage dO^T for this value block
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        const int kk = 16 * (2 * wave + dt) + 4 * kq;
        *reinterpret_cast<uint2*>(&Hs[(16 * vt + li) * SP + kk]) =
            pack4_bf16(dh[dt][vt][0], dh[dt][vt][1], dh[dt][vt][2], dh[dt][vt][3]);
      }
    for (int e = tid; e < kChunk * (VB / 8); e += 256) {
      const int t = e / (VB / 8), sg = e - t * (VB / 8);
      uint4 x = make_uint4(0, 0, 0, 0);
      if (t < ci.len)
        x = *reinterpret_cast<const uint4*>(dO + ((size_t)(ci.t0 + t) * HV + hv) * kHead + v0 + 8 * sg);
      const uint16_t* xs = reinterpret_cast<const uint16_t*>(&x);
#pragma unroll
      for (int u = 0; u < 8; ++u) Os[(8 * sg + u) * DP + t] = xs[u];
    }
    __syncthreads();
    // dh' (gradient of this chunk's end state) as [k][v]
    {
      uint16_t* dhb = bufs.dh + blk * (kHead * kHead);
      for (int e = tid; e < kHead * (VB / 8); e += 256) {
        const int kk = e / (VB / 8), vg = e - kk * (VB / 8);
        *reinterpret_cast<uint4*>(dhb + kk * kHead + v0 + 8 * vg) = gather8(&Hs[(8 * vg) * SP + kk], SP);
      }
    }

    // 2. dD = P^T dO + K_bwd dh; wave w owns tokens 16 w .. 16 w + 15
    {
      const uint16_t* PTb = prep.P + blk * 4096;  // P^T: row i holds P[j][i], j >= i
      const uint16_t* Kbb = prep.Kb + blk * 8192; // K_bwd [tok][k]
      bf16x8 pa[2], ka[4];
#pragma unroll
      for (int s = 0; s < 2; ++s) pa[s] = ld8(PTb + (16 * wave + li) * 64 + 32 * s + 8 * kq);
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = ld8(Kbb + (16 * wave + li) * kHead + 32 * s + 8 * kq);
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) {
        f32x4 acc = zero4();
        if (wave < 2) acc = mfma(pa[0], ld8(&Os[(16 * vt + li) * DP + 8 * kq]), acc);
        acc = mfma(pa[1], ld8(&Os[(16 * vt + li) * DP + 32 + 8 * kq]), acc);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = mfma(ka[s], ld8(&Hs[(16 * vt + li) * SP + 32 * s + 8 * kq]), acc);
        // acc[r] = dD[t = 16 w + 4 kq + r][v = 16 vt + li]
        *reinterpret_cast<uint2*>(&Es[(16 * vt + li) * DP + 16 * wave + 4 * kq]) =
            pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    __syncthreads();
    // dD to global as [v][tok] (row copies) and [tok][v] (column gathers)
    {
      uint16_t* dDT = bufs.dDT + blk * 8192;
      uint16_t* dDr = bufs.dD + blk * 8192;
      for (int e = tid; e < VB * 8; e += 256) {
        const int vl = e >> 3, sg = e & 7;
        *reinterpret_cast<uint4*>(dDT + (v0 + vl) * 64 + 8 * sg) =
            *reinterpret_cast<const uint4*>(&Es[vl * DP + 8 * sg]);
      }
      for (int e = tid; e < kChunk * (VB / 8); e += 256) {
        const int t = e / (VB / 8), vg = e - t * (VB / 8);
        *reinterpret_cast<uint4*>(dDr + t * kHead + v0 + 8 * vg) = gather8(&Es[(8 * vg) * DP + t], DP);
      }
    }

    // 3. dh <- e^gamma_L dh + Q_g^T dO - W^T dD; wave w owns key rows 32 w .. 32 w + 31
    {
      const uint16_t* QgT = prep.Qg + blk * 8192;  // Q_g^T [k][tok]
      const uint16_t* WT = prep.W + blk * 8192;    // W^T [k][tok]
      const float gl = prep.gL[blk];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int kr = 16 * (2 * wave + dt) + li;
        bf16x8 qa[2], wa[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          qa[s] = ld8(QgT + kr * 64 + 32 * s + 8 * kq);
          wa[s] = ld8(WT + kr * 64 + 32 * s + 8 * kq);
        }
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
          f32x4 acc = dh[dt][vt] * gl;
          f32x4 acw = zero4();
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            acc = mfma(qa[s], ld8(&Os[(16 * vt + li) * DP + 32 * s + 8 * kq]), acc);
            acw = mfma(wa[s], ld8(&Es[(16 * vt + li) * DP + 32 * s + 8 * kq]), acw);
          }
          dh[dt][vt] = acc - acw;
        }
      }
    }
    __syncthreads();
  }

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
// Per-chunk gradients: one workgroup per (chunk, key head), value heads of the
// key head in order. Wave w owns tokens 16 w .. 16 w + 15 of every
// token-indexed result, so per-token sums stay inside one wave.
__global__ __launch_bounds__(256) void bwd_chunk_kernel(
    const ChunkInfo* __restrict__ table, int NC, int H, int HV, float scale,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const uint16_t* __restrict__ saved, BwdBufs bufs,
    const uint16_t* __restrict__ dO, uint16_t* __restrict__ dq, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta) {
  const int c = blockIdx.x, h = blockIdx.y;
  const ChunkInfo ci = table[c];
  if (ci.seq < 0) return;
  const int t0 = ci.t0, L = ci.len;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, kq = lane >> 4;

  __shared__ __align__(16) uint16_t Ks[64 * KP];   // k^ rows (bf16); dk staging at the end
  __shared__ __align__(16) uint16_t Qs[64 * KP];   // q~ rows (bf16); dq staging at the end
  __shared__ __align__(16) float Ts[64 * FP];      // T
  __shared__ __align__(16) float As[64 * FP];      // A -> F -> dT -> M
  __shared__ __align__(16) float PS[64 * FP];      // P -> E
  __shared__ __align__(16) float G1[64 * FP];      // dP o Gamma -> Y1
  __shared__ __align__(16) uint16_t dWs[128 * TP]; // dW as [k][tok]
  __shared__ float gam[64], bet[64], eg[64], ebw[64], dgam[64], dbet[64];
  __shared__ float nrm_k[64], nrm_q[64];
  __shared__ float Xs[3 * 256];
  __shared__ float red[8];

  // ---- load and normalise q, k (as the forward does), keep the norms
  {
    const int r = tid >> 2, sg0 = (tid & 3) * 4;
    uint4 kr[4], qr[4];
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r < L) {
        const size_t off = ((size_t)(t0 + r) * H + h) * kHead + (sg0 + j) * 8;
        kr[j] = *reinterpret_cast<const uint4*>(k + off);
        qr[j] = *reinterpret_cast<const uint4*>(q + off);
      } else {
        kr[j] = make_uint4(0, 0, 0, 0);
        qr[j] = make_uint4(0, 0, 0, 0);
      }
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qr[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a0 = bf2f(kw[e] & 0xffffu), a1 = bf2f(kw[e] >> 16);
        const float b0 = bf2f(qw[e] & 0xffffu), b1 = bf2f(qw[e] >> 16);
        sk += a0 * a0 + a1 * a1;
        sq += b0 * b0 + b1 * b1;
      }
    }
    sk = group_sum<4>(sk);
    sq = group_sum<4>(sq);
    const float nk = sqrtf(sk + kNormEps), nq = sqrtf(sq + kNormEps);
    if ((tid & 3) == 0) {
      nrm_k[r] = nk;
      nrm_q[r] = nq;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qr[j]);
      uint4 ko, qo;
      uint32_t* kow = reinterpret_cast<uint32_t*>(&ko);
      uint32_t* qow = reinterpret_cast<uint32_t*>(&qo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kow[e] = (uint32_t)f2bf(bf2f(kw[e] & 0xffffu) / nk) |
                 ((uint32_t)f2bf(bf2f(kw[e] >> 16) / nk) << 16);
        qow[e] = (uint32_t)f2bf((bf2f(qw[e] & 0xffffu) / nq) * scale) |
                 ((uint32_t)f2bf((bf2f(qw[e] >> 16) / nq) * scale) << 16);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KP + (sg0 + j) * 8]) = ko;
      *reinterpret_cast<uint4*>(&Qs[r * KP + (sg0 + j) * 8]) = qo;
    }
  }
  __syncthreads();

  // dq~, dk^ accumulated over the value heads: [kt][r] = d[16 w + 4 kq + r][16 kt + li]
  f32x4 adq[8], adk[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    adq[kt] = zero4();
    adk[kt] = zero4();
  }
  const int trow = 16 * wave + li;          // token row this lane supplies as an A operand
  const bool trow_ok = trow < L;

  const int G = HV / H;
  for (int jg = 0; jg < G; ++jg) {
    const int hv = h * G + jg;
    const size_t blk = (size_t)hv * NC + c;
    const uint16_t* hb = saved + blk_saved(c, hv, HV);  // h [k][v]
    const uint16_t* Db = hb + kSavedH;                   // D [tok][v]
    const uint16_t* dhb = bufs.dh + blk * (kHead * kHead);
    const uint16_t* dDb = bufs.dD + blk * 8192;          // dD [tok][v]
    const uint16_t* dDTb = bufs.dDT + blk * 8192;        // dD^T [v][tok]
    const size_t rs = (size_t)HV * kHead;                // token stride of dO, v, dv
    const uint16_t* dOb = dO + ((size_t)t0 * HV + hv) * kHead;
    const uint16_t* vb = v + ((size_t)t0 * HV + hv) * kHead;

    // ---- gates
    if (wave == 0) {
      float gv = lane < L ? g[(size_t)(t0 + lane) * HV + hv] : 0.f;
      const float bv = lane < L ? beta[(size_t)(t0 + lane) * HV + hv] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gv, off, 64);
        if (lane >= off) gv += y;
      }
      gam[lane] = gv;
      bet[lane] = bv;
      const float gl = __shfl(gv, L - 1, 64);
      eg[lane] = expf(gv);
      ebw[lane] = lane < L ? expf(gl - gv) : 0.f;
      dgam[lane] = 0.f;
      dbet[lane] = 0.f;
    }
    __syncthreads();

    // ---- A (lower tiles) and P (all tiles), fp32 in LDS
    for (int job = wave; job < 26; job += 4) {
      if (job < 10) {
        int ib, jb;
        lower_tile(job, ib, jb);
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = mfma(ld8(&Ks[(16 * ib + li) * KP + 32 * s + 8 * kq]),
                     ld8(&Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), acc);
        const int j = 16 * jb + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * kq + r;
          As[i * FP + j] = i > j ? bet[i] * expf(gam[i] - gam[j]) * acc[r] : 0.f;
        }
      } else {
        const int pt = job - 10, ib = pt >> 2, jb = pt & 3;
        f32x4 acc = zero4();
        if (jb <= ib) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = mfma(ld8(&Qs[(16 * ib + li) * KP + 32 * s + 8 * kq]),
                       ld8(&Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), acc);
        }
        const int j = 16 * jb + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ib + 4 * kq + r;
          PS[i * FP + j] = i >= j ? expf(gam[i] - gam[j]) * acc[r] : 0.f;
        }
      }
    }
    for (int e = tid; e < 64 * 64; e += 256) {
      const int i = e >> 6, j = e & 63;
      if ((j >> 4) > (i >> 4)) Ts[i * FP + j] = 0.f;
    }
    __syncthreads();

    // ---- T = (I + A)^-1
    if (tid < 64) {
      const int o16 = 16 * (tid >> 4), jc = tid & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = i == jc ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc -= As[(o16 + i) * FP + o16 + m] * x[m];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(o16 + i) * FP + o16 + jc] = x[i];
    }
    __syncthreads();
    {
      const int r = tid >> 4, cc = tid & 15;
      for (int ib = 1; ib < 4; ++ib) {
        for (int jb = 0; jb < ib; ++jb) {
          float acc = 0.f;
          for (int m = 16 * jb; m < 16 * ib; ++m)
            acc += As[(16 * ib + r) * FP + m] * Ts[m * FP + 16 * jb + cc];
          Xs[jb * 256 + r * 16 + cc] = acc;
        }
        __syncthreads();
        for (int jb = 0; jb < ib; ++jb) {
          float acc = 0.f;
#pragma unroll
          for (int u = 0; u < 16; ++u)
            acc += Ts[(16 * ib + r) * FP + 16 * ib + u] * Xs[jb * 256 + u * 16 + cc];
          Ts[(16 * ib + r) * FP + 16 * jb + cc] = -acc;
        }
        __syncthreads();
      }
    }

    // ---- dP = dO D^T (i >= j): G1 <- dP o Gamma, As <- F = dP o P
    {
      bf16x8 oa[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) oa[s] = ld8_or0(dOb + (size_t)trow * rs + 32 * s + 8 * kq, trow_ok);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4 acc = zero4();
        if (jb <= wave) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = mfma(oa[s], ld8(Db + (16 * jb + li) * kHead + 32 * s + 8 * kq), acc);
        }
        // acc[r] = dP[i = 16 w + 4 kq + r][j = 16 jb + li]
        const int j = 16 * jb + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * wave + 4 * kq + r;
          const bool on = i >= j;
          G1[i * FP + j] = on ? acc[r] * expf(gam[i] - gam[j]) : 0.f;
          As[i * FP + j] = on ? acc[r] * PS[i * FP + j] : 0.f;
        }
      }
    }
    __syncthreads();
    // dgamma_i += sum_j F_ij - sum_j F_ji
    if (tid < 64) {
      float rsum = 0.f, csum = 0.f;
      for (int j = 0; j < 64; ++j) {
        rsum += As[tid * FP + j];
        csum += As[j * FP + tid];
      }
      dgam[tid] += rsum - csum;
    }

    // ---- token-row products of this wave (contractions over v from global)
    {
      float dg_row[4] = {0.f, 0.f, 0.f, 0.f};   // per r: this lane's partial of row 16w+4kq+r
      float dgl_part = 0.f;                     // partial of the dgamma_L term from K_bwd
      bf16x8 oa[4], da[4], ea[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        oa[s] = ld8_or0(dOb + (size_t)trow * rs + 32 * s + 8 * kq, trow_ok);
        da[s] = ld8(Db + trow * kHead + 32 * s + 8 * kq);
        ea[s] = ld8(dDb + trow * kHead + 32 * s + 8 * kq);
      }
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const int kr = 16 * kt + li;  // key column supplied by this lane as B operand
        f32x4 x1 = zero4(), x2 = zero4(), x3 = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 hf = ld8(hb + kr * kHead + 32 * s + 8 * kq);
          x1 = mfma(oa[s], hf, x1);                                        // dO h^T
          x3 = mfma(ea[s], hf, x3);                                        // dD h^T
          x2 = mfma(da[s], ld8(dhb + kr * kHead + 32 * s + 8 * kq), x2);  // D dh'^T
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * kq + r;
          const float qk = bf2f(Qs[t * KP + kr]);
          const float kk = bf2f(Ks[t * KP + kr]);
          adq[kt][r] += eg[t] * x1[r];
          dg_row[r] += eg[t] * qk * x1[r];          // inter-chunk output decay
          adk[kt][r] += ebw[t] * x2[r];
          const float dc = kk * x2[r];
          dg_row[r] -= ebw[t] * dc;                 // K_bwd decay, token side
          dgl_part += ebw[t] * dc;                  // K_bwd decay, gamma_L side
        }
        // dW = -dD h^T stored as [k][tok]
        *reinterpret_cast<uint2*>(&dWs[kr * TP + 16 * wave + 4 * kq]) =
            pack4_bf16(-x3[0], -x3[1], -x3[2], -x3[3]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) dg_row[r] = sum16(dg_row[r]);
      dgl_part = wave_sum(dgl_part);
      __syncthreads();  // dgam row/col pass above is done before these writes
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dgam[16 * wave + 4 * kq + r] += dg_row[r];
      }
      if (lane == 0) red[wave] = dgl_part;
    }

    // ---- dq~ += (dP o Gamma) K^ ; dk^ += (dP o Gamma)^T Q~
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 acq = adq[kt], ack = adk[kt];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 kcol = gather8_bf16(&Ks[(32 * s + 8 * kq) * KP + 16 * kt + li], KP);
        const bf16x8 qcol = gather8_bf16(&Qs[(32 * s + 8 * kq) * KP + 16 * kt + li], KP);
        if (32 * s <= 16 * wave + 15)  // j <= i
          acq = mfma(cvt8(&G1[trow * FP + 32 * s + 8 * kq]), kcol, acq);
        if (32 * s + 31 >= 16 * wave)  // i >= j
          ack = mfma(gather8_f32(&G1[(32 * s + 8 * kq) * FP + trow], FP), qcol, ack);
      }
      adq[kt] = acq;
      adk[kt] = ack;
    }
    __syncthreads();  // dWs complete; G1 free

    // ---- T^T dW: dk^ += diag(beta e^gamma) T^T dW; dbeta, dgamma of the W factor
    {
      float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        f32x4 z = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (32 * s + 31 >= 16 * wave)  // T[m][t] needs m >= t
            z = mfma(gather8_f32(&Ts[(32 * s + 8 * kq) * FP + trow], FP),
                     ld8(&dWs[(16 * kt + li) * TP + 32 * s + 8 * kq]), z);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * kq + r;
          adk[kt][r] += bet[t] * eg[t] * z[r];
          rowp[r] += bf2f(Ks[t * KP + 16 * kt + li]) * z[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) rowp[r] = sum16(rowp[r]);
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * kq + r;
          dbet[t] += eg[t] * rowp[r];
          dgam[t] += bet[t] * eg[t] * rowp[r];
        }
      }
    }

    // ---- dV = diag(beta) T^T dD (written as dv[t][v..v+3]); dbeta of the U factor
    {
      float bp = 0.f;
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) {
        f32x4 z = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (32 * s + 31 >= 16 * wave)
            z = mfma(ld8(dDTb + (16 * vt + li) * 64 + 32 * s + 8 * kq),
                     gather8_f32(&Ts[(32 * s + 8 * kq) * FP + trow], FP), z);
        }
        // z[r] = (T^T dD)[t = trow][v = 16 vt + 4 kq + r]
        if (trow_ok) {
          const int vv = 16 * vt + 4 * kq;
          const uint2 vr = *reinterpret_cast<const uint2*>(vb + (size_t)trow * rs + vv);
          bp += bf2f(vr.x & 0xffffu) * z[0] + bf2f(vr.x >> 16) * z[1] +
                bf2f(vr.y & 0xffffu) * z[2] + bf2f(vr.y >> 16) * z[3];
          const float bt = bet[trow];
          *reinterpret_cast<uint2*>(dv + ((size_t)(t0 + trow) * HV + hv) * kHead + vv) =
              pack4_bf16(bt * z[0], bt * z[1], bt * z[2], bt * z[3]);
        }
      }
      bp += __shfl_xor(bp, 16, 64);
      bp += __shfl_xor(bp, 32, 64);
      __syncthreads();  // the dbet writes of the previous block are done
      if (kq == 0) dbet[trow] += bp;
    }

    // ---- dT = dD (beta V)^T + dW (beta e^gamma K^)^T, strictly lower -> As
    {
      bf16x8 ea[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) ea[s] = ld8(dDb + trow * kHead + 32 * s + 8 * kq);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f32x4 a1 = zero4(), a2 = zero4();
        if (mb <= wave) {
          const int mrow = 16 * mb + li;
          const bool mok = mrow < L;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            a1 = mfma(ea[s], ld8_or0(vb + (size_t)mrow * rs + 32 * s + 8 * kq, mok), a1);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            a2 = mfma(gather8_bf16(&dWs[(32 * s + 8 * kq) * TP + trow], TP),
                      ld8(&Ks[mrow * KP + 32 * s + 8 * kq]), a2);
        }
        const int m = 16 * mb + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * wave + 4 * kq + r;
          As[i * FP + m] = i > m ? bet[m] * (a1[r] + eg[m] * a2[r]) : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- Y1 = dT T^T (lower) -> G1
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      f32x4 acc = zero4();
      if (jb <= wave) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc = mfma(cvt8(&As[trow * FP + 32 * s + 8 * kq]),
                     cvt8(&Ts[(16 * jb + li) * FP + 32 * s + 8 * kq]), acc);
      }
      const int j = 16 * jb + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * wave + 4 * kq + r;
        G1[i * FP + j] = i > j ? acc[r] : 0.f;
      }
    }
    __syncthreads();

    // ---- dA = -T^T Y1 (i > j); M = dA o beta_i e^(gamma_i - gamma_j) -> As;
    //      E = dA o A -> PS; dbeta and row part of dgamma of the A factor
    {
      float rb[4] = {0.f, 0.f, 0.f, 0.f}, re[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        f32x4 acc = zero4(), kk = zero4();
        if (jb <= wave) {
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (32 * s + 31 >= 16 * wave)
              acc = mfma(gather8_f32(&Ts[(32 * s + 8 * kq) * FP + trow], FP),
                         gather8_f32(&G1[(32 * s + 8 * kq) * FP + 16 * jb + li], FP), acc);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            kk = mfma(ld8(&Ks[trow * KP + 32 * s + 8 * kq]),
                      ld8(&Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), kk);
        }
        const int j = 16 * jb + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * wave + 4 * kq + r;
          float mval = 0.f, eval = 0.f;
          if (i > j) {
            const float da = -acc[r];
            const float dec = expf(gam[i] - gam[j]);
            mval = da * bet[i] * dec;
            eval = mval * kk[r];
            rb[r] += da * dec * kk[r];
            re[r] += eval;
          }
          As[i * FP + j] = mval;
          PS[i * FP + j] = eval;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rb[r] = sum16(rb[r]);
        re[r] = sum16(re[r]);
      }
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * wave + 4 * kq + r;
          dbet[i] += rb[r];
          dgam[i] += re[r];
        }
      }
    }
    __syncthreads();
    // column part of dgamma of the A factor; gamma_L terms; then dg, dbeta out
    if (tid < 64) {
      float csum = 0.f;
      for (int i = 0; i < 64; ++i) csum += PS[i * FP + tid];
      dgam[tid] -= csum;
    }
    {
      // e^gamma_L <h, dh'> over the whole 128 x 128 state
      float p = 0.f;
      for (int e = tid; e < kHead * kHead / 8; e += 256) {
        const uint4 a = *reinterpret_cast<const uint4*>(hb + 8 * e);
        const uint4 d = *reinterpret_cast<const uint4*>(dhb + 8 * e);
        const uint32_t* aw = reinterpret_cast<const uint32_t*>(&a);
        const uint32_t* dw = reinterpret_cast<const uint32_t*>(&d);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          p += bf2f(aw[u] & 0xffffu) * bf2f(dw[u] & 0xffffu) + bf2f(aw[u] >> 16) * bf2f(dw[u] >> 16);
      }
      p = wave_sum(p);
      if (lane == 0) red[4 + wave] = p;
    }
    __syncthreads();
    if (wave == 0) {
      float x = lane < L ? dgam[lane] : 0.f;
      if (lane == L - 1) {
        const float hh = red[4] + red[5] + red[6] + red[7];
        x += (red[0] + red[1] + red[2] + red[3]) + expf(gam[L - 1]) * hh;
      }
      // reverse inclusive cumsum inside the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(x, off, 64);
        if (lane + off < 64) x += y;
      }
      if (lane < L) {
        dg[(size_t)(t0 + lane) * HV + hv] = x;
        dbeta[(size_t)(t0 + lane) * HV + hv] = dbet[lane];
      }
    }

    // ---- dk^ += M K^ + M^T K^
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      f32x4 ack = adk[kt];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 kcol = gather8_bf16(&Ks[(32 * s + 8 * kq) * KP + 16 * kt + li], KP);
        if (32 * s <= 16 * wave + 15)
          ack = mfma(cvt8(&As[trow * FP + 32 * s + 8 * kq]), kcol, ack);
        if (32 * s + 31 >= 16 * wave)
          ack = mfma(gather8_f32(&As[(32 * s + 8 * kq) * FP + trow], FP), kcol, ack);
      }
      adk[kt] = ack;
    }
    __syncthreads();  // everything is rewritten by the next value head
  }

  // ---- L2-norm backward and scale; stage rows in LDS, then coalesced stores
  {
    float dotq[4] = {0.f, 0.f, 0.f, 0.f}, dotk[4] = {0.f, 0.f, 0.f, 0.f};
    float xq[8][4], xk[8][4];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * kq + r;
        const int kc = 16 * kt + li;
        float qv = 0.f, kv = 0.f;
        if (t < L) {
          const size_t off = ((size_t)(t0 + t) * H + h) * kHead + kc;
          qv = bf2f(q[off]) / nrm_q[t];
          kv = bf2f(k[off]) / nrm_k[t];
        }
        xq[kt][r] = qv;
        xk[kt][r] = kv;
        dotq[r] += qv * scale * adq[kt][r];
        dotk[r] += kv * adk[kt][r];
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dotq[r] = sum16(dotq[r]);
      dotk[r] = sum16(dotk[r]);
    }
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * kq + r;
        const int kc = 16 * kt + li;
        const float dqh = scale * adq[kt][r];
        Qs[t * KP + kc] = f2bf((dqh - xq[kt][r] * dotq[r]) / nrm_q[t]);
        Ks[t * KP + kc] = f2bf((adk[kt][r] - xk[kt][r] * dotk[r]) / nrm_k[t]);
      }
  }
  __syncthreads();
  for (int e = tid; e < 64 * 16; e += 256) {
    const int t = e >> 4, sg = e & 15;
    if (t < L) {
      const size_t off = ((size_t)(t0 + t) * H + h) * kHead + sg * 8;
      *reinterpret_cast<uint4*>(dq + off) = *reinterpret_cast<const uint4*>(&Qs[t * KP + sg * 8]);
      *reinterpret_cast<uint4*>(dk + off) = *reinterpret_cast<const uint4*>(&Ks[t * KP + sg * 8]);
    }
  }
}

constexpr int kBwdVB = 32;

hipError_t launch_bwd_dh_scan(const int32_t* seq_first, int N, int HV, int NC,
                              const ChunkInfo* table, const PrepOut& prep, const uint16_t* dO,
                              const float* dhT, float* dh0, const BwdBufs& bufs,
                              hipStream_t stream) {
  const long chains = (long)N * HV;
  const long groups = (chains + 7) / 8;
  const long blocks = groups * 8 * (kHead / kBwdVB);
  hipLaunchKernelGGL(bwd_dh_scan_kernel<kBwdVB>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     seq_first, N, HV, NC, table, prep, dO, dhT, dh0, bufs);
  return hipGetLastError();
}

hipError_t launch_bwd_chunk(const ChunkInfo* table, int NC, int H, int HV, float scale,
                            const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const uint16_t* saved,
                            const BwdBufs& bufs, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                            uint16_t* dv, float* dg, float* dbeta, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_chunk_kernel, dim3(NC, H), dim3(256), 0, stream, table, NC, H, HV, scale,
                     q, k, v, g, beta, saved, bufs, dO, dq, dk, dv, dg, dbeta);
  return hipGetLastError();
}

}  // namespace gdn
