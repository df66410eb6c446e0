// Chunk table and the per-chunk WY pass of the chunked gated delta rule.
//
// Chunk form (one sequence, one value head, chunk of L <= 64 tokens, start
// state h = S^T of size K x V):
//   gamma   = within-chunk inclusive cumsum of g                (fp32)
//   A_ij    = beta_i e^(gamma_i - gamma_j) k^_i . k^_j, i > j
//   T       = (I + A)^-1                                        (fp32)
//   W       = T diag(beta e^gamma) K^,   U = T diag(beta) V
//   P_ij    = e^(gamma_i - gamma_j) q~_i . k^_j, i >= j
//   Q_g     = diag(e^gamma) Q~,   K_bwd = diag(e^(gamma_L - gamma)) K^
// The state-dependent part (D = U - W h, O = Q_g h + P D,
// h' = e^gamma_L h + K_bwd^T D) runs in the scan kernels, and so does U: the
// forward scan forms it from T and the value rows it reads anyway. This is the
// WY / UT-transform pass that the cake_gdn page (miles PR #3597, "What the
// commits add") lists before its forward state scan, and the chunk
// transition h' = (e^gamma_L I - K_bwd^T W) h + K_bwd^T U written on the
// maxtext page ("Qwen3.5-397B RL trainer on 128 v7x", the gdn_cp_m_scan
// commit). Chunks restart at each sequence start; the last chunk of a
// sequence may be short and is zero-padded, which leaves every product exact.
//
// A workgroup (8 waves; two per CU, each looping over (chunk, key head)
// items) handles one chunk of one key head at a time: q and k are normalised
// once and K^K^T / Q~K^T are formed once on MFMA (held in registers), then
// each value head of the key head gets its gates, A, T and the products
// above. Only e^x of x <= 0 (i >= j) is formed, so strong decays underflow
// to 0.
//
// Outputs, bf16 unless noted, in the layouts the forward scan reads with one
// 16-byte load per MFMA operand; the dh scan reads the same tiles and takes
// the transposed operands it contracts from LDS with transposing reads. Only
// what the backward alone needs is written in addition (when the forward
// saves for it). Per (value head, chunk) block:
//   W        [64 tok][128 k]
//   P        [64 i][64 j]                  (the lower 16 x 16 tiles)
//   T        T [i][j]                      (the lower 16 x 16 tiles), then
//            T^T [j][i]                    (backward only; the upper tiles)
//   gL       e^gamma_L (fp32)
//   gE       e^gamma, e^(gamma_L - gamma) and beta per token (fp32)
//   gB       gamma (base 2) and beta per token (fp32; backward only)
// and per (key head, chunk) block, shared by the key head's value heads:
//   Q~       [64 tok][128 k]
//   K^       K^T [128 k][64 tok]
// The scans apply the per-token decays that turn Q~ into Q_g and K^ into
// K_bwd in fp32: Q_g h = diag(e^gamma) (Q~ h) and K_bwd^T D = K^T (diag(e^(gamma_L
// - gamma)) D), and likewise in the backward.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu, int N,
                                                          int T, int NC,
                                                          ChunkInfo* __restrict__ table,
                                                          int32_t* __restrict__ seq_first) {
  __shared__ int s_scan[256], s_bos[256], s_eos[256];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 256) {
    const int n = base + tid;
    int cnt = 0, bos = 0, eos = 0;
    if (n < N && T > 0) {  // clamp so that device boundaries can never address outside [0, T)
      bos = min(max(cu[n], 0), T);
      eos = min(max(cu[n + 1], bos), T);
      cnt = (eos - bos + kChunk - 1) / kChunk;
    }
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int excl = s_carry + s_scan[tid] - cnt;
    if (n < N) seq_first[n] = min(excl, NC);
    s_bos[tid] = bos;
    s_eos[tid] = eos;
    __syncthreads();
    // the chunks of these sequences, one per thread: chunk m of the block
    // belongs to the first sequence whose inclusive count exceeds m
    const int end = min(s_carry + s_scan[255], NC);
    for (int c = s_carry + tid; c < end; c += 256) {
      const int m = c - s_carry;
      int a = 0, b = 255;
      while (a < b) {
        const int mid = (a + b) >> 1;
        if (s_scan[mid] > m) b = mid; else a = mid + 1;
      }
      const int j = m - (a > 0 ? s_scan[a - 1] : 0);
      ChunkInfo ci;
      ci.seq = base + a;
      ci.t0 = s_bos[a] + kChunk * j;
      ci.len = min(kChunk, s_eos[a] - ci.t0);
      ci.pos = j;
      table[c] = ci;
    }
    __syncthreads();
    if (tid == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  const int total = min(s_carry, NC);
  if (tid == 0) seq_first[N] = total;
  for (int c = total + tid; c < NC; c += 256) {
    ChunkInfo ci;
    ci.seq = -1; ci.t0 = 0; ci.len = 0; ci.pos = 0;
    table[c] = ci;
  }
}

namespace {
constexpr int KP = 136;  // LDS row pitch (bf16) of [64][128] tiles
constexpr int FP = 68;   // LDS row pitch (fp32) of [64][64] tiles

// lower-including 16x16 tile t (0..9) of a 64x64 matrix -> (row block, col block)
__device__ __forceinline__ void lower_tile(int t, int& ib, int& jb) {
  ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
  jb = t - (ib * (ib + 1)) / 2;
}
}  // namespace

constexpr int kPrepThreads = 512;               // 8 waves per workgroup
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int kRowThreads = kPrepThreads / 64;  // threads per token row, 2 x 16 bytes each
                                                // (thread m: bytes 16 m and 16 (m + 8) of the
                                                // row, so a request covers whole lines)

// Writes the forward scan's operands to fo and, with kB (a forward that saves
// for a backward), what only the backward reads to bo (T^T, gamma and beta;
// T itself goes to fo.T, which then points into bo's T blocks), so that the
// backward does not form them again. The backward's dh
// scan reads fo's W, P, Q~ and K^T themselves (transposed in LDS), so a
// forward that saves points those into the saved buffer.
template <bool kB>
__global__ __launch_bounds__(kPrepThreads, 2) void chunk_prep_kernel(
    const ChunkInfo* __restrict__ table, int NC, int H, int HV, float scale,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ g, const float* __restrict__ beta, PrepOut fo, PrepOut bo) {
  // Items (chunk c, key head h) = c H + h, in steps of the grid size; the chunk
  // slots past the pack's chunks are the last ones, so a workgroup stops at
  // its first empty item.
  const int NI = NC * H;
  int it = blockIdx.x;
  if (it >= NI) return;
  ChunkInfo ci = table[it / H];
  if (ci.seq < 0) return;
  const int tid = threadIdx.x;

  __shared__ __align__(16) uint16_t Ks[64 * KP];   // k^ rows (bf16)
  __shared__ __align__(16) uint16_t Qs[64 * KP];   // q~ rows (bf16)
  __shared__ __align__(16) float Ts[64 * FP];      // A (strictly lower), inverted in place into T
  // gates of the value head; gam is the cumulative log-decay in base 2
  __shared__ __align__(16) float gam[64], bet[64], fw[64];
  __shared__ float Xs[3 * 256];  // solve scratch

  // A value head's gates (wave 0) and an item's q, k rows through
  // range-checked buffer loads: rows at or past the chunk's end read as zeros,
  // and a zero range (live = false) moves no data. Each value head's gates are
  // requested one value head ahead, and the next item's q, k rows and first
  // value head's gates during the item's last value head, before that head's
  // stores: waiting for a load also waits for every store issued before it.
  const int G = HV / H;
  uint4 kr[2], qr[2];
  float gq, bq;
  auto request = [&](int t0, int L, int hv_, bool live) {
    const int n = live ? L : 0;
    const int lane = tid & 63;
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(g) + (size_t)t0 * HV + hv_, 0, n * HV * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(beta) + (size_t)t0 * HV + hv_, 0, n * HV * 4, kBufferWord3);
    // (wave 0 alone uses the gates; the other waves' requests fall past the end
    // of the range and move nothing: a gate load touches one line per token)
    const int goff = tid < 64 ? lane * HV * 4 : n * HV * 4;
    gq = load_f32(rg, goff);
    bq = load_f32(rb, goff);
  };
  auto request_qk = [&](int t0, int L, int h, bool live) {
    const int n = live ? L : 0;
    const int r = tid / kRowThreads, sg0 = tid % kRowThreads;
    const __amdgpu_buffer_rsrc_t krng = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(k) + ((size_t)t0 * H + h) * kHead, 0, n * H * kHead * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t qrng = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + ((size_t)t0 * H + h) * kHead, 0, n * H * kHead * 2, kBufferWord3);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      kr[j] = load_b128(krng, (r * H * kHead + (sg0 + kRowThreads * j) * 8) * 2);
      qr[j] = load_b128(qrng, (r * H * kHead + (sg0 + kRowThreads * j) * 8) * 2);
    }
  };

  // ---- 1. L2-normalise the item's q, k rows (thread: row tid / 8, 2 x 8
  //      columns), requested before; one division per row, then products with
  //      the reciprocal. Also waits for the item's first value head's inputs,
  //      requested with them, so that no later wait of the item counts them.
  auto norm_rows = [&]() {
    const int r = tid / kRowThreads, sg0 = tid % kRowThreads;
    float sk = 0.f, sq = 0.f;
    asm volatile("" ::"v"(gq), "v"(bq));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
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
    sk = group_sum<kRowThreads>(sk);
    sq = group_sum<kRowThreads>(sq);
    const float rk = 1.f / sqrtf(sk + kNormEps), rq = scale / sqrtf(sq + kNormEps);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[j]);
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qr[j]);
      uint4 ko, qo;
      uint32_t* kow = reinterpret_cast<uint32_t*>(&ko);
      uint32_t* qow = reinterpret_cast<uint32_t*>(&qo);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kow[e] = pk2(bf2f(kw[e] & 0xffffu) * rk, bf2f(kw[e] >> 16) * rk);
        qow[e] = pk2(bf2f(qw[e] & 0xffffu) * rq, bf2f(qw[e] >> 16) * rq);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KP + (sg0 + kRowThreads * j) * 8]) = ko;
      *reinterpret_cast<uint4*>(&Qs[r * KP + (sg0 + kRowThreads * j) * 8]) = qo;
    }
    __syncthreads();
  };

  {
    const int h = it % H;
    request_qk(ci.t0, ci.len, h, true);
    request(ci.t0, ci.len, h * G, true);
  }
  norm_rows();

  for (;;) {
    const int c = it / H, h = it - c * H;
    const int t0 = ci.t0, L = ci.len;
    // the next item, whose rows the last value head requests
    const int itn = it + (int)gridDim.x;
    const ChunkInfo cin = itn < NI ? table[itn / H] : ChunkInfo{-1, 0, 0, 0};
    const bool next = cin.seq >= 0;

    // K^K^T and Q~K^T tiles of the key head, formed once for all its value heads:
    // kk[n] belongs to job wave + n kPrepWaves of step 3 below (an A tile for
    // jobs 0-9, a P tile at or below the diagonal for jobs 16-31, nothing else)
    constexpr int kJobs = 32 / kPrepWaves;
    f32x4 kk[kJobs];
    {
      const int wave = tid >> 6, lane = tid & 63;
      const int li = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int n = 0; n < kJobs; ++n) {
        const int job = wave + kPrepWaves * n;
        f32x4 acc = zero4();
        if (job < 10) {
          int ib, jb;
          lower_tile(job, ib, jb);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = mfma(ld8(&Ks[(16 * ib + li) * KP + 32 * s + 8 * kq]),
                       ld8(&Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]), acc);
        } else if (job >= 16) {
          const int pt = job - 16, ib = pt >> 2, jb = pt & 3;
          if (jb <= ib) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc = mfma(ld8(&Ks[(16 * jb + li) * KP + 32 * s + 8 * kq]),
                         ld8(&Qs[(16 * ib + li) * KP + 32 * s + 8 * kq]), acc);
          }
        }
        kk[n] = acc;
      }
    }

    for (int jg = 0; jg < G; ++jg) {
      // Re-derive the thread coordinates from an opaque copy each iteration, so
      // that the many LDS and global addresses built from them are formed where
      // they are used instead of being hoisted and kept live across the loop.
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int wave = tid >> 6, lane = tid & 63;
      const int li = lane & 15, kq = lane >> 4;
      const int hv = h * G + jg;
      const size_t blk = (size_t)hv * NC + c;

      // ---- 2. gates: gamma = inclusive cumsum of g inside the chunk (kept in
      //      base 2). This head's gates were requested before; the next head's
      //      are requested now.
      float gv = gq;
      const float bv = bq;
      if (jg + 1 < G) {
        request(t0, L, hv + 1, true);
      } else {
        request_qk(cin.t0, cin.len, itn % H, next);
        request(cin.t0, cin.len, (itn % H) * G, next);
      }
      if (wave == 0) {
        gv = wave_prefix_sum(gv, lane);
        const float g2 = gv * kLog2e;
        const float gl2 = lane_value(g2, L - 1);
        gam[lane] = g2;
        bet[lane] = bv;
        const float e = exp2_fast(g2);
        fw[lane] = bv * e;
        const float bw = lane < L ? exp2_fast(gl2 - g2) : 0.f;
        fo.gE[blk * kGates + lane] = e;
        fo.gE[blk * kGates + kChunk + lane] = bw;
        fo.gE[blk * kGates + 2 * kChunk + lane] = bv;
        if (kB) {
          bo.gB[blk * kGatesB + lane] = g2;  // the gradient pass reads these as they are
          bo.gB[blk * kGatesB + kChunk + lane] = bv;
        }
        if (lane == 0) fo.gL[blk] = exp2_fast(gl2);
      }
      __syncthreads();

      // ---- 3. A (fp32, LDS: 10 lower tiles, 6 zero upper tiles) and P (bf16,
      //      global: the 10 lower tiles), 32 jobs over the waves, from the key
      //      head's tiles kk formed above.
#pragma unroll
      for (int n = 0; n < kJobs; ++n) {
        const int job = wave + kPrepWaves * n;
        if (job < 10) {
          int ib, jb;
          lower_tile(job, ib, jb);
          const f32x4 acc = kk[n];
          const int j = 16 * jb + li;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * kq + r;
            Ts[i * FP + j] = i > j ? bet[i] * exp2_fast(gam[i] - gam[j]) * acc[r] : 0.f;
          }
        } else if (job < 16) {
          // strictly upper 16 x 16 blocks: (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
          const int u = job - 10;
          const int ib = u < 3 ? 0 : u < 5 ? 1 : 2;
          const int jb = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
#pragma unroll
          for (int r = 0; r < 4; ++r) Ts[(16 * ib + 4 * kq + r) * FP + 16 * jb + li] = 0.f;
        } else {
          const int pt = job - 16, ib = pt >> 2, jb = pt & 3;  // P tile (row block ib, col block jb)
          // C = K^ Q~^T tile: C[4kq+r][li] = P-row i = 16 ib + li, cols j = 16 jb + 4kq + r
          const f32x4 acc = kk[n];
          const int i = 16 * ib + li;
          float pv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * jb + 4 * kq + r;
            pv[r] = i >= j ? exp2_fast(gam[i] - gam[j]) * acc[r] : 0.f;
          }
          // (the tiles above the diagonal are zero and are not stored: their
          // readers take zeros from past the end of a range-checked buffer)
          if (jb <= ib) {
            const uint2 pk = pack4_bf16(pv[0], pv[1], pv[2], pv[3]);
            st8_nt(fo.P + blk * (64 * 64) + kcm(i, 16 * jb + 4 * kq, 64), pk);
          }
        }
      }
      __syncthreads();

      // ---- 4. T = (I + A)^-1 in place
      invert_unit_lower_64(Ts, Xs, tid);

      // T in bf16 for the forward scan (U = T diag(beta) V) and the backward's
      // gradient pass, and T^T for the latter: chunk (kc, r) of each holds row
      // r, columns 8 kc .. 8 kc + 7 (the chunks of their zero 16 x 16 tiles,
      // above the diagonal of T and below that of T^T, are not stored)
      {
#pragma unroll
        for (int i = 0; i < 512 / kPrepThreads; ++i) {
          const int e = tid + kPrepThreads * i;
          const int kc = e >> 6, r = e & 63;
          uint4 o4, t4;
          uint32_t* ow = reinterpret_cast<uint32_t*>(&o4);
          uint32_t* tw4 = reinterpret_cast<uint32_t*>(&t4);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int ja = 8 * kc + 2 * u;
            ow[u] = pk2(Ts[r * FP + ja], Ts[r * FP + ja + 1]);
            if (kB) tw4[u] = pk2(Ts[ja * FP + r], Ts[(ja + 1) * FP + r]);
          }
          if ((kc >> 1) <= (r >> 4)) st16_nt(fo.T + blk * 8192 + kcm(r, 8 * kc, 64), o4);
          if (kB && (kc >> 1) >= (r >> 4)) st16_nt(bo.T + blk * 8192 + 4096 + kcm(r, 8 * kc, 64), t4);
        }
      }

      // ---- 5. W = (T diag(beta e^gamma)) K^: the factor scales T's columns as
      //      T becomes an MFMA operand, K^ is read by columns from its row tile.
      //      32 tiles of 16 x 16 over the waves, contraction over the chunk.
      for (int tt = wave; tt < 32; tt += kPrepWaves) {
        // C = K^T (T')^T: C[4kq+r][li] = W[t = 16 tb + li][k = 16 db + 4kq + r]
        const int db = tt >> 2, tb = tt & 3;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint4 kc = lds_col8(Ks, KP, 32 * s + 8 * kq, 16 * db, lane);
          acc = mfma(__builtin_bit_cast(bf16x8, kc),
                     cvt8s(&Ts[(16 * tb + li) * FP + 32 * s + 8 * kq], &fw[32 * s + 8 * kq]), acc);
        }
        const uint2 pk = pack4_bf16(acc[0], acc[1], acc[2], acc[3]);
        st8_nt(fo.W + blk * 8192 + kcm(16 * tb + li, 16 * db + 4 * kq, 64), pk);
      }

      __syncthreads();  // gates, A and T are rewritten for the next value head
    }

    // ---- Q~ (rows) and K^T of the key head, after the value heads so that no
    //      load waits for these stores. K^T's pieces (column chunks of 8
    //      tokens) come from the row tile with transposing LDS reads: a wave
    //      covers one token group tg and 64 consecutive features.
    {
      const int wave = tid >> 6, lane = tid & 63;
      const int li = lane & 15, kq = lane >> 4;
      const size_t kblk = (size_t)h * NC + c;
      auto rows_out = [&](const uint16_t* src, uint16_t* dst) {
        for (int e = tid; e < 64 * 16; e += kPrepThreads) {
          const int sg = e >> 6, t = e & 63;
          st16_nt(dst + kcm(t, sg * 8, 64), *reinterpret_cast<const uint4*>(&src[t * KP + sg * 8]));
        }
      };
      auto cols_out = [&](const uint16_t* src, uint16_t* dst) {
#pragma unroll
        for (int i = 0; i < 1024 / kPrepThreads; ++i) {
          const int e0 = kPrepThreads * i + 64 * wave;  // wave-uniform
          const int tg = e0 >> 7, d0 = (e0 & 127) + 16 * kq;
          st16_nt(dst + kcm(d0 + li, 8 * tg, 128), lds_col8(src, KP, 8 * tg, d0, lane));
        }
      };
      rows_out(Qs, fo.Qn + kblk * 8192);   // Q~ [tok][k]
      cols_out(Ks, fo.Kn + kblk * 8192);   // K^T [k][tok]
    }
    if (!next) break;
    __syncthreads();  // the next item's rows overwrite Ks and Qs
    it = itn;
    ci = cin;
    norm_rows();
  }
}

hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int NC, ChunkInfo* table,
                              int32_t* seq_first, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, NC, table,
                     seq_first);
  return hipGetLastError();
}

hipError_t launch_chunk_prep(PrepMode mode, const ChunkInfo* table, int NC, int H, int HV,
                             float scale, const uint16_t* q, const uint16_t* k, const float* g,
                             const float* beta, const PrepOut& fwd_out, const PrepOut& bwd_out,
                             hipStream_t stream) {
  // two workgroups per CU (their LDS allows no third), each looping over the
  // items c H + h, c H + h + grid, ...
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long items = (long)NC * H;
  if (items <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::max(1L, std::min(items, 2L * cus)));
  switch (mode) {
    case PrepMode::kForward:
      hipLaunchKernelGGL((chunk_prep_kernel<false>), grid, dim3(kPrepThreads), 0, stream, table, NC, H, HV,
                         scale, q, k, g, beta, fwd_out, bwd_out);
      break;
    case PrepMode::kBoth:
      hipLaunchKernelGGL((chunk_prep_kernel<true>), grid, dim3(kPrepThreads), 0, stream, table, NC, H, HV,
                         scale, q, k, g, beta, fwd_out, bwd_out);
      break;
  }
  return hipGetLastError();
}

}  // namespace gdn
