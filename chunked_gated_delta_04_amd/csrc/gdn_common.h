// Device helpers shared by the gfx950 kernels of the gated delta rule.
//
// MFMA fragment layout used throughout (v_mfma_f32_16x16x32_bf16, wave64):
// lane l = 16*kq + i (i = l & 15, kq = l >> 4) supplies
//   A[i][kb + 8*kq .. kb + 8*kq + 7]      (8 bf16, one 16-byte read)
//   B[kb + 8*kq .. kb + 8*kq + 7][i]
// and receives C[4*kq + r][i], r = 0..3. Every operand is therefore read as
// 8 consecutive bf16 along the contraction axis, and the kernels keep each
// operand in the memory layout that makes that read contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));  // 16 raw bytes in registers

constexpr int kHead = 128;   // K = V
constexpr int kChunk = 64;   // tokens per chunk
constexpr float kNormEps = 1e-6f;
constexpr int kScanVB = 32;  // value columns per workgroup of the state scans
// per-token gate factors of a block: e^gamma, e^(gamma_L - gamma), beta
constexpr int kGates = 3 * kChunk;
// per-token values of a block that only the backward reads: gamma (base 2), beta
constexpr int kGatesB = 2 * kChunk;

// Tile layout of every intermediate matrix that a kernel reads as MFMA
// operands from global memory: an R x C tile (C the contraction axis) is
// stored as C/8 column chunks, each holding the R rows' 8 consecutive
// elements (16 bytes) back to back. An operand fragment (16 rows, 8 columns
// per lane) is then four runs of 256 contiguous bytes, and the stores of an
// MFMA accumulator tile (4 consecutive contraction indices per lane) fill
// whole cache lines. Row-major fragments, by contrast, touch 16 half lines
// per instruction and stream about four times slower through a CU.
__device__ __host__ __forceinline__ int kcm(int r, int c, int R) {
  return ((c >> 3) * R + r) * 8 + (c & 7);
}

// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format, no swizzle). A raw buffer store whose byte offset lies at or past
// the resource's record count is discarded by the hardware, which lets a
// kernel mask the rows past a chunk's end without a branch.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of a load: non-temporal (streamed data read once, kept from
// displacing reused lines in L2).
constexpr int kNonTemporal = 2;

__device__ __forceinline__ void store_b64(uint2 v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, byte_off, 0, 0);
}

__device__ __forceinline__ void store_b128(uint4 v, __amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, byte_off, 0, 0);
}

// Raw buffer loads; zeros where the offset is past the record count.
__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 load_b64(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ bf16x8 ld8_buf(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(bf16x8, load_b128(r, byte_off));
}
// The same, non-temporal (the last read of the data in the kernel).
__device__ __forceinline__ uint4 load_b128_nt(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kNonTemporal);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Non-temporal (streaming) stores of 8 and 16 bytes: for outputs that the
// writing kernel does not read again, so that they do not displace lines it
// reuses.
__device__ __forceinline__ void st8_nt(uint16_t* p, uint2 x) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v;
  v[0] = x.x;
  v[1] = x.y;
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st16_nt(uint16_t* p, uint4 x) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v;
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> two bf16 (round to nearest even) in one 32-bit word, a in the
// low half; one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pk2(a, b), pk2(c, d));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 8 fp32 from LDS/global -> bf16x8 (round to nearest even)
__device__ __forceinline__ bf16x8 cvt8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  return __builtin_bit_cast(bf16x8, make_uint4(pk2(a.x, a.y), pk2(a.z, a.w), pk2(b.x, b.y), pk2(b.z, b.w)));
}

// 8 fp32 values times 8 per-column factors, as a bf16 MFMA operand fragment
__device__ __forceinline__ bf16x8 cvt8s(const float* p, const float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float4 fa = *reinterpret_cast<const float4*>(f);
  const float4 fb = *reinterpret_cast<const float4*>(f + 4);
  return __builtin_bit_cast(bf16x8, make_uint4(pk2(a.x * fa.x, a.y * fa.y), pk2(a.z * fa.z, a.w * fa.w),
                                               pk2(b.x * fb.x, b.y * fb.y), pk2(b.z * fb.z, b.w * fb.w)));
}

// log2(e): decays are kept as base-2 exponents so that e^x is one v_exp_f32
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt operand that waits for every vector-memory request of the wave
// (vmcnt = 0) and leaves the export and LDS counters alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

// s_waitcnt operand that waits for every LDS (and scalar-memory) request of
// the wave (lgkmcnt = 0) and leaves the vector-memory and export counters alone.
constexpr int kWaitLgkm0 = 0xF | (7 << 4) | (3 << 14);

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// the wave's global requests - in particular not for global-to-LDS copies
// still in flight, whose readers wait for them (s_waitcnt vmcnt) themselves.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS transpose read (ds_read_b64_tr_b16, gfx950). Within each group of 16
// lanes, lane j supplies the address of 4 consecutive 16-bit elements; lane i
// of the group receives element i % 4 of lanes i / 4, 4 + i / 4, 8 + i / 4
// and 12 + i / 4. When lanes 4 e .. 4 e + 3 read row e of a row-major tile in
// four 4-element pieces, lane i therefore receives column i of those 4 rows.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

// Column c0 + (lane % 16) of rows r0 .. r0 + 7 of a row-major bf16 LDS tile
// (pitch in elements, a multiple of 4; c0 a multiple of 16), as 16 bytes:
// two transpose reads, each lane group of the wave taking its own r0, c0.
__device__ __forceinline__ uint4 lds_col8(const uint16_t* tile, int pitch, int r0, int c0,
                                          int lane) {
  const int j = lane & 15;
  const uint2 a = lds_tr16(tile + (r0 + (j >> 2)) * pitch + c0 + 4 * (j & 3));
  const uint2 b = lds_tr16(tile + (r0 + 4 + (j >> 2)) * pitch + c0 + 4 * (j & 3));
  return make_uint4(a.x, a.y, b.x, b.y);
}

// The same for a 16-column tile held as two column groups of 8 in the
// chunk-major layout (row r of a group at 8 r, 16 bytes per row): ga holds
// columns 0-7, gb columns 8-15. Lane i of a lane group receives column i of
// rows r0 .. r0 + 7 (r0 per lane group).
__device__ __forceinline__ uint4 lds_col8_cm(const uint16_t* ga, const uint16_t* gb, int r0,
                                             int lane) {
  const int j = lane & 15;
  const uint16_t* p = ((j & 2) ? gb : ga) + (r0 + (j >> 2)) * 8 + 4 * (j & 1);
  const uint2 a = lds_tr16(p);
  const uint2 b = lds_tr16(p + 32);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// One fp32 MFMA step (16 x 16 x 4): lane 16 kk + i supplies A[i][kk] and
// B[kk][i]; the accumulator holds C[4 kk + r][i] in element r.
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// In-place inverse of I + A for a strictly lower-triangular 64 x 64 fp32 matrix A
// in LDS (row pitch 68): on return T = (I + A)^-1, unit lower triangular, with
// zeros above the diagonal blocks as on entry. Blocked in 16 x 16: each
// diagonal block by forward substitution (one column per lane of wave 3), then
// the blocks below the diagonal from T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj,
// column j on wave j (j = 0, 1, 2), top to bottom, with fp32 MFMA (the sum into
// the wave's scratch tile, then the product with T_ii). A column uses only the
// diagonal blocks and its own earlier blocks, so the columns need no barrier
// between them; each wave reads the blocks of A it contracts into registers
// before the one barrier (while wave 3 solves the diagonal), because the
// blocks are overwritten in place by other columns. scratch: 768 floats. Must
// be called by all threads of the workgroup (at least 4 waves; it
// synchronises). Fixed summation order.
__device__ __forceinline__ void invert_unit_lower_64(float* M, float* scratch, int tid) {
  constexpr int P = 68;
  const int jb = tid >> 6, lane = tid & 63, li = lane & 15, kk = lane >> 4;
  // a[i - 1][m][s]: A_im as the MFMA operand of k-step s (lane: row li, column 4 s + kk)
  float a[3][3][4];
  if (jb < 3) {
#pragma unroll
    for (int ib = 1; ib < 4; ++ib)
#pragma unroll
      for (int mb = 0; mb < 3; ++mb)
        if (mb < ib && mb >= jb) {
#pragma unroll
          for (int s = 0; s < 4; ++s) a[ib - 1][mb][s] = M[(16 * ib + li) * P + 16 * mb + 4 * s + kk];
        }
  } else if (jb == 3) {
    // diagonal blocks: lane = column jc of block o16 / 16 (this wave alone reads
    // and then writes them; its LDS operations complete in order)
    const int o16 = 16 * (lane >> 4), jc = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == jc ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= M[(o16 + i) * P + o16 + m] * x[m];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) M[(o16 + i) * P + o16 + jc] = x[i];
  }
  __syncthreads();
  if (jb < 3) {
    float* St = scratch + 256 * jb;
#pragma unroll
    for (int ib = 1; ib < 4; ++ib) {
      if (ib > jb) {  // S = sum_m A_(ib, m) T_(m, jb); T_(ib, jb) = -T_(ib, ib) S
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mb = 0; mb < 3; ++mb)
          if (mb < ib && mb >= jb) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc = mfma_f32_k4(a[ib - 1][mb][s], M[(16 * mb + 4 * s + kk) * P + 16 * jb + li], acc);
          }
#pragma unroll
        for (int r = 0; r < 4; ++r) St[(4 * kk + r) * 16 + li] = acc[r];
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          d = mfma_f32_k4(M[(16 * ib + li) * P + 16 * ib + 4 * s + kk], St[(4 * s + kk) * 16 + li], d);
#pragma unroll
        for (int r = 0; r < 4; ++r) M[(16 * ib + 4 * kk + r) * P + 16 * jb + li] = -d[r];
      }
    }
  }
  __syncthreads();
}

// Saved-for-backward block of one (chunk, value head): the chunk-start state
// h = S^T in bf16 as [v / 32][v % 32 / 8][k][v % 8] (each scan workgroup
// writes one contiguous 8 KiB piece), then the chunk's D [tok][v] in bf16,
// chunk-major (kcm).
constexpr int kSavedH = kHead * kHead;
constexpr int kSavedBlock = kSavedH + kChunk * kHead;
__device__ __host__ __forceinline__ size_t blk_saved(int c, int hv, int HV) {
  return ((size_t)c * HV + hv) * kSavedBlock;
}

// Sum over the 64 lanes of a wave; every lane gets the total. Fixed order.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// DPP row shifts inside each 16-lane row of the wave; a lane whose source
// falls outside its row reads 0.
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {  // lane i <- lane i - N
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float dpp_row_shl(float x) {  // lane i <- lane i + N
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_value(float x, int l) {  // x of lane l (l uniform)
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Sum of each 16-lane row, complete in the row's first lane (the others hold
// partial sums): lane i adds lane i + 1, 2, 4, 8.
__device__ __forceinline__ float row_sum_first_lane(float x) {
  x += dpp_row_shl<1>(x);
  x += dpp_row_shl<2>(x);
  x += dpp_row_shl<4>(x);
  x += dpp_row_shl<8>(x);
  return x;
}

// Inclusive prefix sum over the 64 lanes, in a fixed order: a scan inside
// each 16-lane row, then the totals of the earlier rows, nearest first.
// lane: the caller's lane index.
__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
  x += dpp_row_shr<1>(x);
  x += dpp_row_shr<2>(x);
  x += dpp_row_shr<4>(x);
  x += dpp_row_shr<8>(x);
  const float r0 = lane_value(x, 15), r1 = lane_value(x, 31), r2 = lane_value(x, 47);
  const int row = lane >> 4;
  if (row == 3) x += r2;
  if (row >= 2) x += r1;
  if (row >= 1) x += r0;
  return x;
}

// Suffix sum (lane t: lanes t .. 63) in a fixed order: a reverse scan inside
// each row, then the totals of the later rows, nearest first.
__device__ __forceinline__ float wave_suffix_sum(float x, int lane) {
  x = row_sum_first_lane(x);
  const float r1 = lane_value(x, 16), r2 = lane_value(x, 32), r3 = lane_value(x, 48);
  const int row = lane >> 4;
  if (row == 0) x += r1;
  if (row <= 1) x += r2;
  if (row <= 2) x += r3;
  return x;
}

// Sum over the 64 lanes, the same value in every lane, in a fixed order.
__device__ __forceinline__ float wave_sum_uniform(float x) {
  x = row_sum_first_lane(x);
  return ((lane_value(x, 0) + lane_value(x, 16)) + lane_value(x, 32)) + lane_value(x, 48);
}

// Sum over the four 16-lane rows of the wave (lanes i, i + 16, i + 32,
// i + 48), the same value in all four: the gfx950 row swaps (32-lane halves,
// then 16-lane rows) as VALU operations, (r0 + r2) + (r1 + r3) in every lane.
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over groups of `W` consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// L2 warm-up for the sequential scans. A chain's chunk operands come from HBM
// when they are first requested, a latency of the order of a whole chunk step
// under load; requesting them one chunk ahead therefore still stalls every
// step. Each workgroup instead touches its share of the operand lines of the
// chunk three steps ahead - one 4-byte load per 128-byte line and lane - so
// that the real requests one chunk ahead hit L2. The loaded words are folded
// into a sink two steps after they were requested (by then they have arrived,
// as the counter of outstanding loads drains in order, so the fold waits for
// nothing) and the sink is consumed once at the end of the kernel.
constexpr int kLineElems16 = 64;  // bf16 elements per 128-byte line
constexpr int kLineElems32 = 32;  // fp32 elements per 128-byte line
// Line l (0 .. 39) of the 40 128-byte lines that a 64 x 64 bf16 block holds
// when only its 16 x 16 tiles at or below the diagonal are stored in the
// chunk-major layout of kcm(): column chunk kc (1 KiB, 8 lines of 8 rows)
// holds rows 16 (kc / 2) .. 63, i.e. its lines 2 (kc / 2) .. 7. Returns the
// line's index in the block (0 .. 63).
__device__ __forceinline__ int lower_tile_line(int l) {
  int kc = 0;
#pragma unroll
  for (int x = 0; x < 7; ++x) {
    const int n = 8 - 2 * (kc >> 1);
    if (l >= n) {
      l -= n;
      ++kc;
    }
  }
  return 8 * kc + 2 * (kc >> 1) + l;
}

__device__ __forceinline__ uint32_t touch_line(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ void consume(uint32_t sink) { asm volatile("" ::"v"(sink)); }

// One chunk of the packed token axis: sequence, first token, length, and
// the chunk's position inside its sequence. seq < 0 marks an unused slot.
struct ChunkInfo {
  int seq, t0, len, pos;
};

}  // namespace gdn
