// Causal short convolution in front of the gated delta rule: a depthwise
// filter of width W (2..4) per channel over the tokens of each sequence,
// preceded by the sequence's W - 1 carried inputs (its conv state), with an
// optional bias and SiLU:
//   pre_t = bias_c + sum_{i<W} w[c][i] xe[t - (W - 1) + i],   y_t = act(pre_t)
// (the goldens page "[WS1][CUDA][Qwen3-Next] C6: GDN decode-step goldens and
// recurrent/conv state contract", RL-Kernel PR #469, "What": the conv update,
// its bias and SiLU, the state [num_blocks, dim, W - 1]; the cake_gdn page,
// miles PR #3597, asks for a weight gradient without atomics; the torchtitan
// PR #4389 page for the paged prefill reading and advancing cache slots).
//
// All of it is HBM-bound element-wise work: every kernel streams token rows
// of [T, C] bf16 with each thread owning 4 adjacent channels (one 8-byte load
// per row, 512 contiguous bytes per wave) and walking a 64-token tile, the
// W - 1 previous inputs kept in registers. Sequence boundaries inside a tile
// are found from cu_seqlens (binary search at the tile start, then walking).
// The weight gradient is reduced without atomics: each tile writes its
// per-channel partial sums, two fixed-order passes add them up.
#include "gdn.h"
#include "gdn_common.h"

#include <vector>

#define GDN_API extern "C" __attribute__((visibility("default")))

namespace gdn {
namespace {

constexpr int kTile = 64;     // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kCpt = 4;       // channels per thread
constexpr int kGroup = 16;    // tiles per first-pass reduction group

// Where a sequence's carried inputs come from and its end inputs go.
// Direct: in / out are [N, C, W - 1] (either NULL). Paged: in == out is a pool
// [slots, C, W - 1]; sequence n uses block idx[n] when 0 < idx[n] < slots,
// reading it only when init is NULL or init[n] != 0.
struct ConvStates {
  const uint16_t* in;
  uint16_t* out;
  const int32_t* idx;
  const int32_t* init;
  int slots;
};

__device__ __forceinline__ int seq_of(const int32_t* cu, int N, int t) {
  int a = 0, b = N + 1;  // first i with cu[i] > t, minus one
  while (a < b) {
    const int m = (a + b) >> 1;
    if (cu[m] <= t) a = m + 1; else b = m;
  }
  return min(max(a - 1, 0), N - 1);
}

__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int T, int& bos, int& eos) {
  if (T == 0) {  // no tokens: cu_seqlens may be NULL and is not read
    bos = eos = 0;
    return;
  }
  bos = min(max(cu[n], 0), T);
  eos = min(max(cu[n + 1], bos), T);
}

template <int W>
__device__ __forceinline__ const uint16_t* state_src(const ConvStates& s, int n, int C) {
  if (s.idx) {
    const int sl = s.idx[n];
    if (sl <= 0 || sl >= s.slots || (s.init && s.init[n] == 0)) return nullptr;
    return s.in + (size_t)sl * C * (W - 1);
  }
  return s.in ? s.in + (size_t)n * C * (W - 1) : nullptr;
}

__device__ __forceinline__ void unpack4(uint2 v, float* f) {
  f[0] = bf2f(v.x & 0xffffu); f[1] = bf2f(v.x >> 16);
  f[2] = bf2f(v.y & 0xffffu); f[3] = bf2f(v.y >> 16);
}

__device__ __forceinline__ uint2 ld_row4(const uint16_t* p) {
  return *reinterpret_cast<const uint2*>(p);
}

// sigmoid with one v_exp_f32 and one v_rcp_f32 (about 1 ulp each); for
// p -> -inf, e^-p overflows to inf and the reciprocal gives 0, never NaN
__device__ __forceinline__ float sigmoid_fast(float p) {
  return __builtin_amdgcn_rcpf(1.f + exp2_fast(-p * kLog2e));
}

template <bool kSilu>
__device__ __forceinline__ float act(float p) {
  return kSilu ? p * sigmoid_fast(p) : p;
}

template <bool kSilu>
__device__ __forceinline__ float act_grad(float p) {
  if (!kSilu) return 1.f;
  const float s = sigmoid_fast(p);
  return s * (1.f + p * (1.f - s));
}

// The window of the W - 1 inputs before token t (t inside [bos, eos)) of
// sequence n: x rows at or after bos, the carried state before it.
template <int W>
__device__ __forceinline__ void load_window(float (&win)[kCpt][W - 1], const uint16_t* x,
                                            const uint16_t* sp, int t, int bos, int C, int c0) {
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int pos = t - (W - 1) + k;
    if (pos >= bos) {
      float f[4];
      unpack4(ld_row4(x + (size_t)pos * C + c0), f);
#pragma unroll
      for (int j = 0; j < kCpt; ++j) win[j][k] = f[j];
    } else {
      const int js = pos - bos + (W - 1);  // >= 0 for t >= bos; guarded for malformed bounds
#pragma unroll
      for (int j = 0; j < kCpt; ++j)
        win[j][k] = sp && js >= 0 ? bf2f(sp[(size_t)(c0 + j) * (W - 1) + js]) : 0.f;
    }
  }
}

template <int W>
__device__ __forceinline__ void load_taps(float (&wf)[kCpt][W], float (&bf)[kCpt],
                                          const uint16_t* w, const uint16_t* bias, int c0) {
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
#pragma unroll
    for (int i = 0; i < W; ++i) wf[j][i] = bf2f(w[(size_t)(c0 + j) * W + i]);
    bf[j] = bias ? bf2f(bias[c0 + j]) : 0.f;
  }
}

// ------------------------------------------------------------------ forward
template <int W, bool kSilu>
__global__ __launch_bounds__(kThreads) void conv_fwd_kernel(
    const int32_t* __restrict__ cu, int N, int T, int C, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias, ConvStates st,
    uint16_t* __restrict__ y) {
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  const int t0 = blockIdx.x * kTile, t1 = min(t0 + kTile, T);
  float wf[kCpt][W], bf[kCpt];
  load_taps<W>(wf, bf, w, bias, c0);
  int n = seq_of(cu, N, t0), bos, eos;
  seq_bounds(cu, n, T, bos, eos);
  float win[kCpt][W - 1];
  load_window<W>(win, x, state_src<W>(st, n, C), t0, bos, C, c0);
  for (int tb = t0; tb < t1; tb += 16) {
    uint2 xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      xv[u] = tb + u < t1 ? ld_row4(x + (size_t)(tb + u) * C + c0) : make_uint2(0u, 0u);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = tb + u;
      if (t >= t1) continue;  // (no break: the loop must unroll)
      if (t >= eos) {  // a new sequence starts here
        n = seq_of(cu, N, t);
        seq_bounds(cu, n, T, bos, eos);
        load_window<W>(win, x, state_src<W>(st, n, C), t, bos, C, c0);
      }
      float xf[4], out[4];
      unpack4(xv[u], xf);
#pragma unroll
      for (int j = 0; j < kCpt; ++j) {
        float p = bf[j];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) p += wf[j][i] * win[j][i];
        p += wf[j][W - 1] * xf[j];
        out[j] = act<kSilu>(p);
#pragma unroll
        for (int i = 0; i < W - 2; ++i) win[j][i] = win[j][i + 1];
        win[j][W - 2] = xf[j];
      }
      *reinterpret_cast<uint2*>(y + (size_t)t * C + c0) = pack4_bf16(out[0], out[1], out[2], out[3]);
    }
  }
}

// End inputs of every sequence (its new conv state): the last W - 1 inputs,
// reaching into the carried state when the sequence is shorter than W - 1.
// Each thread reads all its values before writing any, so a paged block is
// read and rewritten in place safely.
template <int W>
__global__ __launch_bounds__(kThreads) void conv_state_out_kernel(
    const int32_t* __restrict__ cu, int N, int T, int C, const uint16_t* __restrict__ x,
    ConvStates st) {
  const int n = blockIdx.x;
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  uint16_t* dst;
  if (st.idx) {
    const int sl = st.idx[n];
    if (sl <= 0 || sl >= st.slots) return;
    dst = st.out + (size_t)sl * C * (W - 1);
  } else {
    if (!st.out) return;
    dst = st.out + (size_t)n * C * (W - 1);
  }
  const uint16_t* sp = state_src<W>(st, n, C);
  int bos, eos;
  seq_bounds(cu, n, T, bos, eos);
  uint16_t v[kCpt][W - 1];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int pos = eos - (W - 1) + k;
    if (pos >= bos) {
      const uint2 r = ld_row4(x + (size_t)pos * C + c0);
      v[0][k] = r.x & 0xffffu; v[1][k] = r.x >> 16; v[2][k] = r.y & 0xffffu; v[3][k] = r.y >> 16;
    } else {
      const int js = pos - bos + (W - 1);
#pragma unroll
      for (int j = 0; j < kCpt; ++j) v[j][k] = sp ? sp[(size_t)(c0 + j) * (W - 1) + js] : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < kCpt; ++j)
#pragma unroll
    for (int k = 0; k < W - 1; ++k) dst[(size_t)(c0 + j) * (W - 1) + k] = v[j][k];
}

// ------------------------------------------------------------------ backward
// Per tile: dpre = dy act'(pre) for the tile's tokens and the W - 1 tokens
// after it (same sequence), dx by gathering w dpre over the taps in a fixed
// order (a sliding set of W - 1 pending positions, each emitted once its last
// tap has been added), the carried-state gradient for a sequence starting in
// the tile, and the tile's partial sums of dw and dbias over its own tokens.
template <int W, bool kSilu>
__global__ __launch_bounds__(kThreads) void conv_bwd_kernel(
    const int32_t* __restrict__ cu, int N, int T, int C, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias, ConvStates st,
    const uint16_t* __restrict__ dy, uint16_t* __restrict__ dx, float* __restrict__ dstate,
    float* __restrict__ part) {
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  const int tile = blockIdx.x;
  const int t0 = tile * kTile, t1 = min(t0 + kTile, T);
  float wf[kCpt][W], bf[kCpt];
  load_taps<W>(wf, bf, w, bias, c0);
  int n = seq_of(cu, N, t0), bos, eos;
  seq_bounds(cu, n, T, bos, eos);
  float win[kCpt][W - 1], pend[kCpt][W - 1];
  load_window<W>(win, x, state_src<W>(st, n, C), t0, bos, C, c0);
#pragma unroll
  for (int j = 0; j < kCpt; ++j)
#pragma unroll
    for (int k = 0; k < W - 1; ++k) pend[j][k] = 0.f;
  float dwp[kCpt][W], dbp[kCpt];
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
    dbp[j] = 0.f;
#pragma unroll
    for (int i = 0; i < W; ++i) dwp[j][i] = 0.f;
  }
  // emit a completed position (all kCpt channels): dx inside the tile, the
  // carried state's gradient before a sequence start that lies inside the tile
  auto emit = [&](int pos, const float (&val)[kCpt]) {
    if (pos >= bos) {
      if (pos >= t0 && pos < t1)
        *reinterpret_cast<uint2*>(dx + (size_t)pos * C + c0) = pack4_bf16(val[0], val[1], val[2], val[3]);
    } else if (pos >= bos - (W - 1) && bos >= t0 && dstate) {
#pragma unroll
      for (int j = 0; j < kCpt; ++j)
        dstate[((size_t)n * C + c0 + j) * (W - 1) + pos - bos + (W - 1)] = val[j];
    }
  };
  auto flush = [&](int tnext) {  // positions tnext - (W - 1) .. tnext - 1 are complete
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
      float v[kCpt];
#pragma unroll
      for (int j = 0; j < kCpt; ++j) v[j] = pend[j][k];
      emit(tnext - (W - 1) + k, v);
    }
  };
  const int tend = min(t1 + W - 1, T);
  bool crossed = false;  // left the last sequence that reaches into the tile
  for (int tb = t0; tb < tend && !crossed; tb += 16) {
    uint2 xv[16], gv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = tb + u < tend;
      xv[u] = in ? ld_row4(x + (size_t)(tb + u) * C + c0) : make_uint2(0u, 0u);
      gv[u] = in ? ld_row4(dy + (size_t)(tb + u) * C + c0) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = tb + u;
      if (crossed || t >= tend) continue;  // (no break: the loop must unroll)
      if (t >= eos) {
        flush(eos);
        if (t >= t1) {
          crossed = true;
          continue;
        }
        n = seq_of(cu, N, t);
        seq_bounds(cu, n, T, bos, eos);
        load_window<W>(win, x, state_src<W>(st, n, C), t, bos, C, c0);
#pragma unroll
        for (int j = 0; j < kCpt; ++j)
#pragma unroll
          for (int k = 0; k < W - 1; ++k) pend[j][k] = 0.f;
      }
      float xf[4], gf[4], first[kCpt];
      unpack4(xv[u], xf);
      unpack4(gv[u], gf);
      const bool own = t < t1;
#pragma unroll
      for (int j = 0; j < kCpt; ++j) {
        float p = bf[j];
#pragma unroll
        for (int i = 0; i < W - 1; ++i) p += wf[j][i] * win[j][i];
        p += wf[j][W - 1] * xf[j];
        const float d = gf[j] * act_grad<kSilu>(p);
        if (own) {
#pragma unroll
          for (int i = 0; i < W - 1; ++i) dwp[j][i] += d * win[j][i];
          dwp[j][W - 1] += d * xf[j];
          dbp[j] += d;
        }
#pragma unroll
        for (int k = 0; k < W - 1; ++k) pend[j][k] += wf[j][k] * d;
        first[j] = pend[j][0];  // position t - (W - 1): its last tap is in
#pragma unroll
        for (int k = 0; k < W - 2; ++k) pend[j][k] = pend[j][k + 1];
        pend[j][W - 2] = wf[j][W - 1] * d;
#pragma unroll
        for (int i = 0; i < W - 2; ++i) win[j][i] = win[j][i + 1];
        win[j][W - 2] = xf[j];
      }
      emit(t - (W - 1), first);
    }
  }
  if (!crossed && tend == eos) flush(eos);  // the sequence ends where the walk stops
  float* pt = part + (size_t)tile * (W + 1) * C + c0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    *reinterpret_cast<float4*>(pt + (size_t)i * C) = make_float4(dwp[0][i], dwp[1][i], dwp[2][i], dwp[3][i]);
  *reinterpret_cast<float4*>(pt + (size_t)W * C) = make_float4(dbp[0], dbp[1], dbp[2], dbp[3]);
}

// Zero the carried-state gradient of sequences without tokens (the backward
// kernel writes the others).
template <int W>
__global__ __launch_bounds__(kThreads) void conv_dstate_empty_kernel(
    const int32_t* __restrict__ cu, int N, int T, int C, float* __restrict__ dstate) {
  const int n = blockIdx.x;
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  int bos, eos;
  seq_bounds(cu, n, T, bos, eos);
  if (eos > bos) return;
#pragma unroll
  for (int j = 0; j < kCpt * (W - 1); ++j) dstate[((size_t)n * C + c0) * (W - 1) + j] = 0.f;
}

// Fixed-order reduction of the tiles' partial sums: rows [tile][W + 1][C].
// Pass 1 adds groups of kGroup consecutive tiles (one row of one group per
// thread, all kGroup loads in flight), pass 2 adds the groups in order.
__global__ __launch_bounds__(kThreads) void conv_reduce_pass1(const float* __restrict__ part,
                                                              int ntiles, int rows, int C,
                                                              float* __restrict__ part2) {
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  const int g = blockIdx.y, r = blockIdx.z;
  float4 v[kGroup];
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    const int t = g * kGroup + u;
    v[u] = t < ntiles ? *reinterpret_cast<const float4*>(part + ((size_t)t * rows + r) * C + c0)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 s = v[0];
#pragma unroll
  for (int u = 1; u < kGroup; ++u) {
    s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
  }
  *reinterpret_cast<float4*>(part2 + ((size_t)g * rows + r) * C + c0) = s;
}

template <int W>
__global__ __launch_bounds__(kThreads) void conv_reduce_pass2(const float* __restrict__ part2,
                                                              int ngroups, int C,
                                                              float* __restrict__ dw,
                                                              float* __restrict__ db) {
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  const int r = blockIdx.y;  // 0 .. W - 1: taps, W: bias
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g0 = 0; g0 < ngroups; g0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = g0 + u < ngroups
                 ? *reinterpret_cast<const float4*>(part2 + ((size_t)(g0 + u) * (W + 1) + r) * C + c0)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
    }
  }
  if (r < W) {
    dw[(size_t)(c0 + 0) * W + r] = s.x;
    dw[(size_t)(c0 + 1) * W + r] = s.y;
    dw[(size_t)(c0 + 2) * W + r] = s.z;
    dw[(size_t)(c0 + 3) * W + r] = s.w;
  } else if (db) {
    db[c0] = s.x;
    db[c0 + 1] = s.y;
    db[c0 + 2] = s.z;
    db[c0 + 3] = s.w;
  }
}

// ------------------------------------------------------------------ decode update
template <int W, bool kSilu>
__global__ __launch_bounds__(kThreads) void conv_update_kernel(
    int C, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ pool, int slots,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ y) {
  const int n = blockIdx.x;
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * kCpt;
  if (c0 >= C) return;
  const int sl = idx[n];
  uint16_t* yr = y + (size_t)n * C + c0;
  if (sl <= 0 || sl >= slots) {  // null block: zero output, no block touched
    *reinterpret_cast<uint2*>(yr) = make_uint2(0u, 0u);
    return;
  }
  float wf[kCpt][W], bf[kCpt];
  load_taps<W>(wf, bf, w, bias, c0);
  uint16_t* blk = pool + (size_t)sl * C * (W - 1);
  const uint2 xr = ld_row4(x + (size_t)n * C + c0);
  const uint16_t xs[4] = {(uint16_t)(xr.x & 0xffffu), (uint16_t)(xr.x >> 16),
                          (uint16_t)(xr.y & 0xffffu), (uint16_t)(xr.y >> 16)};
  float out[4];
#pragma unroll
  for (int j = 0; j < kCpt; ++j) {
    uint16_t s[W - 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) s[k] = blk[(size_t)(c0 + j) * (W - 1) + k];
    float p = bf[j];
#pragma unroll
    for (int i = 0; i < W - 1; ++i) p += wf[j][i] * bf2f(s[i]);
    p += wf[j][W - 1] * bf2f(xs[j]);
    out[j] = act<kSilu>(p);
#pragma unroll
    for (int k = 0; k < W - 2; ++k) blk[(size_t)(c0 + j) * (W - 1) + k] = s[k + 1];
    blk[(size_t)(c0 + j) * (W - 1) + W - 2] = xs[j];
  }
  *reinterpret_cast<uint2*>(yr) = pack4_bf16(out[0], out[1], out[2], out[3]);
}

// ------------------------------------------------------------------ dispatch over (W, activation)
template <template <int, bool> class F, typename... A>
hipError_t dispatch_w_act(int W, bool silu, A&&... a) {
  switch (W * 2 + (silu ? 1 : 0)) {
    case 4: return F<2, false>::run(a...);
    case 5: return F<2, true>::run(a...);
    case 6: return F<3, false>::run(a...);
    case 7: return F<3, true>::run(a...);
    case 8: return F<4, false>::run(a...);
    case 9: return F<4, true>::run(a...);
    default: return hipErrorInvalidValue;
  }
}

unsigned cblocks(int C) { return (unsigned)((C / kCpt + kThreads - 1) / kThreads); }
int ntiles_of(int T) { return (T + kTile - 1) / kTile; }
int ngroups_of(int T) { return (ntiles_of(T) + kGroup - 1) / kGroup; }

template <int W, bool S>
struct FwdLaunch {
  static hipError_t run(const int32_t* cu, int N, int T, int C, const uint16_t* x,
                        const uint16_t* w, const uint16_t* b, ConvStates st, uint16_t* y,
                        hipStream_t s) {
    if (T > 0)
      hipLaunchKernelGGL((conv_fwd_kernel<W, S>), dim3(ntiles_of(T), cblocks(C)), dim3(kThreads),
                         0, s, cu, N, T, C, x, w, b, st, y);
    if (N > 0 && st.out)
      hipLaunchKernelGGL((conv_state_out_kernel<W>), dim3(N, cblocks(C)), dim3(kThreads), 0, s,
                         cu, N, T, C, x, st);
    return hipGetLastError();
  }
};

template <int W, bool S>
struct BwdLaunch {
  static hipError_t run(const int32_t* cu, int N, int T, int C, const uint16_t* x,
                        const uint16_t* w, const uint16_t* b, ConvStates st, const uint16_t* dy,
                        uint16_t* dx, float* dw, float* db, float* dstate, float* part,
                        float* part2, hipStream_t s) {
    if (dstate && N > 0)
      hipLaunchKernelGGL((conv_dstate_empty_kernel<W>), dim3(N, cblocks(C)), dim3(kThreads), 0,
                         s, cu, N, T, C, dstate);
    if (T > 0) {
      hipLaunchKernelGGL((conv_bwd_kernel<W, S>), dim3(ntiles_of(T), cblocks(C)), dim3(kThreads),
                         0, s, cu, N, T, C, x, w, b, st, dy, dx, dstate, part);
      hipLaunchKernelGGL(conv_reduce_pass1, dim3(cblocks(C), ngroups_of(T), W + 1),
                         dim3(kThreads), 0, s, part, ntiles_of(T), W + 1, C, part2);
      hipLaunchKernelGGL((conv_reduce_pass2<W>), dim3(cblocks(C), W + 1), dim3(kThreads), 0, s,
                         part2, ngroups_of(T), C, dw, db);
    } else {
      // no tokens: zero weight and bias gradients through the same reduction
      hipLaunchKernelGGL((conv_reduce_pass2<W>), dim3(cblocks(C), W + 1), dim3(kThreads), 0, s,
                         part2, 0, C, dw, db);
    }
    return hipGetLastError();
  }
};

template <int W, bool S>
struct UpdLaunch {
  static hipError_t run(int N, int C, const uint16_t* x, const uint16_t* w, const uint16_t* b,
                        uint16_t* pool, int slots, const int32_t* idx, uint16_t* y,
                        hipStream_t s) {
    hipLaunchKernelGGL((conv_update_kernel<W, S>), dim3(N, cblocks(C)), dim3(kThreads), 0, s, C,
                       x, w, b, pool, slots, idx, y);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ host checks
bool al8(const void* p) { return ((uintptr_t)p & 7u) == 0; }
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

gdn_status check_conv(const gdn_conv_problem* p) {
  if (!p) return GDN_ERR_NULL;
  if (p->N < 0 || p->T < 0 || p->C <= 0 || p->W <= 0) return GDN_ERR_SHAPE;
  if (p->W < 2 || p->W > 4 || p->C % kCpt != 0 || (p->activation != 0 && p->activation != 1))
    return GDN_ERR_UNSUPPORTED;
  if (p->N == 0 && p->T != 0) return GDN_ERR_SHAPE;
  if (p->N > 65535 || (int64_t)p->T * p->C > ((int64_t)1 << 40)) return GDN_ERR_SHAPE;
  if (p->T > 0 && !p->cu_seqlens) return GDN_ERR_NULL;
  if (p->cu_seqlens_host) {
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0 || cu[p->N] != p->T) return GDN_ERR_SEQLENS;
    for (int n = 0; n < p->N; ++n)
      if (cu[n + 1] < cu[n]) return GDN_ERR_SEQLENS;
  }
  return GDN_OK;
}

// conv state blocks: 0 is the null block; a negative index, one >= slots or
// an active index used twice is an error
gdn_status check_conv_indices(int N, int slots, const int32_t* h) {
  if (!h) return GDN_OK;
  std::vector<char> seen((size_t)slots, 0);
  for (int n = 0; n < N; ++n) {
    const int s = h[n];
    if (s == 0) continue;
    if (s < 0 || s >= slots || seen[s]) return GDN_ERR_INDEX;
    seen[s] = 1;
  }
  return GDN_OK;
}

size_t conv_ws_bytes(const gdn_conv_problem* p) {
  const size_t rows = (size_t)(p->W + 1) * p->C * sizeof(float);
  return (size_t)(ntiles_of(p->T) + ngroups_of(p->T)) * rows + 256;
}

int conv_fwd_impl(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                  const uint16_t* bias, const ConvStates& st, uint16_t* y, void* stream) {
  if (!weight) return GDN_ERR_NULL;
  if (p->T > 0 && (!x || !y)) return GDN_ERR_NULL;
  if (!al8(x) || !al8(y)) return GDN_ERR_ALIGN;
  if (p->N == 0) return GDN_OK;
  const hipError_t e = dispatch_w_act<FwdLaunch>(p->W, p->activation == 1, p->cu_seqlens, p->N,
                                                 p->T, p->C, x, weight, bias, st, y,
                                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

GDN_API int gdn_conv_fwd(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                         const uint16_t* bias, const uint16_t* state_in, uint16_t* y,
                         uint16_t* state_out, void* stream) {
  const gdn_status s = check_conv(p);
  if (s != GDN_OK) return s;
  const ConvStates st{state_in, state_out, nullptr, nullptr, 0};
  return conv_fwd_impl(p, x, weight, bias, st, y, stream);
}

GDN_API int gdn_conv_fwd_paged(const gdn_conv_problem* p, const uint16_t* x,
                               const uint16_t* weight, const uint16_t* bias, uint16_t* state_pool,
                               int32_t slots, const int32_t* indices,
                               const int32_t* has_initial_state, const int32_t* indices_host,
                               uint16_t* y, void* stream) {
  const gdn_status s = check_conv(p);
  if (s != GDN_OK) return s;
  if (slots < 0) return GDN_ERR_SHAPE;
  if (p->N > 0 && (!state_pool || !indices)) return GDN_ERR_NULL;
  if (check_conv_indices(p->N, slots, indices_host) != GDN_OK) return GDN_ERR_INDEX;
  const ConvStates st{state_pool, state_pool, indices, has_initial_state, slots};
  return conv_fwd_impl(p, x, weight, bias, st, y, stream);
}

GDN_API size_t gdn_conv_bwd_workspace_size(const gdn_conv_problem* p) {
  return check_conv(p) == GDN_OK ? conv_ws_bytes(p) : 0;
}

GDN_API int gdn_conv_bwd(const gdn_conv_problem* p, const uint16_t* x, const uint16_t* weight,
                         const uint16_t* bias, const uint16_t* state_in, const uint16_t* dy,
                         uint16_t* dx, float* dweight, float* dbias, float* dstate_in,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const gdn_status s = check_conv(p);
  if (s != GDN_OK) return s;
  if (!weight || !dweight) return GDN_ERR_NULL;
  if (p->T > 0 && (!x || !dy || !dx)) return GDN_ERR_NULL;
  if (!al8(x) || !al8(dy) || !al8(dx) || !al16(workspace)) return GDN_ERR_ALIGN;
  if (!workspace || workspace_bytes < conv_ws_bytes(p)) return GDN_ERR_WORKSPACE;
  float* part = static_cast<float*>(workspace);
  float* part2 = part + (size_t)ntiles_of(p->T) * (p->W + 1) * p->C;
  const ConvStates st{state_in, nullptr, nullptr, nullptr, 0};
  const hipError_t e = dispatch_w_act<BwdLaunch>(
      p->W, p->activation == 1, p->cu_seqlens, p->N, p->T, p->C, x, weight, bias, st, dy, dx,
      dweight, dbias, dstate_in, part, part2, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

GDN_API int gdn_conv_update(int32_t N, int32_t C, int32_t W, int32_t activation,
                            const uint16_t* x, const uint16_t* weight, const uint16_t* bias,
                            uint16_t* state_pool, int32_t slots, const int32_t* indices,
                            const int32_t* indices_host, uint16_t* y, void* stream) {
  if (N < 0 || C <= 0 || W <= 0 || slots < 0) return GDN_ERR_SHAPE;
  if (W < 2 || W > 4 || C % kCpt != 0 || (activation != 0 && activation != 1))
    return GDN_ERR_UNSUPPORTED;
  if (N > 65535) return GDN_ERR_SHAPE;
  if (N == 0) return GDN_OK;
  if (!x || !weight || !state_pool || !indices || !y) return GDN_ERR_NULL;
  if (!al8(x) || !al8(y)) return GDN_ERR_ALIGN;
  if (check_conv_indices(N, slots, indices_host) != GDN_OK) return GDN_ERR_INDEX;
  const hipError_t e = dispatch_w_act<UpdLaunch>(W, activation == 1, N, C, x, weight, bias,
                                                 state_pool, slots, indices, y,
                                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
