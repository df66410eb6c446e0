// Recurrent decode step of the gated delta rule over a paged state pool.
//
// Arithmetic (RL-Kernel PR #469, "[WS1][CUDA][Qwen3-Next] C6: GDN decode-step
// goldens", "What" section and the note on where the kernel and the HF model
// disagree): fp32 gating beta = sigmoid(b), g = -exp(A_log) softplus(a +
// dt_bias) with softplus(x) = x above 20; q and k divided by
// sqrt(sum x^2 + 1e-6), q then scaled; value head hv reads key head
// hv / (HV/H); then S <- e^g S, delta = beta (v - S k), S <- S + delta k^T,
// o = S q. State contract (same page, state-contract bullet): pool
// [slots, HV, V, K] fp32 addressed by ssm_state_indices, every index <= 0
// skipped.
//
// The step is bound by HBM: each active (row, value head) streams its 64 KiB
// fp32 state block in and out once. One 256-thread workgroup owns one
// (row, value head); thread t holds columns 4*(t%32) .. +3 of rows
// t/32 + 8 i (i = 0..15), so each half-wave reads one 512-byte state row per
// load and all 16 loads of a thread are in flight together.
#include "gdn_common.h"

namespace gdn {

__global__ __launch_bounds__(256) void decode_step_kernel(
    int H, int HV, float scale,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ a,
    const uint16_t* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ pool, int slots,
    const int32_t* __restrict__ idx, uint16_t* __restrict__ o) {
  const int row = blockIdx.x / HV;
  const int hv = blockIdx.x - row * HV;
  const int tid = threadIdx.x;
  const int slot = idx[row];
  uint16_t* orow = o + ((size_t)row * HV + hv) * kHead;

  if (slot <= 0 || slot >= slots) {  // null block, negative, or out of range: skip
    if (tid < kHead / 2) reinterpret_cast<uint32_t*>(orow)[tid] = 0u;
    return;
  }

  __shared__ float kn[kHead], qn[kHead], vs[kHead];
  const int h = hv / (HV / H);
  float* S = pool + ((size_t)slot * HV + hv) * (size_t)(kHead * kHead);
  const int c4 = tid & 31;
  const int r0 = tid >> 5;

  // issue the state loads first: they are the whole cost of the step; the
  // state is streamed exactly once in and once out, so the accesses are
  // non-temporal
  f32x4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (size_t)(r0 + 8 * i) * kHead) + c4);

  if (tid < 64) {
    // q and k rows of the key head: lane holds elements 2*lane, 2*lane + 1
    const uint32_t qp = reinterpret_cast<const uint32_t*>(q + ((size_t)row * H + h) * kHead)[tid];
    const uint32_t kp = reinterpret_cast<const uint32_t*>(k + ((size_t)row * H + h) * kHead)[tid];
    const float q0 = bf2f(qp & 0xffffu), q1 = bf2f(qp >> 16);
    const float k0 = bf2f(kp & 0xffffu), k1 = bf2f(kp >> 16);
    const float nq = sqrtf(wave_sum(q0 * q0 + q1 * q1) + kNormEps);
    const float nk = sqrtf(wave_sum(k0 * k0 + k1 * k1) + kNormEps);
    qn[2 * tid] = (q0 / nq) * scale;
    qn[2 * tid + 1] = (q1 / nq) * scale;
    kn[2 * tid] = k0 / nk;
    kn[2 * tid + 1] = k1 / nk;
  } else if (tid < 64 + kHead) {
    vs[tid - 64] = bf2f(v[((size_t)row * HV + hv) * kHead + (tid - 64)]);
  }
  const float x = bf2f(a[(size_t)row * HV + hv]) + (dt_bias ? dt_bias[hv] : 0.f);
  const float sp = x > 20.f ? x : log1pf(expf(x));
  const float decay = expf(-expf(A_log[hv]) * sp);
  const float beta = 1.f / (1.f + expf(-bf2f(b[(size_t)row * HV + hv])));
  __syncthreads();

  const float4 kk = reinterpret_cast<const float4*>(kn)[c4];
  const float4 qq = reinterpret_cast<const float4*>(qn)[c4];
  float outv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f32x4 x4 = s[i];
    x4[0] *= decay; x4[1] *= decay; x4[2] *= decay; x4[3] *= decay;
    float p = x4[0] * kk.x + x4[1] * kk.y + x4[2] * kk.z + x4[3] * kk.w;
    p = group_sum<32>(p);
    const float delta = beta * (vs[r0 + 8 * i] - p);
    x4[0] += delta * kk.x; x4[1] += delta * kk.y; x4[2] += delta * kk.z; x4[3] += delta * kk.w;
    s[i] = x4;
    outv[i] = x4[0] * qq.x + x4[1] * qq.y + x4[2] * qq.z + x4[3] * qq.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) outv[i] = group_sum<32>(outv[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (size_t)(r0 + 8 * i) * kHead) + c4);
  if (c4 == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) orow[r0 + 8 * i] = f2bf(outv[i]);
  }
}

hipError_t launch_decode_step(int N, int H, int HV, float scale, const uint16_t* q,
                              const uint16_t* k, const uint16_t* v, const uint16_t* a,
                              const uint16_t* b, const float* A_log, const float* dt_bias,
                              float* pool, int slots, const int32_t* idx, uint16_t* o,
                              hipStream_t stream) {
  hipLaunchKernelGGL(decode_step_kernel, dim3((unsigned)N * (unsigned)HV), dim3(256), 0, stream,
                     H, HV, scale, q, k, v, a, b, A_log, dt_bias, pool, slots, idx, o);
  return hipGetLastError();
}

}  // namespace gdn
