// RMSNorm prologue shared by the GEMV and rotation kernels: xhat = gamma * x / sqrt(mean_k x^2 + eps)
// per activation row, gamma in bf16. The normalisation is the one the BlockHadamard operation of
// "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr) fuses in one of its
// variants (section "Running in the browser with WebGPU"); the norm weights stay in bf16 (section
// "The 0.0976% kept at high precision").
//
// A workgroup that needs the norm of a row reads the whole row once more: each thread adds the
// squares of its strided 16-byte units in fp32, the wave adds its lanes with a butterfly (every
// lane ends with the same sum), and the waves' sums go through LDS and are added in wave order by
// every thread that needs the result. The order is fixed, so the result is identical run to run
// and in every workgroup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lane_ops.h"

namespace tgs {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float half_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

typedef _Float16 norm_half2 __attribute__((ext_vector_type(2)));

// acc + the squares of the two fp16 values of a word (one dot2; fp32 accumulation)
__device__ __forceinline__ float add_squares(uint32_t w, float acc) {
  const norm_half2 h = __builtin_bit_cast(norm_half2, w);
  return __builtin_amdgcn_fdot2(h, h, acc, false);
}

// two fp16 activations (one word) times two bf16 norm weights (one word) times r -> two fp16
// (gamma * r first, so the fp16 activation enters a mixed-precision multiply directly)
__device__ __forceinline__ uint32_t norm_word(uint32_t xw, uint32_t gw, float r) {
  const _Float16 lo = (_Float16)(half_lo(xw) * (bf16_lo(gw) * r));
  const _Float16 hi = (_Float16)(half_hi(xw) * (bf16_hi(gw) * r));
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// sum of v over the 64 lanes; every lane returns the same value
__device__ __forceinline__ float wave_sum(float v, int lane) {
  v += xor_lane<1>(v, lane);
  v += xor_lane<2>(v, lane);
  v += xor_lane<4>(v, lane);
  v += xor_lane<8>(v, lane);
  v += xor_lane<16>(v, lane);
  v += xor_lane<32>(v, lane);
  return v;
}

// Per-wave sums of squares of the fp16 rows m0 .. m0 + MT - 1 of x [m][k], into
// part[t * waves + wave]; rows at or past m count as zero. Every thread of the workgroup
// (`threads` of them, a multiple of 64) must call it; k is a multiple of 8 and x 16-byte aligned.
template <int MT>
__device__ __forceinline__ void rms_partials(const uint16_t* x, int k, int m, int m0, float* part, int threads) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, waves = threads >> 6;
  const int units = k >> 3;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float acc = 0.f;
    if (m0 + t < m) {
      const uint4* row = reinterpret_cast<const uint4*>(x + (int64_t)(m0 + t) * k);
      for (int u = tid; u < units; u += threads) {
        const uint4 q = row[u];
        acc = add_squares(q.x, acc);
        acc = add_squares(q.y, acc);
        acc = add_squares(q.z, acc);
        acc = add_squares(q.w, acc);
      }
    }
    acc = wave_sum(acc, lane);
    if (lane == 0) part[t * waves + wave] = acc;
  }
}

// 1 / sqrt(sum / k + eps) with the hardware reciprocal and reciprocal square root (each within
// about one ulp in fp32); sub-normal arguments, which those may flush, take the exact route.
// The value is the same for every lane that calls it with the same sum.
__device__ __forceinline__ float rms_scale(float sum, int k, float eps) {
  const float v = sum * __builtin_amdgcn_rcpf((float)k) + eps;
  if (v < 1.17549435e-38f) return 1.0f / sqrtf(v);
  return __builtin_amdgcn_rsqf(v);
}

// 1 / sqrt(sum_k x^2 / k + eps) of row t from the partial sums (after a barrier)
__device__ __forceinline__ float rms_inverse(const float* part, int t, int waves, int k, float eps) {
  float s = 0.f;
  for (int w = 0; w < waves; ++w) s += part[t * waves + w];
  return rms_scale(s, k, eps);
}

}  // namespace tgs
