// Block-wise signed Walsh-Hadamard rotation of activations, 128 or 1024 elements per block.
//
// y = R x with R = blockdiag((1/sqrt(n)) H_n S): signs first, then the natural-order Sylvester
// Hadamard transform, then the 1/sqrt(n) normalisation ("Ternary Bonsai 2 27B, 5.93GB ... (feat.
// PrismML)" (discuss.pytorch.kr), subsection "Block-wise Hadamard rotation", which names
// n = 1024; n = 128 makes one block per scale group). One wave owns one block of one row: lane l
// holds the n/64 consecutive elements n/64 * l .., the butterfly stages of stride below n/64 run
// inside the lane, and the six others exchange values with lane l ^ s (DPP quad permutes, masked
// row rotations and the lane-half swaps; no LDS). The sign flip is applied as the data is loaded.
//
// The RMSNorm-fused variant (the page's WebGPU runtime has one, section "Running in the browser
// with WebGPU") rotates xhat = gamma * x / sqrt(mean_k x^2 + eps) instead: one workgroup per row
// first adds the row's squares (a fixed-order reduction, rms_norm.h), then its four waves rotate
// the row's blocks with gamma and 1 / rms applied at load.
#include "lane_ops.h"
#include "rms_norm.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load_as_f32(const void* p, int32_t dtype, int64_t i) {
  if (dtype == TGS_F16) return (float)reinterpret_cast<const _Float16*>(p)[i];
  if (dtype == TGS_BF16) {
    uint32_t bits = (uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16;
    return __builtin_bit_cast(float, bits);
  }
  return reinterpret_cast<const float*>(p)[i];
}

template <int S, int E>
__device__ __forceinline__ void cross_stage(float (&v)[E], int lane) {
  const float sgn = (lane & S) ? -1.f : 1.f;  // the upper lane of a pair keeps partner - own
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = fmaf(v[i], sgn, xor_lane<S>(v[i], lane));
}

// the butterfly over one block held as E = BLOCK / 64 consecutive elements per lane, the
// normalisation, and the store of the lane's elements at y[base ..]
template <int BLOCK>
__device__ __forceinline__ void rotate_store(float (&v)[BLOCK / 64], int lane, void* y, int32_t y_dtype,
                                             int64_t base) {
  constexpr int E = BLOCK / 64;
#pragma unroll
  for (int h = 1; h < E; h <<= 1)
#pragma unroll
    for (int i = 0; i < E; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  cross_stage<1>(v, lane);
  cross_stage<2>(v, lane);
  cross_stage<4>(v, lane);
  cross_stage<8>(v, lane);
  cross_stage<16>(v, lane);
  cross_stage<32>(v, lane);
  const float norm = BLOCK == 128 ? 0.08838834764831845f : 0.03125f;  // 1/sqrt(BLOCK)
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (y_dtype == TGS_F16)
      reinterpret_cast<_Float16*>(y)[base + i] = (_Float16)(v[i] * norm);
    else
      reinterpret_cast<float*>(y)[base + i] = v[i] * norm;
  }
}

template <int BLOCK>
__global__ __launch_bounds__(kThreads) void hadamard_kernel(const void* __restrict__ x, int32_t x_dtype,
                                                            int64_t blocks_total, int64_t k,
                                                            const int8_t* __restrict__ sign, void* __restrict__ y,
                                                            int32_t y_dtype) {
  constexpr int E = BLOCK / 64;
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (blk >= blocks_total) return;  // whole waves leave together
  const int64_t kb_per_row = k / BLOCK;
  const int64_t row = blk / kb_per_row, kb = (blk - row * kb_per_row) * BLOCK;
  const int64_t base = row * k + kb + (int64_t)E * lane;
  float v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = load_as_f32(x, x_dtype, base + i) * (float)sign[kb + E * lane + i];
  rotate_store<BLOCK>(v, lane, y, y_dtype, base);
}

// one workgroup per row: the row's 1 / rms, then its blocks, wave by wave
template <int BLOCK>
__global__ __launch_bounds__(kThreads) void rmsnorm_hadamard_kernel(const void* __restrict__ x, int32_t x_dtype,
                                                                    int64_t k, const uint16_t* __restrict__ gamma,
                                                                    float eps, const int8_t* __restrict__ sign,
                                                                    void* __restrict__ y, int32_t y_dtype) {
  constexpr int E = BLOCK / 64, kWavesPerGroup = kThreads / 64;
  __shared__ float part[kWavesPerGroup];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < k; i += kThreads) {
    const float v = load_as_f32(x, x_dtype, row * k + i);
    acc = fmaf(v, v, acc);
  }
  acc = wave_sum(acc, lane);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  const float r = rms_inverse(part, 0, kWavesPerGroup, (int)k, eps);
  for (int64_t kb = (int64_t)wave * BLOCK; kb < k; kb += (int64_t)kWavesPerGroup * BLOCK) {
    const int64_t base = row * k + kb + (int64_t)E * lane;
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int64_t c = kb + E * lane + i;
      const float g = __builtin_bit_cast(float, (uint32_t)gamma[c] << 16);
      v[i] = load_as_f32(x, x_dtype, base + i) * g * r * (float)sign[c];
    }
    rotate_store<BLOCK>(v, lane, y, y_dtype, base);
  }
}

}  // namespace

hipError_t hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block, const int8_t* signs,
                           void* y, int32_t y_dtype, hipStream_t stream) {
  const int64_t blocks_total = m * (k / block);
  const int64_t grid = (blocks_total + 3) / 4;
  if (block == 1024)
    hipLaunchKernelGGL(hadamard_kernel<1024>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, x_dtype,
                       blocks_total, k, signs, y, y_dtype);
  else
    hipLaunchKernelGGL(hadamard_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, x_dtype,
                       blocks_total, k, signs, y, y_dtype);
  return hipGetLastError();
}

hipError_t rmsnorm_hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                                   const uint16_t* gamma, float eps, const int8_t* signs, void* y, int32_t y_dtype,
                                   hipStream_t stream) {
  if (block == 1024)
    hipLaunchKernelGGL(rmsnorm_hadamard_kernel<1024>, dim3((unsigned)m), dim3(kThreads), 0, stream, x, x_dtype, k,
                       gamma, eps, signs, y, y_dtype);
  else
    hipLaunchKernelGGL(rmsnorm_hadamard_kernel<128>, dim3((unsigned)m), dim3(kThreads), 0, stream, x, x_dtype, k,
                       gamma, eps, signs, y, y_dtype);
  return hipGetLastError();
}

}  // namespace tgs
