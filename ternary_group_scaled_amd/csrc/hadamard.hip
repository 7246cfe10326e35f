// Block-wise signed Walsh-Hadamard rotation of activations, 128 elements per block.
//
// y = R x with R = blockdiag((1/sqrt(128)) H_128 S): signs first, then the natural-order
// Sylvester Hadamard transform, then the 1/sqrt(128) normalisation ("Ternary Bonsai 2 27B,
// 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsection "Block-wise Hadamard rotation";
// block size 128 here, one block per scale group). The sign flip is applied as the data is
// loaded, so there is no separate pass over the activations (the page's Metal kernel does the
// same), and the whole wave shares one block: lane l holds elements l and l + 64, the stride-64
// stage runs inside the lane, the six others exchange values between lanes.
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

__global__ __launch_bounds__(kThreads) void hadamard_kernel(const void* __restrict__ x, int32_t x_dtype,
                                                            int64_t blocks_total, int64_t k,
                                                            const int8_t* __restrict__ sign, void* __restrict__ y,
                                                            int32_t y_dtype) {
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (blk >= blocks_total) return;
  const int64_t kb_per_row = k / 128;
  const int64_t row = blk / kb_per_row, kb = (blk - row * kb_per_row) * 128;
  const int64_t base = row * k + kb;
  float v0 = load_as_f32(x, x_dtype, base + lane) * (float)sign[kb + lane];
  float v1 = load_as_f32(x, x_dtype, base + lane + 64) * (float)sign[kb + lane + 64];
  float a = v0 + v1, b = v0 - v1;
  v0 = a;
  v1 = b;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float p0 = __shfl_xor(v0, s), p1 = __shfl_xor(v1, s);
    const bool upper = (lane & s) != 0;
    v0 = upper ? (p0 - v0) : (v0 + p0);
    v1 = upper ? (p1 - v1) : (v1 + p1);
  }
  const float norm = 0.08838834764831845f;  // 1/sqrt(128)
  v0 *= norm;
  v1 *= norm;
  if (y_dtype == TGS_F16) {
    reinterpret_cast<_Float16*>(y)[base + lane] = (_Float16)v0;
    reinterpret_cast<_Float16*>(y)[base + lane + 64] = (_Float16)v1;
  } else {
    reinterpret_cast<float*>(y)[base + lane] = v0;
    reinterpret_cast<float*>(y)[base + lane + 64] = v1;
  }
}

}  // namespace

hipError_t hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, const int8_t* signs, void* y,
                           int32_t y_dtype, hipStream_t stream) {
  const int64_t blocks_total = m * (k / 128);
  const int64_t grid = (blocks_total + 3) / 4;
  hipLaunchKernelGGL(hadamard_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, x_dtype, blocks_total, k,
                     signs, y, y_dtype);
  return hipGetLastError();
}

}  // namespace tgs
