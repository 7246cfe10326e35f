// Block-wise signed Walsh-Hadamard rotation of activations, 128 or 1024 elements per block.
//
// y = R x with R = blockdiag((1/sqrt(n)) H_n S): signs first, then the natural-order Sylvester
// Hadamard transform, then the 1/sqrt(n) normalisation ("Ternary Bonsai 2 27B, 5.93GB ... (feat.
// PrismML)" (discuss.pytorch.kr), subsection "Block-wise Hadamard rotation", which names
// n = 1024; n = 128 makes one block per scale group). The activations are streamed once, in
// 16-byte vector loads and stores: a wave works on a tile of 512 consecutive elements (four
// 128-blocks, 16 lanes each) or of 1024 (one block), lane l holding the eight consecutive
// elements 8l .. 8l + 7 of each 512-element half. The butterfly stages of stride 1, 2 and 4 run
// inside the lane, those of stride 8 .. 256 exchange values with lane l ^ (stride / 8) (DPP quad
// permutes, masked row rotations and the lane-half swaps; no LDS), and stride 512 pairs the two
// halves a lane holds. The stages commute, so this order gives the same transform. The sign
// flip is applied as the data is loaded; the output type is rounded once from fp32.
//
// The RMSNorm-fused variant (the page's WebGPU runtime has one, section "Running in the browser
// with WebGPU") rotates xhat = gamma * x / sqrt(mean_k x^2 + eps) instead: one workgroup per row
// first adds the row's squares (a fixed-order reduction, rms_norm.h), then its four waves rotate
// the row's tiles with gamma and 1 / rms applied at load.
#include <algorithm>

#include "lane_ops.h"
#include "rms_norm.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

constexpr int kThreads = 256, kWaves = kThreads / 64;

// elements a lane holds: 8 for 128-blocks (16 lanes per block), 16 for 1024-blocks
template <int BLOCK>
constexpr int kElems = BLOCK == 1024 ? 16 : 8;

// fp32 -> bf16 bits, round to nearest with ties to even (NaN stays a quiet NaN of the same sign)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// the eight elements x[e .. e + 7] (e a multiple of 8, x 16-byte aligned) as fp32
template <int XD>
__device__ __forceinline__ void load8(const void* x, int64_t e, float* v) {
  if constexpr (XD == TGS_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + e);
    const float4 a = p[0], b = p[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = XD == TGS_F16 ? half_lo(w[i]) : bf16_lo(w[i]);
      v[2 * i + 1] = XD == TGS_F16 ? half_hi(w[i]) : bf16_hi(w[i]);
    }
  }
}

// v[0 .. 7] * norm stored at y[e .. e + 7] in the output type
template <int YD>
__device__ __forceinline__ void store8(void* y, int64_t e, const float* v, float norm) {
  if constexpr (YD == TGS_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + e);
    p[0] = make_float4(v[0] * norm, v[1] * norm, v[2] * norm, v[3] * norm);
    p[1] = make_float4(v[4] * norm, v[5] * norm, v[6] * norm, v[7] * norm);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = v[2 * i] * norm, b = v[2 * i + 1] * norm;
      if constexpr (YD == TGS_F16)
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
      else
        w[i] = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + e) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// v[0 .. 7] *= signs[c .. c + 7] (c a multiple of 8, signs 16-byte aligned)
__device__ __forceinline__ void apply_signs8(const int8_t* sign, int64_t c, float* v) {
  const uint2 sw = *reinterpret_cast<const uint2*>(sign + c);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] *= (float)(int8_t)((i < 4 ? sw.x : sw.y) >> (8 * (i & 3)));
}

// v[0 .. 7] *= gamma[c .. c + 7] * r (bf16 gamma, 16-byte aligned)
__device__ __forceinline__ void apply_gamma8(const uint16_t* gamma, int64_t c, float r, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(gamma + c);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] *= bf16_lo(w[i]) * r;
    v[2 * i + 1] *= bf16_hi(w[i]) * r;
  }
}

template <int S, int E>
__device__ __forceinline__ void cross_stage(float (&v)[E], int lane) {
  const float sgn = (lane & S) ? -1.f : 1.f;  // the upper lane of a pair keeps partner - own
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = fmaf(v[i], sgn, xor_lane<S>(v[i], lane));
}

// the unnormalised transform of the wave's tile: E = 8 elements per 512-element half a lane holds
template <int BLOCK>
__device__ __forceinline__ void transform(float (&v)[kElems<BLOCK>], int lane) {
  constexpr int E = kElems<BLOCK>;
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
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
  if constexpr (BLOCK == 1024) {
    cross_stage<16>(v, lane);
    cross_stage<32>(v, lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // stride 512: the lane's two halves
      const float a = v[i], b = v[i + 8];
      v[i] = a + b;
      v[i + 8] = a - b;
    }
  }
}

// Tiles of 512 elements (BLOCK 128) or 1024 (BLOCK 1024) of the flattened [m][k], grid-stride
// over waves; every lane of a wave runs the same iterations, and a 128-block lies in one
// 16-lane group, so lanes past the end only exchange values with one another.
template <int BLOCK, int XD, int YD>
__global__ __launch_bounds__(kThreads) void hadamard_kernel(const void* __restrict__ x, int64_t total, int64_t k,
                                                            const int8_t* __restrict__ sign, void* __restrict__ y) {
  constexpr int E = kElems<BLOCK>, H = E / 8, TILE = 512 * H;
  constexpr float kNorm = BLOCK == 128 ? 0.08838834764831845f : 0.03125f;  // 1 / sqrt(BLOCK)
  const int lane = threadIdx.x & 63;
  const int64_t wave0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kWaves * TILE;
  for (int64_t t0 = wave0 * TILE; t0 < total; t0 += stride) {
    float v[E];
    const bool valid = t0 + 8 * lane < total;  // total is a multiple of BLOCK
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t e = t0 + 512 * h + 8 * lane;
      if (valid) {
        load8<XD>(x, e, v + 8 * h);
        apply_signs8(sign, e % k, v + 8 * h);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[8 * h + i] = 0.f;
      }
    }
    transform<BLOCK>(v, lane);
    if (valid)
#pragma unroll
      for (int h = 0; h < H; ++h) store8<YD>(y, t0 + 512 * h + 8 * lane, v + 8 * h, kNorm);
  }
}

// one workgroup per row: the row's 1 / rms, then its tiles, wave by wave
template <int BLOCK, int XD, int YD>
__global__ __launch_bounds__(kThreads) void rmsnorm_hadamard_kernel(const void* __restrict__ x, int64_t k,
                                                                    const uint16_t* __restrict__ gamma, float eps,
                                                                    const int8_t* __restrict__ sign,
                                                                    void* __restrict__ y) {
  constexpr int E = kElems<BLOCK>, H = E / 8, TILE = 512 * H;
  constexpr float kNorm = BLOCK == 128 ? 0.08838834764831845f : 0.03125f;
  __shared__ float part[kWaves];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * k;
  float acc = 0.f;
  for (int64_t c = 8 * (int64_t)threadIdx.x; c < k; c += 8 * kThreads) {
    float f[8];
    load8<XD>(x, row0 + c, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(f[i], f[i], acc);
  }
  acc = wave_sum(acc, lane);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  const float r = rms_inverse(part, 0, kWaves, (int)k, eps);
  for (int64_t t0 = (int64_t)wave * TILE; t0 < k; t0 += (int64_t)kWaves * TILE) {
    float v[E];
    const bool valid = t0 + 8 * lane < k;  // k is a multiple of BLOCK
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t c = t0 + 512 * h + 8 * lane;
      if (valid) {
        load8<XD>(x, row0 + c, v + 8 * h);
        apply_gamma8(gamma, c, r, v + 8 * h);
        apply_signs8(sign, c, v + 8 * h);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[8 * h + i] = 0.f;
      }
    }
    transform<BLOCK>(v, lane);
    if (valid)
#pragma unroll
      for (int h = 0; h < H; ++h) store8<YD>(y, row0 + t0 + 512 * h + 8 * lane, v + 8 * h, kNorm);
  }
}

template <int BLOCK, int XD>
hipError_t launch_plain(const void* x, int64_t total, int64_t k, const int8_t* signs, void* y, int32_t y_dtype,
                        dim3 grid, hipStream_t stream) {
  if (y_dtype == TGS_F16)
    hipLaunchKernelGGL((hadamard_kernel<BLOCK, XD, TGS_F16>), grid, dim3(kThreads), 0, stream, x, total, k, signs, y);
  else if (y_dtype == TGS_BF16)
    hipLaunchKernelGGL((hadamard_kernel<BLOCK, XD, TGS_BF16>), grid, dim3(kThreads), 0, stream, x, total, k, signs, y);
  else
    hipLaunchKernelGGL((hadamard_kernel<BLOCK, XD, TGS_F32>), grid, dim3(kThreads), 0, stream, x, total, k, signs, y);
  return hipGetLastError();
}

template <int BLOCK>
hipError_t launch_plain_x(const void* x, int32_t x_dtype, int64_t total, int64_t k, const int8_t* signs, void* y,
                          int32_t y_dtype, dim3 grid, hipStream_t stream) {
  if (x_dtype == TGS_F16) return launch_plain<BLOCK, TGS_F16>(x, total, k, signs, y, y_dtype, grid, stream);
  if (x_dtype == TGS_BF16) return launch_plain<BLOCK, TGS_BF16>(x, total, k, signs, y, y_dtype, grid, stream);
  return launch_plain<BLOCK, TGS_F32>(x, total, k, signs, y, y_dtype, grid, stream);
}

template <int BLOCK, int XD>
hipError_t launch_norm(const void* x, int64_t m, int64_t k, const uint16_t* gamma, float eps, const int8_t* signs,
                       void* y, int32_t y_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)m), threads(kThreads);
  if (y_dtype == TGS_F16)
    hipLaunchKernelGGL((rmsnorm_hadamard_kernel<BLOCK, XD, TGS_F16>), grid, threads, 0, stream, x, k, gamma, eps, signs,
                       y);
  else if (y_dtype == TGS_BF16)
    hipLaunchKernelGGL((rmsnorm_hadamard_kernel<BLOCK, XD, TGS_BF16>), grid, threads, 0, stream, x, k, gamma, eps,
                       signs, y);
  else
    hipLaunchKernelGGL((rmsnorm_hadamard_kernel<BLOCK, XD, TGS_F32>), grid, threads, 0, stream, x, k, gamma, eps, signs,
                       y);
  return hipGetLastError();
}

template <int BLOCK>
hipError_t launch_norm_x(const void* x, int32_t x_dtype, int64_t m, int64_t k, const uint16_t* gamma, float eps,
                         const int8_t* signs, void* y, int32_t y_dtype, hipStream_t stream) {
  if (x_dtype == TGS_F16) return launch_norm<BLOCK, TGS_F16>(x, m, k, gamma, eps, signs, y, y_dtype, stream);
  if (x_dtype == TGS_BF16) return launch_norm<BLOCK, TGS_BF16>(x, m, k, gamma, eps, signs, y, y_dtype, stream);
  return launch_norm<BLOCK, TGS_F32>(x, m, k, gamma, eps, signs, y, y_dtype, stream);
}

}  // namespace

hipError_t hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block, const int8_t* signs,
                           void* y, int32_t y_dtype, hipStream_t stream) {
  const int64_t total = m * k, tile = block == 1024 ? 1024 : 512;
  const int64_t waves = (total + tile - 1) / tile;
  const int64_t groups = std::min<int64_t>((waves + kWaves - 1) / kWaves, int64_t(1) << 20);
  const dim3 grid((unsigned)groups);
  if (block == 1024) return launch_plain_x<1024>(x, x_dtype, total, k, signs, y, y_dtype, grid, stream);
  return launch_plain_x<128>(x, x_dtype, total, k, signs, y, y_dtype, grid, stream);
}

hipError_t rmsnorm_hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                                   const uint16_t* gamma, float eps, const int8_t* signs, void* y, int32_t y_dtype,
                                   hipStream_t stream) {
  if (block == 1024) return launch_norm_x<1024>(x, x_dtype, m, k, gamma, eps, signs, y, y_dtype, stream);
  return launch_norm_x<128>(x, x_dtype, m, k, gamma, eps, signs, y, y_dtype, stream);
}

}  // namespace tgs
