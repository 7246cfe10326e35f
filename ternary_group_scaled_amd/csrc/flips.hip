// Code flips between two packed checkpoints: per row and in total, the number of weights whose
// ternary code differs ("Fine-tuning the ternary Bonsai-8B on Metal" (molayo1419.me): a code
// flip is a weight's code changing, e.g. 0 -> +1 or +1 -> -1, the only way training changes what
// the model computes; the closing advice records the flips per checkpoint).
//
// Both matrices are streamed once. A workgroup of 256 threads owns 16 rows, 16 threads per row;
// the 16 threads of a row read 256 contiguous bytes of each matrix per load, and every thread
// keeps four 16-byte pairs in flight. The count never leaves the integers, so results are exact
// and identical run to run, including the 64-bit atomic total.
//   - Slot-2: a code word v = a ^ b is nonzero in a 2-bit field exactly where the codes differ,
//     so the flips of 16 codes are popcount((v | v >> 1) & 0x55555555).
//   - Binary: one bit per weight, so the flips of 32 codes are popcount(a ^ b).
//   - Base-3: each byte is first rewritten as its five trits in 2-bit fields (peeling base-3
//     digits with v = v * 171 >> 9 on packed 16-bit halves, as the GEMV kernels do), then the
//     same XOR and popcount.
// Pad trits and pad bytes are compared as stored; in valid matrices they are equal on both sides.
#include "lane_ops.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 16;
constexpr int kThreadsPerRow = kThreads / kRowsPerBlock;
constexpr int kUnroll = 4;  // 16-byte pairs in flight per thread

__device__ __forceinline__ uint32_t flips_slot2(uint32_t a, uint32_t b) {
  const uint32_t v = a ^ b;
  return __builtin_popcount((v | (v >> 1)) & 0x55555555u);
}

// two bytes (the low byte of each 16-bit half) -> their five trits as 2-bit fields, bits 0..9
__device__ __forceinline__ u16x2 trit_fields(u16x2 v) {
  u16x2 out = {0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x2 q = (v * (u16x2)171) >> (u16x2)9;  // v / 3 for v < 256
    out |= (v - q * (u16x2)3) << (u16x2)(2 * j);
    v = q;
  }
  return out | (v << (u16x2)8);
}

__device__ __forceinline__ uint32_t flips_base3(uint32_t a, uint32_t b) {
  const u16x2 ae = trit_fields(__builtin_bit_cast(u16x2, a & 0x00FF00FFu));
  const u16x2 ao = trit_fields(__builtin_bit_cast(u16x2, (a >> 8) & 0x00FF00FFu));
  const u16x2 be = trit_fields(__builtin_bit_cast(u16x2, b & 0x00FF00FFu));
  const u16x2 bo = trit_fields(__builtin_bit_cast(u16x2, (b >> 8) & 0x00FF00FFu));
  return flips_slot2(__builtin_bit_cast(uint32_t, ae), __builtin_bit_cast(uint32_t, be)) +
         flips_slot2(__builtin_bit_cast(uint32_t, ao), __builtin_bit_cast(uint32_t, bo));
}

template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void code_flip_kernel(const FlipArgs args) {
  __shared__ uint32_t row_sums[kRowsPerBlock];

  int jb = 0;
  while (jb + 1 < args.count && (int)blockIdx.x >= args.job[jb + 1].block0) ++jb;
  const FlipJob& job = args.job[jb];
  const int n = job.n;
  const int chunks = job.row_bytes / 16;

  const int tid = threadIdx.x;
  const int local = tid / kThreadsPerRow, j = tid % kThreadsPerRow;
  const int row = ((int)blockIdx.x - job.block0) * kRowsPerBlock + local;

  // rows past n read as zero on both sides (no flips); their counts are not stored
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.a, 0, (int)((int64_t)n * job.stride_a), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.b, 0, (int)((int64_t)n * job.stride_b), kRsrcWord3);
  const uint32_t a_row = (uint32_t)row * (uint32_t)job.stride_a, b_row = (uint32_t)row * (uint32_t)job.stride_b;
  const bool row_ok = row < n;

  uint32_t count = 0;
  for (int c0 = j; c0 < chunks; c0 += kUnroll * kThreadsPerRow) {
    uint4 va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kThreadsPerRow;
      const bool ok = row_ok && c < chunks;  // pairs past the row are parked: zero on both sides
      va[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            a_rsrc, ok ? (int)(a_row + 16u * (uint32_t)c) : kOobOffset, 0, kStreamAux));
      vb[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            b_rsrc, ok ? (int)(b_row + 16u * (uint32_t)c) : kOobOffset, 0, kStreamAux));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t wa[4] = {va[u].x, va[u].y, va[u].z, va[u].w};
      const uint32_t wb[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (LAYOUT == TGS_LAYOUT_SLOT2)
          count += flips_slot2(wa[i], wb[i]);
        else if constexpr (LAYOUT == TGS_LAYOUT_BINARY)
          count += __builtin_popcount(wa[i] ^ wb[i]);
        else
          count += flips_base3(wa[i], wb[i]);
      }
    }
  }

  // the 16 threads of a row are one 16-lane DPP row: add across it
  float f = __builtin_bit_cast(float, count);
  uint32_t s = count;
  s += __builtin_bit_cast(uint32_t, dpp<kDppRor8>(f));
  f = __builtin_bit_cast(float, s);
  s += __builtin_bit_cast(uint32_t, dpp<kDppRor4>(f));
  f = __builtin_bit_cast(float, s);
  s += __builtin_bit_cast(uint32_t, dpp<kDppRor2>(f));
  f = __builtin_bit_cast(float, s);
  s += __builtin_bit_cast(uint32_t, dpp<kDppRor1>(f));
  if (j == 0) {
    row_sums[local] = row_ok ? s : 0u;
    if (row_ok && job.rows) job.rows[row] = s;
  }
  if (job.total) {
    __syncthreads();
    if (tid == 0) {
      uint64_t t = 0;
#pragma unroll
      for (int r = 0; r < kRowsPerBlock; ++r) t += row_sums[r];
      if (t) atomicAdd(reinterpret_cast<unsigned long long*>(job.total), (unsigned long long)t);
    }
  }
}

// totals start at zero (a kernel, not a memset, so that the call can be captured in a graph)
__global__ void zero_totals_kernel(const FlipArgs args) {
  const int i = threadIdx.x;
  if (i < args.count && args.job[i].total) *args.job[i].total = 0;
}

}  // namespace

int code_flip_rows_per_block() { return kRowsPerBlock; }

hipError_t code_flip_launch(FlipArgs& args, int32_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL(zero_totals_kernel, dim3(1), dim3(64), 0, stream, args);
  if (args.layout == TGS_LAYOUT_SLOT2)
    hipLaunchKernelGGL(code_flip_kernel<TGS_LAYOUT_SLOT2>, dim3(blocks), dim3(kThreads), 0, stream, args);
  else if (args.layout == TGS_LAYOUT_BINARY)
    hipLaunchKernelGGL(code_flip_kernel<TGS_LAYOUT_BINARY>, dim3(blocks), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(code_flip_kernel<TGS_LAYOUT_BASE3>, dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace tgs
