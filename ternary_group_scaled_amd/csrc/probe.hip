// Streaming-read probe: the plainest kernel that reads a large buffer once from HBM, used to
// measure the read bandwidth a kernel can actually reach on this device (the ceiling the GEMV's
// achieved bandwidth is compared with, next to the nominal peak).
//
// Every thread walks the buffer with a grid-sized stride in 16-byte non-temporal loads, four
// independent loads per iteration, and folds what it reads into one word with XOR. Each thread
// stores its word (grid * 4 bytes in all, negligible next to the buffer), so no load can be removed.
#include "tgs_internal.h"

namespace tgs {
namespace {

constexpr int kProbeThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(const u32x4* p) {
  const u32x4 v = __builtin_nontemporal_load(p);
  return v.x ^ v.y ^ v.z ^ v.w;
}

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const uint64_t tid = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  uint64_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    acc ^= fold(p + i) ^ fold(p + i + stride) ^ fold(p + i + 2 * stride) ^ fold(p + i + 3 * stride);
  }
  for (; i < n16; i += stride) {
    acc ^= fold(p + i);
  }
  sink[tid] = acc;
}

}  // namespace

int stream_read_grid() { return 256 * 8; }

hipError_t stream_read_launch(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(stream_read_grid()), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace tgs
