// Single-token slot-2 GEMV on the matrix cores: m = 1, plain basis, K a multiple of 512, K <= 16384.
//
// y[j] = sum_k s[j][k/128] * t[j][k] * x[k], with the weights w = s_g * t of "Ternary Bonsai 2 27B,
// 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsection "Group-scaled ternary format": one
// fp16 scale per 128 consecutive weights of a row. The codes are read once, in packed form. The
// window layout, the signed decode and the activation pairs are described in s2_mfma.h.
//
// Work split. A workgroup owns 16 rows and has one wave per SW windows of K. Each thread issues the
// loads of its staging activations first, then every code and scale load of its wave, so the
// staging waits only for the activations (vector-memory waits retire in issue order) and for the
// small launches of a decode step every load is in flight at once. A wave multiplies its windows
// one after the other, in the order their loads were issued, so each window's MFMAs start as soon
// as its own codes have arrived. The waves' row sums meet in LDS and are added
// in wave order (deterministic, no atomics). RMSNorm (NORM): the staging threads first add the
// squares of their activations (fixed order: threads, waves in LDS), then scale by gamma / rms
// before the one rounding to fp16.
#include "lane_ops.h"
#include "rms_norm.h"
#include "s2_mfma.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

using namespace s2;

constexpr int kSW = 2;  // windows per wave

template <int SW, bool NORM>
__global__ __launch_bounds__(1024) void gemv_s2_mfma_kernel(const GemvArgs args) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ float norm_part[NORM ? 16 : 1];

  const GemvJob job = gemv_job_of_block(args);
  const int n = job.n, k = job.k;
  const int groups = k >> 7, windows = k / kWinK;
  const int waves = (int)(blockDim.x >> 6);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, q = lane >> 4;
  const int row0 = ((int)blockIdx.x - job.block0) * 16;
  const int w0 = wave * SW;

  uint32_t* pairs = reinterpret_cast<uint32_t*>(lds);             // [groups][kGroupPitch]
  const int zero_off = groups * kGroupPitch * 4;                   // kZeroBytes of zeros
  float* red = reinterpret_cast<float*>(lds + zero_off + kZeroBytes);  // [waves][16]

  // 1. the activations (and norm weights) of the thread's staging units: issued first, since
  // vector-memory waits retire in issue order and the staging below waits only for these
  const int units = k >> 4, threads = waves * 64;
  // units per thread: k / 16 = 32 windows and threads >= 64 windows / SW, so at most SW / 2
  constexpr int kMaxUnits = SW / 2 > 1 ? SW / 2 : 1;
  uint32_t xw[kMaxUnits][8];
  uint32_t gw[NORM ? kMaxUnits : 1][8];
  {
    const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)job.x, 0, k * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kMaxUnits; ++i) {
      const int u = (int)threadIdx.x + i * threads;
      const int xo = u < units ? u * 32 : kOobOffset;
      const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo, 0, 0));
      const uint4 b = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, u < units ? xo + 16 : kOobOffset, 0, 0));
      xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
      xw[i][4] = b.x; xw[i][5] = b.y; xw[i][6] = b.z; xw[i][7] = b.w;
      if constexpr (NORM) {
        const __amdgpu_buffer_rsrc_t g_rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)job.gamma, 0, k * 2, kRsrcWord3);
        const uint4 c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, xo, 0, 0));
        const uint4 d = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, u < units ? xo + 16 : kOobOffset, 0, 0));
        gw[i][0] = c.x; gw[i][1] = c.y; gw[i][2] = c.z; gw[i][3] = c.w;
        gw[i][4] = d.x; gw[i][5] = d.y; gw[i][6] = d.z; gw[i][7] = d.w;
      }
    }
  }

  // 2. every code and scale load of this wave. Rows past n read zero codes (t = -1) that meet
  // real activations, but those rows are never stored; a window past K is parked out of range.
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.codes, 0, (int)((int64_t)n * job.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);
  const uint32_t row = (uint32_t)(row0 + col);
  const uint32_t code_row = __umul24(row, (uint32_t)job.stride);
  const uint32_t scale_row = __umul24(row, (uint32_t)groups) * 2u;
  uint4 cw[SW][2];
  uint2 sc[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const int w = w0 + i;
    const bool live = w < windows;
    const int off = live ? (int)(code_row + (uint32_t)(w * 128 + q * 32)) : kOobOffset;
    cw[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, off, 0, kStreamAux));
    cw[i][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             code_rsrc, live ? off + 16 : kOobOffset, 0, kStreamAux));
    // lanes of the first quarter hold the four groups' partials: they take the four scales
    const int soff = (live && q == 0) ? (int)(scale_row + (uint32_t)(w * 8)) : kOobOffset;
    sc[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(scale_rsrc, soff, 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is out before anything waits

  // 3. stage the activation pairs (each thread 16 consecutive elements per unit)
  if constexpr (NORM) {
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxUnits; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sq = add_squares(xw[i][j], sq);  // zero past the end
    sq = wave_sum(sq, lane);
    if (lane == 0) norm_part[wave] = sq;
    __syncthreads();
    float total = 0.f;
    for (int w = 0; w < waves; ++w) total += norm_part[w];
    const float r = rms_scale(total, k, args.eps);
#pragma unroll
    for (int i = 0; i < kMaxUnits; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) xw[i][j] = norm_word(xw[i][j], gw[i][j], r);
  }
#pragma unroll
  for (int i = 0; i < kMaxUnits; ++i) {
    const int u = (int)threadIdx.x + i * threads;
    if (u < units) store_unit_pairs(pairs, u, xw[i]);
  }
  if (threadIdx.x < 16) reinterpret_cast<uint4*>(lds + zero_off)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // 4. the wave's windows, one MFMA chain after the other (a window's chain waits only for its own
  // codes: measured +2% in layer order and +4% as a set against interleaving the chains step by
  // step); a window past K reads the zero region and its scales are zero
  const ExpBits e = exp_bits();
  const char* a_base[SW];
  f32x4 d[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const int w = w0 + i;
    a_base[i] = (col == q && w < windows) ? lds + (4 * w + q) * kGroupPitch * 4 : lds + zero_off;
    d[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < SW; ++i) mfma_windows<1>(a_base + i, cw + i, d + i, e);
  // D[g][col] (group g of the window) is register g of lane col
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < SW; ++i) acc = scale_window(acc, sc[i], d[i]);

  // 5. add the waves' sums in wave order
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (threadIdx.x < 16) {
    float sum = 0.f;
    for (int w = 0; w < waves; ++w) sum += red[w * 16 + threadIdx.x];
    const int r = row0 + (int)threadIdx.x;
    if (r < n) job.y[r] = sum;
  }
}

}  // namespace

int gemv_s2_mfma_waves(int64_t k) { return (int)((k / kWinK + kSW - 1) / kSW); }

bool gemv_s2_mfma_fits(int64_t k) { return k % kWinK == 0 && k <= kMaxK; }

hipError_t gemv_s2_mfma_launch(GemvArgs& args, int32_t blocks, int64_t k, bool norm, hipStream_t stream) {
  const int waves = gemv_s2_mfma_waves(k);
  const size_t lds = (size_t)pair_bytes((int)k) + kZeroBytes + (size_t)waves * 16 * 4;
  if (norm)
    hipLaunchKernelGGL((gemv_s2_mfma_kernel<kSW, true>), dim3(blocks), dim3(64 * waves), lds, stream, args);
  else
    hipLaunchKernelGGL((gemv_s2_mfma_kernel<kSW, false>), dim3(blocks), dim3(64 * waves), lds, stream, args);
  return hipGetLastError();
}

}  // namespace tgs
