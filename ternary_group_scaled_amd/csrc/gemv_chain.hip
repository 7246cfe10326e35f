// A chain of single-token slot-2 GEMV steps in one launch: step t multiplies only after step t - 1
// is complete on every workgroup, exactly as if the steps were launched one by one on a stream (a
// decode step's projections in layer order), but the weights of step t are already streaming in
// while the workgroups wait for step t - 1.
//
// Each step is the product of "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)"
// (discuss.pytorch.kr), subsection "Group-scaled ternary format" (w = s_g * t, one fp16 scale per
// 128 weights), for one to three matrices sharing the step's input: y = W xh, where xh is the
// step's activation vector in fp16 (an fp32 input, such as an earlier step's output, is rounded
// to fp16 to nearest even), RMS-normalised first when the step asks for it (gamma in bf16; the
// norm of the BlockHadamard-with-RMSNorm variant of the same page, section "Running in the
// browser with WebGPU"). The matrix-core window, decode and activation pairs are those of
// s2_mfma.h.
//
// Launch. One workgroup per compute unit (the grid is the device's compute-unit count and the
// workgroup's registers and LDS leave room for one per unit), so every workgroup is resident and
// the waits between steps cannot deadlock; every wait is bounded besides (see below).
//
// Roles. Each workgroup has 16 waves:
//   - 12 compute waves. Step t's work of the workgroup is its 16-row blocks rb = wg, wg + G, ...
//     times the K windows of 512 weights; item i of the list goes to compute wave i % 12. A
//     compute wave keeps up to 4 items' code and scale loads in flight (a register ring), and
//     issues the loads of its first items of step t + 1 as soon as step t's row sums are in LDS,
//     before any wait: weights never depend on the activations. Items are multiplied two at a time (two
//     interleaved MFMA chains) and each item's row sums (scaled per group in fp32) go to LDS.
//   - 4 staging waves. They read and stage step t's activations (vector loads of their own, so
//     their waits never include the weight stream: vector-memory waits retire in issue order per
//     wave), and the first of them adds each row block's window sums in window order, stores y,
//     publishes the workgroup's completed-step count and polls the other workgroups' counts.
//
// Step boundary. The workspace holds one word per workgroup: the number of steps that workgroup
// has completed over all chain launches that used the workspace (plus an error word). Each
// workgroup reads its own count c0 when the launch starts; since every launch runs every step on
// every workgroup, c0 is the same on all of them. After step t the publishing wave stores its y
// values at device coherence (sc1, written through to the memory side), waits until those stores
// have completed, and stores c0 + t + 1; before step t + 1 stages its input, the poller waits
// until every workgroup's word reaches c0 + t + 1 (wrap-around safe difference), and the staging
// waves then read the input at device coherence too. Neither side needs an L2 write-back or
// invalidation, and no atomic read-modify-write or reset is needed. A wait gives up
// after about 2^20 polls and sets the error word; a workgroup that sees the error word skips its
// remaining waits, so a launch always ends (with garbage outputs and the error word set).
//
// Determinism: fixed item assignment, fixed reduction orders, no float atomics.
#include <mutex>

#include "lane_ops.h"
#include "rms_norm.h"
#include "s2_mfma.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

using namespace s2;

constexpr int kComputeWaves = 12;
constexpr int kStageWaves = 4;
constexpr int kWaves = kComputeWaves + kStageWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kStageThreads = 64 * kStageWaves;
constexpr int kRing = 4;      // items in flight per compute wave
constexpr int kPrefetch = 1;  // of which loaded before the wait for the previous step
constexpr int kMaxWindows = kMaxK / kWinK;
constexpr int kMaxUnitsPerStager = kMaxK / 16 / kStageThreads;
constexpr uint32_t kMaxPolls = 1u << 20;
// cache policy of loads that must see other workgroups' coherent stores: sc1 (device coherence)
constexpr int kCoherentAux = 16;
// LDS: activation pairs for the largest K, the zero region, the items' row sums [rb][window][16]
constexpr int kPairRegion = pair_bytes(kMaxK);
constexpr int kPartOffset = kPairRegion + kZeroBytes;
constexpr int kPartBytes = kChainMaxRbsPerWg * kMaxWindows * 16 * 4;
// more than half of a compute unit's 160 KB: one workgroup per unit whatever the registers allow
constexpr int kLdsBytes = 81 * 1024;
static_assert(kPartOffset + kPartBytes <= kLdsBytes, "LDS layout fits");

// The matrix of a step that row block rb belongs to (uniform)
__device__ __forceinline__ int mat_of(const ChainStep& st, int rb) {
  int m = 0;
  if (st.count > 1 && rb >= st.mat[1].rb0) m = 1;
  if (st.count > 2 && rb >= st.mat[2].rb0) m = 2;
  return m;
}

// Loads of item i of step st for this wave's lanes: row block j = i / windows of the workgroup
// (global rb = wg + j G), window w = i % windows. Items past the list (i >= items) park their
// loads out of range (zero data, no traffic).
__device__ __forceinline__ void load_item(uint4* c, uint2& sc, const ChainStep& st, int i, int items, int wg, int G,
                                          int col, int q) {
  const int windows = st.k / kWinK, groups = st.k >> 7;
  const bool live = i < items;
  const int j = live ? i / windows : 0, w = live ? i - j * windows : 0;
  const int rb = wg + j * G;
  const ChainMat& mt = st.mat[mat_of(st, rb)];
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)mt.codes, 0, (int)((int64_t)mt.n * mt.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)mt.scales, 0, (int)((int64_t)mt.n * groups * 2), kRsrcWord3);
  const uint32_t row = (uint32_t)((rb - mt.rb0) * 16 + col);
  const int off = live ? (int)(__umul24(row, (uint32_t)mt.stride) + (uint32_t)(w * 128 + q * 32)) : kOobOffset;
  c[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, off, 0, kStreamAux));
  c[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, live ? off + 16 : kOobOffset, 0,
                                                                          kStreamAux));
  const int soff = (live && q == 0) ? (int)(__umul24(row, (uint32_t)groups) * 2u + (uint32_t)(w * 8)) : kOobOffset;
  sc = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(scale_rsrc, soff, 0, 0));
}

__device__ __forceinline__ int items_of(const ChainStep& st, int wg, int G) {
  const int my_rbs = wg < st.rbs ? (st.rbs - wg + G - 1) / G : 0;
  return my_rbs * (st.k / kWinK);
}

// The shared memory of a chain workgroup
struct ChainLds {
  uint32_t* pairs;    // activation pairs of the current step
  const char* zero;   // the zero region
  float* part;        // [rb][window][16] row sums of the items
  float* norm_part;   // [kStageWaves] sums of squares
  int* failed;        // a wait gave up: skip the remaining waits
};

// Compute waves (wave index cw < kComputeWaves). Barriers per step, in the same order as the
// staging waves: B0 (t > 0), B1a (norm steps), B1, B2.
__device__ __forceinline__ void compute_role(const ChainArgs& args, const ChainLds& sm, int cw, int wg, int G,
                                             int lane) {
  const int col = lane & 15, q = lane >> 4;
  const ExpBits e = exp_bits();
  uint4 rc[kRing][2];
  uint2 rs[kRing];
  {
    const int items0 = items_of(args.step[0], wg, G);
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u)
      if (cw + kComputeWaves * u < items0) load_item(rc[u], rs[u], args.step[0], cw + kComputeWaves * u, items0, wg, G, col, q);
  }
  for (int t = 0; t < args.count; ++t) {
    const ChainStep& st = args.step[t];
    const int windows = st.k / kWinK;
    const int items = items_of(st, wg, G);
    if (t > 0) __syncthreads();     // B0: step t - 1 complete everywhere
    if (st.norm) __syncthreads();   // B1a
    __syncthreads();                // B1: activations staged
    // the ring slots not prefetched across the step boundary
#pragma unroll
    for (int u = kPrefetch; u < kRing; ++u)
      if (cw + kComputeWaves * u < items) load_item(rc[u], rs[u], st, cw + kComputeWaves * u, items, wg, G, col, q);
    const int mine = items > cw ? (items - cw + kComputeWaves - 1) / kComputeWaves : 0;
    for (int p0 = 0; p0 < mine; p0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; u += 2) {
        const int pa = p0 + u;
        const char* lds = reinterpret_cast<const char*>(sm.pairs);
        if (pa + 1 < mine) {
          // two items, as interleaved MFMA chains
          const int ia = cw + kComputeWaves * pa, ib = ia + kComputeWaves;
          const int ja = ia / windows, wa = ia - ja * windows;
          const int jb = ib / windows, wb = ib - jb * windows;
          const char* ab[2] = {col == q ? lds + (4 * wa + q) * kGroupPitch * 4 : sm.zero,
                               col == q ? lds + (4 * wb + q) * kGroupPitch * 4 : sm.zero};
          f32x4 d[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          mfma_windows<2>(ab, rc + u, d, e);
          const float sa = scale_window(0.f, rs[u], d[0]), sb = scale_window(0.f, rs[u + 1], d[1]);
          if (lane < 16) {
            sm.part[(ja * kMaxWindows + wa) * 16 + lane] = sa;
            sm.part[(jb * kMaxWindows + wb) * 16 + lane] = sb;
          }
        } else if (pa < mine) {
          // the wave's last item alone
          const int ia = cw + kComputeWaves * pa;
          const int ja = ia / windows, wa = ia - ja * windows;
          const char* ab[1] = {col == q ? lds + (4 * wa + q) * kGroupPitch * 4 : sm.zero};
          f32x4 d[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
          mfma_windows<1>(ab, rc + u, d, e);
          const float sa = scale_window(0.f, rs[u], d[0]);
          if (lane < 16) sm.part[(ja * kMaxWindows + wa) * 16 + lane] = sa;
        }
        // the refills must not move above the uses of the slots: a later load waited on early
        // would make every earlier one wait for it (waits retire in issue order)
        __builtin_amdgcn_sched_barrier(0);
        // refill the two slots with the items kRing positions further on, when there are any
        if (pa + kRing < mine) {
          load_item(rc[u], rs[u], st, cw + kComputeWaves * (pa + kRing), items, wg, G, col, q);
          load_item(rc[u + 1], rs[u + 1], st, cw + kComputeWaves * (pa + 1 + kRing), items, wg, G, col, q);
        }
      }
    }
    __syncthreads();  // B2: every item's row sums are in LDS
    // step t + 1's first items: their weights stream in while the workgroups publish step t and
    // wait for each other (issued after B2: the memory pipeline takes them only as fast as earlier
    // loads drain, and the publication of step t must not wait for that)
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < args.count) {
      const ChainStep& nx = args.step[t + 1];
      const int items1 = items_of(nx, wg, G);
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u)
        if (cw + kComputeWaves * u < items1) load_item(rc[u], rs[u], nx, cw + kComputeWaves * u, items1, wg, G, col, q);
    }
  }
}

// Staging waves (sw = wave - kComputeWaves). The first one also polls, reduces and publishes.
__device__ __forceinline__ void stage_role(const ChainArgs& args, const ChainLds& sm, int sw, int wg, int G, int lane,
                                           uint32_t c0) {
  uint32_t* flags = args.flags;
  const int st_tid = sw * 64 + lane;
  for (int t = 0; t < args.count; ++t) {
    const ChainStep& st = args.step[t];
    const int k = st.k, windows = k / kWinK, units = k >> 4;

    // ---- the norm weights do not depend on the previous step: load them before the wait
    uint32_t xw[kMaxUnitsPerStager][8];
    uint32_t gw[kMaxUnitsPerStager][8];
    if (st.norm) {
      const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)st.gamma, 0, k * 2, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kMaxUnitsPerStager; ++i) {
        const int u = st_tid + i * kStageThreads;
        const bool live = u < units;
        const uint4 a =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, live ? u * 32 : kOobOffset, 0, 0));
        const uint4 b = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, live ? u * 32 + 16 : kOobOffset, 0, 0));
        gw[i][0] = a.x; gw[i][1] = a.y; gw[i][2] = a.z; gw[i][3] = a.w;
        gw[i][4] = b.x; gw[i][5] = b.y; gw[i][6] = b.z; gw[i][7] = b.w;
      }
    }

    // ---- B0: wait until step t - 1 is complete on every workgroup. The outputs of step t - 1
    // were stored coherently (below) and are read coherently: no cache maintenance is needed.
    if (t > 0) {
      if (sw == 0 && !*sm.failed) {
        uint32_t polls = 0;
        while (true) {
          bool ok = true;
          for (int i = lane; i < G; i += 64)
            ok &= (int)(__hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - c0) >= t;
          const bool err = __hip_atomic_load(flags + G, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
          if (__ballot(!ok) == 0) break;
          if (err || ++polls > kMaxPolls) {
            if (lane == 0) {
              __hip_atomic_store(flags + G, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              *sm.failed = 1;
            }
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
    }

    // ---- the activations: fp16 words (rounded from fp32 inputs), then optional RMSNorm, pairs.
    // An input may be an earlier step's output, written by other workgroups: read it at device
    // coherence (sc1), past any stale cached copy.
    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)st.x, 0, k * (st.x_f32 ? 4 : 2), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kMaxUnitsPerStager; ++i) {
      const int u = st_tid + i * kStageThreads;
      const bool live = u < units;
      if (st.x_f32) {
        float f[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        x_rsrc, live ? u * 64 + 16 * v : kOobOffset, 0, kCoherentAux));
          f[4 * v] = __builtin_bit_cast(float, a.x);
          f[4 * v + 1] = __builtin_bit_cast(float, a.y);
          f[4 * v + 2] = __builtin_bit_cast(float, a.z);
          f[4 * v + 3] = __builtin_bit_cast(float, a.w);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xw[i][j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * j]) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f[2 * j + 1]) << 16);
      } else {
        const uint4 a = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? u * 32 : kOobOffset, 0, kCoherentAux));
        const uint4 b = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? u * 32 + 16 : kOobOffset, 0, kCoherentAux));
        xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
        xw[i][4] = b.x; xw[i][5] = b.y; xw[i][6] = b.z; xw[i][7] = b.w;
      }
    }
    if (st.norm) {
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxUnitsPerStager; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) sq = add_squares(xw[i][j], sq);  // zero past the end
      sq = wave_sum(sq, lane);
      if (lane == 0) sm.norm_part[sw] = sq;
      __syncthreads();  // B1a
      float total = 0.f;
#pragma unroll
      for (int w = 0; w < kStageWaves; ++w) total += sm.norm_part[w];
      const float r = rms_scale(total, k, st.eps);
#pragma unroll
      for (int i = 0; i < kMaxUnitsPerStager; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) xw[i][j] = norm_word(xw[i][j], gw[i][j], r);
    }
#pragma unroll
    for (int i = 0; i < kMaxUnitsPerStager; ++i) {
      const int u = st_tid + i * kStageThreads;
      if (u < units) store_unit_pairs(sm.pairs, u, xw[i]);
    }
    __syncthreads();  // B1: the activations are staged
    __syncthreads();  // B2: the compute waves' row sums are in LDS

    // ---- the first staging wave: add the windows in order, store y, publish the count
    if (sw == 0) {
      const int my_rbs = wg < st.rbs ? (st.rbs - wg + G - 1) / G : 0;
      for (int r = lane; r < my_rbs * 16; r += 64) {
        const int j = r >> 4, row = r & 15;
        float sum = 0.f;
        for (int w = 0; w < windows; ++w) sum += sm.part[(j * kMaxWindows + w) * 16 + row];
        const int rb = wg + j * G;
        const ChainMat& mt = st.mat[mat_of(st, rb)];
        const int grow = (rb - mt.rb0) * 16 + row;
        // stored at device coherence (sc1), so the count below publishes them without an L2 write-back
        if (grow < mt.n) __hip_atomic_store(mt.y + grow, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // every store of this wave has completed before the count that publishes them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0) __hip_atomic_store(flags + wg, c0 + (uint32_t)t + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ __launch_bounds__(kThreads) void gemv_chain_kernel(const ChainArgs args) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ float norm_part[kStageWaves];
  __shared__ uint32_t sh_c0;
  __shared__ int sh_failed;
  const int G = (int)gridDim.x, wg = (int)blockIdx.x;
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ChainLds sm{reinterpret_cast<uint32_t*>(lds), lds + kPairRegion, reinterpret_cast<float*>(lds + kPartOffset),
                    norm_part, &sh_failed};
  if (tid < 16) reinterpret_cast<uint4*>(lds + kPairRegion)[tid] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) {
    sh_c0 = __hip_atomic_load(args.flags + wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_failed = 0;
  }
  __syncthreads();
  // the two roles keep no values in common, so each gets the registers of its own path
  if (wave >= kComputeWaves)
    stage_role(args, sm, wave - kComputeWaves, wg, G, lane, sh_c0);
  else
    compute_role(args, sm, wave, wg, G, lane);
}

__global__ __launch_bounds__(256) void chain_clear_kernel(uint32_t* words, int32_t count) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < count) words[i] = 0u;
}

// The workspace of chains launched without one: one array per device, alive until the process
// ends. In host code `scratch` names a host-side stand-in, never the device memory: the device
// address comes from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint32_t scratch[kChainStaticWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint32_t* g_scratch[kMaxDevices];

}  // namespace

hipError_t chain_static_workspace(uint32_t** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t chain_clear(uint32_t* words, int32_t count, hipStream_t stream) {
  hipLaunchKernelGGL(chain_clear_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, words, count);
  return hipGetLastError();
}

int chain_grid() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return -1;
  return cus;
}

hipError_t chain_launch(const ChainArgs& args, int32_t grid, hipStream_t stream) {
  hipLaunchKernelGGL(gemv_chain_kernel, dim3(grid), dim3(kThreads), kLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace tgs
