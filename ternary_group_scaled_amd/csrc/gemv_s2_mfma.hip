// Single-token slot-2 GEMV on the matrix cores: m = 1, plain basis, K a multiple of 512, K <= 16384.
//
// y[j] = sum_k s[j][k/128] * t[j][k] * x[k], with the weights w = s_g * t of "Ternary Bonsai 2 27B,
// 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsection "Group-scaled ternary format": one
// fp16 scale per 128 consecutive weights of a row. The codes are read once, in packed form.
//
// Decode. Codes q = t + 1 sit in 2-bit slots, element j of a little-endian 32-bit word in bits
// 2j..2j+1. A pair (j, j+8) sits in bits p..p+1 of both 16-bit halves of the word, or of the word
// shifted right by 6 (p in {0, 2, 4, 6, 8}). One v_and_or_b32 keeps those bits and sets the
// exponent field 25 - p, which makes each half the fp16 number 2^(10-p) + q exactly; one packed
// fp16 add of -(2^(10-p) + 1) leaves t = q - 1 (-1.0, 0 or +1.0) in each half, again exactly. Two
// VALU operations per two weights, and no difference of sums: every product t * x is exact and a
// zero code adds nothing, so a row with one nonzero code gives s * t * x_k exactly.
//
// Multiply. v_mfma_f32_16x16x32_f16 computes D[r][c] = sum over 32 k of A[r][k] B[k][c]. B holds
// the weights: lane (c, q) (c = lane % 16, q = lane / 16) holds 8 weights of output row c. A window
// is 512 weights of 16 rows: lane (c, q) owns group q of the window (32 bytes of row c, two 16-byte
// loads; the four lanes of a row read its 128 contiguous bytes), and each of 16 MFMA steps takes
// 8 of its 128 weights. The activations go in A, row r holding the window's group r: lane (r, q)
// holds them only when r == q and zeros otherwise (rows 4..15 are all zero). So D[r][c] is the
// partial sum of group r for output row c: lane c holds all four groups' partials in its four D
// registers and scales each by its fp16 scale in fp32 (one 8-byte load of the four scales). The
// K-reduction inside a window happens in the matrix core; no cross-lane reduction is needed.
//
// Activations. The workgroup stages x once as dot2-style pairs (x_j, x_{j+8}) of every 16
// elements, in LDS, in the order of the weight operand: A fragment s of group g is 16 bytes at
// word 68 g + 4 s (64 words per group plus 4 of padding, so the four groups a step reads fall in
// different banks). Lanes whose A entries are zero read a 256-byte zero region instead, one shared
// address per step (a broadcast). RMSNorm (NORM): the staging threads first add the squares of
// their activations (fixed order: threads, waves in LDS), then scale by gamma / rms before the one
// rounding to fp16.
//
// Work split. A workgroup owns 16 rows and has one wave per SW windows of K. Each thread issues the
// loads of its staging activations first, then every code and scale load of its wave, so the
// staging waits only for the activations (vector-memory waits retire in issue order) and for the
// small launches of a decode step every load is in flight at once. A wave's windows run as
// independent MFMA chains, interleaved step by step. The waves' row sums meet in LDS and are added
// in wave order (deterministic, no atomics).
#include "lane_ops.h"
#include "rms_norm.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWinK = 512;           // weights of a row per window: four scale groups
constexpr int kGroupPitch = 68;      // LDS words per group of activation pairs (64 + 4)
constexpr int kZeroBytes = 16 * 16;  // one 16-byte zero fragment per MFMA step
constexpr int kSW = 2;               // windows per wave

// A 32-bit constant in a vector register: the three-operand AND-OR takes no literal, and its
// other constant (the mask) goes in a scalar register.
template <uint32_t V>
__device__ __forceinline__ uint32_t vconst() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}

// exponent bits that give the code bits p..p+1 the weight 1: 2^(10-p) + q in each half
template <int P>
constexpr uint32_t kExpBits = ((uint32_t)(25 - P) << 10) * 0x00010001u;

// t in both fp16 halves from the codes in bits P..P+1 of each half of `word`; exp_bits = vconst of
// kExpBits<P>
template <int P>
__device__ __forceinline__ uint32_t signed_pair(uint32_t word, uint32_t exp_bits) {
  constexpr uint32_t kMask = 0x00030003u << P;
  // -(2^(10-P) + 1) in both halves, exactly representable (11 significant bits at most)
  constexpr uint32_t kNeg = (0x8000u | ((uint32_t)(25 - P) << 10) | (1u << P)) * 0x00010001u;
  const half2v h = __builtin_bit_cast(half2v, (word & kMask) | exp_bits);
  return __builtin_bit_cast(uint32_t, h + __builtin_bit_cast(half2v, kNeg));
}

// Activation pair (element e1 in the low half, e2 in the high half) from fp16 words w[e/2].
template <int E1, int E2>
__device__ __forceinline__ uint32_t xpair(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

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
    if (u < units) {
      uint4* dst = reinterpret_cast<uint4*>(pairs + (u >> 3) * kGroupPitch + (u & 7) * 8);
      dst[0] = make_uint4(xpair<0, 8>(xw[i]), xpair<1, 9>(xw[i]), xpair<2, 10>(xw[i]), xpair<3, 11>(xw[i]));
      dst[1] = make_uint4(xpair<4, 12>(xw[i]), xpair<5, 13>(xw[i]), xpair<6, 14>(xw[i]), xpair<7, 15>(xw[i]));
    }
  }
  if (threadIdx.x < 16) reinterpret_cast<uint4*>(lds + zero_off)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // 4. the wave's windows, their MFMA chains interleaved step by step (independent accumulators);
  // a window past K reads the zero region and its scales are zero
  const uint32_t e0 = vconst<kExpBits<0>>(), e2 = vconst<kExpBits<2>>(), e4 = vconst<kExpBits<4>>(),
                 e6 = vconst<kExpBits<6>>(), e8 = vconst<kExpBits<8>>();
  const char* a_base[SW];
  f32x4 d[SW];
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const int w = w0 + i;
    a_base[i] = (col == q && w < windows) ? lds + (4 * w + q) * kGroupPitch * 4 : lds + zero_off;
    d[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 16; ++s) {
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      const half8 a = *reinterpret_cast<const half8*>(a_base[i] + 16 * s);
      const uint4& c = cw[i][s >> 3];
      const uint32_t u = (s & 6) == 0 ? c.x : ((s & 6) == 2 ? c.y : ((s & 6) == 4 ? c.z : c.w));
      uint4 b;
      if ((s & 1) == 0) {  // pairs j = 0..3: bits 0, 2, 4, 6 of u
        b = make_uint4(signed_pair<0>(u, e0), signed_pair<2>(u, e2), signed_pair<4>(u, e4), signed_pair<6>(u, e6));
      } else {  // pairs j = 4..7: bit 8 of u, bits 4, 6, 8 of u >> 6
        const uint32_t v = u >> 6;
        b = make_uint4(signed_pair<8>(u, e8), signed_pair<4>(v, e4), signed_pair<6>(v, e6), signed_pair<8>(v, e8));
      }
      d[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, b), d[i], 0, 0, 0);
    }
  }
  // D[g][col] (group g of the window) is register g of lane col
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    acc = fmaf(half_lo(sc[i].x), d[i][0], acc);
    acc = fmaf(half_hi(sc[i].x), d[i][1], acc);
    acc = fmaf(half_lo(sc[i].y), d[i][2], acc);
    acc = fmaf(half_hi(sc[i].y), d[i][3], acc);
  }

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

bool gemv_s2_mfma_fits(int64_t k) { return k % kWinK == 0 && k <= 16384; }

hipError_t gemv_s2_mfma_launch(GemvArgs& args, int32_t blocks, int64_t k, bool norm, hipStream_t stream) {
  const int waves = gemv_s2_mfma_waves(k);
  const size_t lds = (size_t)(k / 128) * kGroupPitch * 4 + kZeroBytes + (size_t)waves * 16 * 4;
  if (norm)
    hipLaunchKernelGGL((gemv_s2_mfma_kernel<kSW, true>), dim3(blocks), dim3(64 * waves), lds, stream, args);
  else
    hipLaunchKernelGGL((gemv_s2_mfma_kernel<kSW, false>), dim3(blocks), dim3(64 * waves), lds, stream, args);
  return hipGetLastError();
}

}  // namespace tgs
