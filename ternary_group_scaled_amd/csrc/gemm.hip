// Ternary group-scaled GEMM (prefill, many activation rows) for gfx950 matrix cores.
//
// y[i][n] = sum_k s[n][k/128] * t[n][k] * x[i][k] with x in bf16. The decode of the packed codes
// and the group scale are fused into the product, the combination the CUDA backend of
// "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr) uses for prompt
// processing (section "Low-bit kernels for hybrid attention"); the format is the page's
// "Group-scaled ternary format" (w = s_g * t, one fp16 scale per 128 weights along K).
//
// Tiled product (any number of activation rows). A workgroup of 4 waves (2 x 2) computes a
// BM x BN tile of y and walks K one scale group (128) at a time, with the next group's data in
// flight while the current one is multiplied:
//   1. each thread's share of group g + 1 is loaded into registers: activation units of 16 k
//      values, and 16 bytes (64 codes) of one weight row;
//   2. meanwhile v_mfma_f32_16x16x32_bf16 runs over group g from LDS, and the group's partial is
//      scaled by 0.5 * s[n][g] in fp32 and added to the running sum (the scale never enters a
//      bf16 operand: rounding s to bf16 would cost 2^-9 relative);
//   3. after a barrier the registers go to LDS: activations reordered, weights decoded to bf16
//      2t in {-2, 0, +2} (exact; the factor 2 keeps the low byte of every bf16 zero, so one
//      v_perm table lookup makes two weights).
// Within every 16 consecutive k, both tiles are stored in the order 0,8,1,9,...,7,15 (the order
// the slot-2 decode produces pairs in); the contraction over k does not depend on that order.
// Binary codes (t in {-1, +1}, one bit per weight) decode the same way into bf16 2t in {-2, +2}.
// Up to 32 activation rows of slot-2 or binary codes take the skinny kernel further below instead.
#include <algorithm>

#include "tgs_internal.h"

namespace tgs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 128;
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 elements (16 bytes of padding)

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// word holding (e1 in the low half, e2 in the high half) from 16-bit elements packed in w
template <int E1, int E2>
__device__ __forceinline__ uint32_t pair16(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

// 16 consecutive k values (8 words) -> the 0,8,1,9,... order
__device__ __forceinline__ void interleave16(const uint32_t* w, uint32_t* out) {
  out[0] = pair16<0, 8>(w);
  out[1] = pair16<1, 9>(w);
  out[2] = pair16<2, 10>(w);
  out[3] = pair16<3, 11>(w);
  out[4] = pair16<4, 12>(w);
  out[5] = pair16<5, 13>(w);
  out[6] = pair16<6, 14>(w);
  out[7] = pair16<7, 15>(w);
}

// 16 slot-2 codes -> 8 words of bf16 pairs (2 t_i, 2 t_{i+8}).
// bf16(-2) = 0xC000, bf16(0) = 0, bf16(+2) = 0x4000: only the high byte differs, so the
// selector puts code q_i in byte 1 and q_{i+8} in byte 3 and 0x0C (a constant zero) in bytes
// 0 and 2, and v_perm reads the high byte from the table {0xC0, 0x00, 0x40}.
__device__ __forceinline__ void decode16_slot2(uint32_t u, uint32_t* out) {
  constexpr uint32_t kTable = 0x004000C0u;
  out[0] = __builtin_amdgcn_perm(0u, kTable, ((u << 8) & 0x03000300u) | 0x000C000Cu);
  out[1] = __builtin_amdgcn_perm(0u, kTable, ((u << 6) & 0x03000300u) | 0x000C000Cu);
  out[2] = __builtin_amdgcn_perm(0u, kTable, ((u << 4) & 0x03000300u) | 0x000C000Cu);
  out[3] = __builtin_amdgcn_perm(0u, kTable, ((u << 2) & 0x03000300u) | 0x000C000Cu);
  out[4] = __builtin_amdgcn_perm(0u, kTable, (u & 0x03000300u) | 0x000C000Cu);
  out[5] = __builtin_amdgcn_perm(0u, kTable, ((u >> 2) & 0x03000300u) | 0x000C000Cu);
  out[6] = __builtin_amdgcn_perm(0u, kTable, ((u >> 4) & 0x03000300u) | 0x000C000Cu);
  out[7] = __builtin_amdgcn_perm(0u, kTable, ((u >> 6) & 0x03000300u) | 0x000C000Cu);
}

// 16 binary codes (bits 0..15 of u, a set bit meaning t = +1) -> 8 words of bf16 pairs
// (2 t_i, 2 t_{i+8}): the bit picks the high byte from the table {0xC0, 0x40} (bf16 -2, +2)
__device__ __forceinline__ void decode16_binary(uint32_t u, uint32_t* out) {
  constexpr uint32_t kTable = 0x000040C0u;
  const uint32_t v = (u & 0xFFu) | ((u & 0xFF00u) << 8);  // bit i + 8 -> bit i + 16
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = __builtin_amdgcn_perm(0u, kTable, ((v << (8 - i)) & 0x01000100u) | 0x000C000Cu);
}

__device__ __forceinline__ uint16_t bf16_of_2t_digit(uint32_t digit) {
  // digit = t + 1 in {0, 1, 2} -> bf16(2t)
  return digit == 0 ? 0xC000u : (digit == 2 ? 0x4000u : 0u);
}

// Two waves per SIMD (at most 256 registers; slot-2), so that two workgroups share a CU and one's
// MFMAs run while the other waits on its loads (measured +40% at 2048 rows over one per CU).
// KS = 2 splits K between two halves of the workgroup (4 waves each, groups taken alternately,
// own LDS tiles); the second half's sums are added to the first's at the end, through LDS. It is
// used when the tiles alone give too few workgroups.
template <int LAYOUT, int BM, int BN, int KS>
__global__ __launch_bounds__(kThreads * KS)
__attribute__((amdgpu_waves_per_eu(LAYOUT == TGS_LAYOUT_BASE3 ? 1 : 2, 8))) void gemm_tile_kernel(
    const uint8_t* __restrict__ codes, int64_t stride, const uint16_t* __restrict__ scales, int n, int k,
    const uint16_t* __restrict__ x, int m, float* __restrict__ y) {
  constexpr int kWM = BM / 2, kWN = BN / 2;  // tile of one wave
  constexpr int kBlkM = kWM / 16, kBlkN = kWN / 16;
  constexpr int kXUnits = BM * 8 / kThreads;  // 16-value activation units per thread and group
  constexpr int kCodeThreads = BN * 2;        // threads that each hold 64 codes of one row

  __shared__ __attribute__((aligned(16))) uint16_t xs_all[KS][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ws_all[KS][BN * kPitch];

  const int kh = (int)threadIdx.x / kThreads;  // K half
  const int tid = (int)threadIdx.x % kThreads, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  uint16_t* xs = xs_all[kh];
  uint16_t* ws = ws_all[kh];
  const int n_base = blockIdx.x * BN, m_base = blockIdx.y * BM;
  const int groups = k / 128;

  // Rows past m (activations) and past n (codes, scales) land beyond their buffers and read as
  // zero; they only feed outputs that are never stored. Offsets are unsigned: the host keeps
  // m * k * 2 and n * stride below 2^31, and one tile more stays below 2^32.
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)((int64_t)m * k * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, 0, (int)((int64_t)n * stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);

  uint32_t xr[kXUnits][8];
  uint4 cr = make_uint4(0, 0, 0, 0);
  auto load_stage = [&](int g) {
#pragma unroll
    for (int u = 0; u < kXUnits; ++u) {
      const int unit = tid + u * kThreads, r = unit >> 3, c16 = (unit & 7) * 16;
      const uint32_t off = ((uint32_t)(m_base + r) * (uint32_t)k + (uint32_t)(g * 128 + c16)) * 2u;
      const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)off, 0, 0));
      const uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, (int)off + 16, 0, 0));
      xr[u][0] = a.x; xr[u][1] = a.y; xr[u][2] = a.z; xr[u][3] = a.w;
      xr[u][4] = b.x; xr[u][5] = b.y; xr[u][6] = b.z; xr[u][7] = b.w;
    }
    if (LAYOUT == TGS_LAYOUT_SLOT2 && tid < kCodeThreads) {
      const uint32_t off = (uint32_t)(n_base + (tid >> 1)) * (uint32_t)stride + (uint32_t)(g * 32 + 16 * (tid & 1));
      cr = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, (int)off, 0, kStreamAux));
    }
    if (LAYOUT == TGS_LAYOUT_BINARY && tid < kCodeThreads) {  // 64 codes are 8 bytes
      const uint32_t off = (uint32_t)(n_base + (tid >> 1)) * (uint32_t)stride + (uint32_t)(g * 16 + 8 * (tid & 1));
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, (int)off, 0, kStreamAux));
      cr.x = v.x;
      cr.y = v.y;
    }
  };
  auto store_stage = [&](int g) {
#pragma unroll
    for (int u = 0; u < kXUnits; ++u) {
      const int unit = tid + u * kThreads, r = unit >> 3, c16 = (unit & 7) * 16;
      uint32_t o[8];
      interleave16(xr[u], o);
      uint4* dst = reinterpret_cast<uint4*>(xs + r * kPitch + c16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    if (tid < kCodeThreads) {
      const int r = tid >> 1, h = tid & 1;
      uint32_t out[32];
      if (LAYOUT == TGS_LAYOUT_SLOT2) {
        decode16_slot2(cr.x, out + 0);
        decode16_slot2(cr.y, out + 8);
        decode16_slot2(cr.z, out + 16);
        decode16_slot2(cr.w, out + 24);
      } else if (LAYOUT == TGS_LAYOUT_BINARY) {
        decode16_binary(cr.x, out + 0);
        decode16_binary(cr.x >> 16, out + 8);
        decode16_binary(cr.y, out + 16);
        decode16_binary(cr.y >> 16, out + 24);
      } else {
        // base-3: digit by digit from the packed bytes (not on a measured path)
        const int row = n_base + r;
        uint32_t w[32];
        const int kk0 = g * 128 + 64 * h;
        for (int e = 0; e < 64; e += 2) {
          uint32_t lo = 0, hi = 0;
          if (row < n) {
            const uint8_t* rp = codes + (int64_t)row * stride;
            uint32_t d0 = rp[(kk0 + e) / 5], d1 = rp[(kk0 + e + 1) / 5];
            for (int j = 0; j < (kk0 + e) % 5; ++j) d0 /= 3;
            for (int j = 0; j < (kk0 + e + 1) % 5; ++j) d1 /= 3;
            lo = bf16_of_2t_digit(d0 % 3);
            hi = bf16_of_2t_digit(d1 % 3);
          }
          w[e / 2] = lo | (hi << 16);
        }
        for (int q = 0; q < 4; ++q) interleave16(w + 8 * q, out + 8 * q);
      }
      uint4* dst = reinterpret_cast<uint4*>(ws + r * kPitch + 64 * h);
#pragma unroll
      for (int v = 0; v < 8; ++v) dst[v] = make_uint4(out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]);
    }
  };

  f32x4 acc[kBlkM][kBlkN];
#pragma unroll
  for (int a = 0; a < kBlkM; ++a)
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  // this half takes groups kh, kh + KS, ...; both halves run the same number of iterations (the
  // barriers are shared), and a group index past the end is loaded harmlessly but not multiplied
  const int iters = (groups + KS - 1) / KS;
  load_stage(kh);
  store_stage(kh);
  __syncthreads();
  for (int i = 0; i < iters; ++i) {
    const int g = i * KS + kh;
    const bool more = i + 1 < iters;
    if (more) load_stage(g + KS);
    // this lane's output columns: their scales, loaded ahead of the MFMAs
    uint32_t sraw[kBlkN];
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) {
      const uint32_t col = (uint32_t)(n_base + wn * kWN + 16 * b + fr);
      sraw[b] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)((col * (uint32_t)groups + (uint32_t)g) * 2u), 0, 0);
    }
    f32x4 part[kBlkM][kBlkN];
#pragma unroll
    for (int a = 0; a < kBlkM; ++a)
#pragma unroll
      for (int b = 0; b < kBlkN; ++b) part[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af[kBlkM], bfr[kBlkN];
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(xs + (wm * kWM + 16 * a + fr) * kPitch + 32 * s + fk);
#pragma unroll
      for (int b = 0; b < kBlkN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(ws + (wn * kWN + 16 * b + fr) * kPitch + 32 * s + fk);
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int b = 0; b < kBlkN; ++b)
          part[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], part[a][b], 0, 0, 0);
    }
    if (KS == 1 || g < groups) {
#pragma unroll
      for (int b = 0; b < kBlkN; ++b) {
        const float sc = 0.5f * f16_to_f32((uint16_t)sraw[b]);  // the weights were decoded as 2t
#pragma unroll
        for (int a = 0; a < kBlkM; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(sc, part[a][b][r], acc[a][b][r]);
      }
    }
    __syncthreads();
    if (more) {
      store_stage(g + KS);
      __syncthreads();
    }
  }
  if constexpr (KS == 2) {
    // the second half hands its sums to the first (fixed order: first + second)
    float* red = reinterpret_cast<float*>(xs_all[1]);  // 4 waves x 64 lanes x kBlkM*kBlkN*4 floats
    static_assert(kBlkM * kBlkN * 4 * 256 * 4 <= BM * kPitch * 2, "reduction buffer fits the tile");
    if (kh == 1) {
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int b = 0; b < kBlkN; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((a * kBlkN + b) * 4 + r) * 256 + tid] = acc[a][b][r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int a = 0; a < kBlkM; ++a)
#pragma unroll
      for (int b = 0; b < kBlkN; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b][r] += red[((a * kBlkN + b) * 4 + r) * 256 + tid];
  }

  // epilogue: D[i][j] of a 16x16 block sits in lane (i/4)*16 + j, register i%4
#pragma unroll
  for (int a = 0; a < kBlkM; ++a)
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) {
      const int col = n_base + wn * kWN + 16 * b + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m_base + wm * kWM + 16 * a + 4 * (lane >> 4) + r;
        if (row < m && col < n) y[(int64_t)row * n + col] = acc[a][b][r];
      }
    }
}

// ---- skinny product: up to 32 activation rows, slot-2 or binary codes -----------------------
//
// With few activation rows the tile kernel above has too few workgroups (n / 128) to fill the
// chip, and its LDS round trips sit on the critical path. Here a workgroup of W waves owns
// 16 * FB outputs and 16 * TB activation rows, and splits K across its waves: wave w takes
// scale groups [w * G / W, (w + 1) * G / W). Every wave builds its MFMA operands in
// registers: x fragments straight from memory, weights decoded from 8 bytes of codes per lane
// per group. Within each 16 consecutive k, both operands use the order 0,8,1,9,...,7,15 of the
// slot-2 decode, so the contraction is unchanged. Each group's partial is scaled in fp32; the W
// per-wave results are added through LDS in wave order (deterministic, no atomics).
// Binary codes (BIN) take 4 bytes (32 weights) per lane per group and decode to the same pair order.
// Every workgroup reads all of x for its outputs, so x traffic from L2 falls as FB grows. The
// host picks FB so that a launch is about one workgroup per CU (one round of workgroups) rather
// than shrinking FB to get more workgroups.

// pairs 4H..4H+3 of decode16_slot2(u): bf16(2t_i) in the low half, bf16(2t_{i+8}) in the high half
template <int H>
__device__ __forceinline__ uint4 decode4_slot2(uint32_t u) {
  constexpr uint32_t kTable = 0x004000C0u;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * H + j;  // shift left by 8 - 2i (negative: right)
    const uint32_t v = i <= 4 ? (u << (8 - 2 * i)) : (u >> (2 * i - 8));
    o[j] = __builtin_amdgcn_perm(0u, kTable, (v & 0x03000300u) | 0x000C000Cu);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// pairs 4H..4H+3 of decode16_binary(u): bf16(2t_i) low, bf16(2t_{i+8}) high, from bits 0..15 of u
template <int H>
__device__ __forceinline__ uint4 decode4_binary(uint32_t u) {
  constexpr uint32_t kTable = 0x000040C0u;
  const uint32_t v = (u & 0xFFu) | ((u & 0xFF00u) << 8);  // bit i + 8 -> bit i + 16
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * H + j;
    o[j] = __builtin_amdgcn_perm(0u, kTable, ((v << (8 - i)) & 0x01000100u) | 0x000C000Cu);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// pairs 4H..4H+3 of interleave16 over 16 consecutive bf16 values in w[0..7]
template <int H>
__device__ __forceinline__ uint4 interleave4(const uint32_t* w) {
  if constexpr (H == 0)
    return make_uint4(pair16<0, 8>(w), pair16<1, 9>(w), pair16<2, 10>(w), pair16<3, 11>(w));
  else
    return make_uint4(pair16<4, 12>(w), pair16<5, 13>(w), pair16<6, 14>(w), pair16<7, 15>(w));
}

template <int TB, int kFB, int kWaves, int kStages, bool BIN>
__global__ __launch_bounds__(kWaves * 64) void gemm_skinny_kernel(const uint8_t* __restrict__ codes, int64_t stride,
                                                          const uint16_t* __restrict__ scales, int n, int k,
                                                          const uint16_t* __restrict__ x, int m,
                                                          float* __restrict__ y) {
  // kFB: 16-output blocks per workgroup; kWaves: K slices (waves) per workgroup; kStages: groups
  // of loads in flight per wave
  __shared__ float red[kWaves][TB * kFB * 4][64];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int fr = lane & 15, kq = lane >> 4;  // fragment row and k quarter
  const int n_base = blockIdx.x * 16 * kFB, m_base = blockIdx.y * 16 * TB;
  const int groups = k / 128;
  const int g_begin = wave * groups / kWaves, g_end = (wave + 1) * groups / kWaves;

  // reads past each buffer (rows >= n, activation rows >= m) return zero
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, 0, (int)((int64_t)n * stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)((int64_t)m * k * 2), kRsrcWord3);

  // per lane: output row (feature) n_base + 16 fb + fr reads 8 bytes of codes per group at 8 * kq;
  // activation row m_base + 16 tb + fr reads 32 values per group at 32 * kq
  // Rows past n and activation rows past m land beyond their buffer and read as zero. The
  // offsets are unsigned: n * stride <= 2^31 - 2^20 and 64 rows more add at most 2^30, and m <= 32,
  // so none wraps around.
  uint32_t code_off[kFB], scale_off[kFB], x_off[TB];
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb) {
    const uint32_t row = (uint32_t)(n_base + 16 * fb + fr);
    code_off[fb] = row * (uint32_t)stride + (BIN ? 4u : 8u) * (uint32_t)kq;
    scale_off[fb] = row * (uint32_t)groups * 2u;
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const uint32_t row = (uint32_t)(m_base + 16 * tb + fr);
    x_off[tb] = (row * (uint32_t)k + 32u * (uint32_t)kq) * 2u;
  }

  struct Stage {
    uint32_t cw[kFB][2];
    uint32_t sc[kFB];
    uint32_t xv[TB][16];
  };
  // Every workgroup reads the same activations; if all started at the same group, hundreds of CUs
  // would request the same few L2 lines at once. Each workgroup walks its waves' groups in a
  // rotated order instead: its i-th group is g_begin + (i + rot) mod count.
  const int count = g_end - g_begin;
  const int rot = count > 0 ? (int)(blockIdx.x % (unsigned)count) : 0;
  auto load = [&](Stage& st, int i) {
    const bool live = i < count;
    int g = g_begin + i + rot;
    if (g >= g_end) g -= count;
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      if constexpr (BIN) {  // 16 bytes of codes per group
        const int off = live ? (int)(code_off[fb] + 16u * (uint32_t)g) : kOobOffset;
        st.cw[fb][0] = __builtin_amdgcn_raw_buffer_load_b32(code_rsrc, off, 0, 0);
        st.cw[fb][1] = 0;
      } else {  // 32 bytes of codes per group
        const int off = live ? (int)(code_off[fb] + 32u * (uint32_t)g) : kOobOffset;
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, off, 0, 0);
        st.cw[fb][0] = v[0];
        st.cw[fb][1] = v[1];
      }
      st.sc[fb] = __builtin_amdgcn_raw_buffer_load_b16(
          scale_rsrc, live ? (int)(scale_off[fb] + 2u * (uint32_t)g) : kOobOffset, 0, 0);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int off = live ? (int)(x_off[tb] + 256u * (uint32_t)g + 16u * (uint32_t)v) : kOobOffset;
        const uint4 q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off, 0, 0));
        st.xv[tb][4 * v + 0] = q.x;
        st.xv[tb][4 * v + 1] = q.y;
        st.xv[tb][4 * v + 2] = q.z;
        st.xv[tb][4 * v + 3] = q.w;
      }
  };

  f32x4 acc[TB][kFB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) acc[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& st) {
    f32x4 part[TB][kFB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) part[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // 32 k per step: this lane's k quarter holds 8 of them
      bf16x8 a[TB], b[kFB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        a[tb] = __builtin_bit_cast(bf16x8, (s & 1) ? interleave4<1>(st.xv[tb] + 8 * (s >> 1))
                                                   : interleave4<0>(st.xv[tb] + 8 * (s >> 1)));
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) {
        if constexpr (BIN)  // step s: bits 16 (s >> 1) .. + 15 of the lane's word
          b[fb] = __builtin_bit_cast(bf16x8, (s & 1) ? decode4_binary<1>(st.cw[fb][0] >> (16 * (s >> 1)))
                                                     : decode4_binary<0>(st.cw[fb][0] >> (16 * (s >> 1))));
        else
          b[fb] = __builtin_bit_cast(bf16x8, (s & 1) ? decode4_slot2<1>(st.cw[fb][s >> 1])
                                                     : decode4_slot2<0>(st.cw[fb][s >> 1]));
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int fb = 0; fb < kFB; ++fb)
          part[tb][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], b[fb], part[tb][fb], 0, 0, 0);
    }
    // D[i][j] (activation row i, output j) sits in lane 16 * (i / 4) + j, register i % 4
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      const float sc = 0.5f * f16_to_f32((uint16_t)st.sc[fb]);  // the weights were decoded as 2t
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tb][fb][r] = fmaf(sc, part[tb][fb][r], acc[tb][fb][r]);
    }
  };

  // kStages groups of loads in flight; a stage is reloaded as soon as it has been multiplied
  // (loads past the wave's last group are parked out of range, so every load is unconditional
  // and the compiler's wait counts stay exact)
  Stage st[kStages];
#pragma unroll
  for (int u = 0; u < kStages; ++u) load(st[u], u);
  for (int base = 0; base < count; base += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      if (base + u < count) compute(st[u]);
      load(st[u], base + u + kStages);
    }
  }

#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(tb * kFB + fb) * 4 + r][lane] = acc[tb][fb][r];
  __syncthreads();
  for (int e = threadIdx.x; e < TB * kFB * 4 * 64; e += kWaves * 64) {
    const int idx = e >> 6, ln = e & 63;
    const int tb = idx / (kFB * 4), fb = (idx / 4) % kFB, r = idx % 4;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w][idx][ln];
    const int row = m_base + 16 * tb + 4 * (ln >> 4) + r, col = n_base + 16 * fb + (ln & 15);
    if (row < m && col < n) y[(int64_t)row * n + col] = sum;
  }
}

template <int LAYOUT>
hipError_t launch_layout(const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n, int64_t k,
                         const uint16_t* x, int64_t m, float* y, hipStream_t stream) {
  constexpr bool kBin = LAYOUT == TGS_LAYOUT_BINARY;
  if ((LAYOUT == TGS_LAYOUT_SLOT2 || kBin) && m <= 32) {
    const int ni = (int)n, ki = (int)k, mi = (int)m;
    if (m <= 16) {
      // 16 * FB outputs per workgroup of 8 waves, FB = n / 4096 rounded up, within 2..6: about one
      // workgroup per CU (the kernel's registers allow one), and every workgroup reads all of x,
      // so its L2 traffic falls as FB grows. (Measured on 17408 x 5120 and 5120 x 17408: FB = 5
      // and 2 beat both neighbours and the 16-wave variants.)
      const int64_t fb = std::min<int64_t>(6, std::max<int64_t>(2, (n + 4095) / 4096));
      const dim3 grid((unsigned)((n + 16 * fb - 1) / (16 * fb)));
#define TGS_SKINNY(FB_)                                                                                          \
  hipLaunchKernelGGL((gemm_skinny_kernel<1, FB_, 8, 2, kBin>), grid, dim3(512), 0, stream, codes, stride, scales, ni, \
                     ki, x, mi, y)
      switch (fb) {
        case 2: TGS_SKINNY(2); break;
        case 3: TGS_SKINNY(3); break;
        case 4: TGS_SKINNY(4); break;
        case 5: TGS_SKINNY(5); break;
        default: TGS_SKINNY(6); break;
      }
#undef TGS_SKINNY
    } else {
      // 16 outputs per block: the most (4, 2, 1) that still gives 512 workgroups
      const int64_t fb = (n + 63) / 64 >= 512 ? 4 : ((n + 31) / 32 >= 512 ? 2 : 1);
      const dim3 grid((unsigned)((n + 16 * fb - 1) / (16 * fb)), (unsigned)((m + 31) / 32));
      if (fb == 4)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 4, 8, 3, kBin>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
      else if (fb == 2)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 2, 8, 3, kBin>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 1, 8, 3, kBin>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
    }
    return hipGetLastError();
  }
  // tiles: 128 x 128 for many activation rows, else 64 rows; 64 columns when 128 gives too few tiles;
  // K split in two inside the workgroup when even then there are fewer than 512 tiles
  const int bm = m > 128 ? 128 : 64;
  const int64_t m_tiles = (m + bm - 1) / bm;
  const int bn = (n + 127) / 128 * m_tiles >= 512 ? 128 : 64;
  const int64_t tiles = (n + bn - 1) / bn * m_tiles;
  const bool ks2 = tiles < 512 && k / 128 >= 16;
  const dim3 grid((unsigned)((n + bn - 1) / bn), (unsigned)m_tiles);
  const int ni = (int)n, ki = (int)k, mi = (int)m;
#define TGS_TILE(BM_, BN_, KS_)                                                                           \
  hipLaunchKernelGGL((gemm_tile_kernel<LAYOUT, BM_, BN_, KS_>), grid, dim3(kThreads * KS_), 0, stream, codes, \
                     stride, scales, ni, ki, x, mi, y)
  // (128-column tiles are only chosen with >= 512 tiles, so never with the K split)
  if (bm == 128 && bn == 128) {
    TGS_TILE(128, 128, 1);
  } else if (bm == 128) {
    if (ks2) TGS_TILE(128, 64, 2); else TGS_TILE(128, 64, 1);
  } else if (bn == 128) {
    TGS_TILE(64, 128, 1);
  } else {
    if (ks2) TGS_TILE(64, 64, 2); else TGS_TILE(64, 64, 1);
  }
#undef TGS_TILE
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_launch(int32_t layout, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x_bf16, int64_t m, float* y, hipStream_t stream) {
  // activation rows per launch: the kernels address x with 32-bit offsets (m * k * 2 < 2^31)
  const int64_t max_rows = std::max<int64_t>(128, (kMaxDeviceCodeBytes / (2 * k)) / 128 * 128);
  for (int64_t r0 = 0; r0 < m; r0 += max_rows) {
    const int64_t mr = std::min(max_rows, m - r0);
    const uint16_t* xr = x_bf16 + r0 * k;
    float* yr = y + r0 * n;
    const hipError_t e =
        layout == TGS_LAYOUT_SLOT2   ? launch_layout<TGS_LAYOUT_SLOT2>(codes, stride, scales, n, k, xr, mr, yr, stream)
        : layout == TGS_LAYOUT_BASE3 ? launch_layout<TGS_LAYOUT_BASE3>(codes, stride, scales, n, k, xr, mr, yr, stream)
                                     : launch_layout<TGS_LAYOUT_BINARY>(codes, stride, scales, n, k, xr, mr, yr, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tgs
