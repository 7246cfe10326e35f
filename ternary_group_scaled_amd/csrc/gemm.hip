// Ternary group-scaled GEMM (prefill, many activation rows) for gfx950 matrix cores.
//
// y[i][n] = sum_k s[n][k/128] * t[n][k] * x[i][k] with x in bf16. The decode of the packed codes
// and the group scale are fused into the product, the combination the CUDA backend of
// "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr) uses for prompt
// processing (section "Low-bit kernels for hybrid attention"); the format is the page's
// "Group-scaled ternary format" (w = s_g * t, one fp16 scale per 128 weights along K).
//
// Tiling. A workgroup computes a BM x 128 tile of y and walks K one scale group (128) at a time:
//   1. the activation tile [BM][128] is copied into LDS;
//   2. the weight tile [128][128] is decoded from packed codes straight into LDS as bf16 values
//      2t in {-2, 0, +2} (exact; the factor 2 keeps the low byte of every bf16 zero, so one
//      v_perm table lookup makes two weights);
//   3. v_mfma_f32_16x16x32_bf16 accumulates the group's partial product in fp32;
//   4. the partial is scaled by 0.5 * s[n][g] in fp32 and added to the running sum.
// Step 4 keeps the scale out of the bf16 operands: rounding s to bf16 would cost 2^-9 relative.
// Within every 16 consecutive k, both tiles are stored in the order 0,8,1,9,...,7,15 (the order
// the slot-2 decode produces pairs in); the contraction over k does not depend on that order.
#include "tgs_internal.h"

namespace tgs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBN = 128;
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

__device__ __forceinline__ uint16_t bf16_of_2t_digit(uint32_t digit) {
  // digit = t + 1 in {0, 1, 2} -> bf16(2t)
  return digit == 0 ? 0xC000u : (digit == 2 ? 0x4000u : 0u);
}

template <int LAYOUT, int BM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ codes, int64_t stride,
                                                        const uint16_t* __restrict__ scales, int n, int k,
                                                        const uint16_t* __restrict__ x, int m,
                                                        float* __restrict__ y) {
  constexpr int kWavesN = (BM >= 64) ? 2 : 4;
  constexpr int kWavesM = 4 / kWavesN;
  constexpr int kWM = BM / kWavesM;       // rows of y per wave
  constexpr int kWN = kBN / kWavesN;      // columns of y per wave
  constexpr int kBlkM = kWM / 16, kBlkN = kWN / 16;

  __shared__ __attribute__((aligned(16))) uint16_t xs[BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ws[kBN * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int n_base = blockIdx.x * kBN, m_base = blockIdx.y * BM;
  const int groups = k / 128;

  f32x4 acc[kBlkM][kBlkN];
#pragma unroll
  for (int a = 0; a < kBlkM; ++a)
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < groups; ++g) {
    const int k0 = g * 128;
    __syncthreads();
    // 1. activations [BM][128] -> LDS, 16 k values per unit
    for (int u = tid; u < BM * 8; u += kThreads) {
      const int r = u >> 3, c16 = (u & 7) * 16;
      uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (m_base + r < m) {
        const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)(m_base + r) * k + k0 + c16);
        uint4 a = src[0], b = src[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
      }
      uint32_t o[8];
      interleave16(w, o);
      uint4* dst = reinterpret_cast<uint4*>(xs + r * kPitch + c16);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    // 2. weights [128][128] -> LDS as bf16(2t); each thread decodes 64 k values of one row
    {
      const int r = tid >> 1, h = tid & 1;
      const int row = n_base + r;
      uint32_t out[32];
      if (LAYOUT == TGS_LAYOUT_SLOT2) {
        uint4 cw = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);  // q = 1: t = 0
        if (row < n) cw = *reinterpret_cast<const uint4*>(codes + (int64_t)row * stride + k0 / 4 + 16 * h);
        decode16_slot2(cw.x, out + 0);
        decode16_slot2(cw.y, out + 8);
        decode16_slot2(cw.z, out + 16);
        decode16_slot2(cw.w, out + 24);
      } else {
        uint32_t w[32];
        const int kk0 = k0 + 64 * h;
        for (int e = 0; e < 64; e += 2) {
          uint32_t lo = 0, hi = 0;
          if (row < n) {
            const uint8_t* rp = codes + (int64_t)row * stride;
            uint32_t b0 = rp[(kk0 + e) / 5], b1 = rp[(kk0 + e + 1) / 5];
            uint32_t d0 = b0, d1 = b1;
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
    __syncthreads();

    // 3. MFMA over the group, 4 steps of 32 k
    f32x4 part[kBlkM][kBlkN];
#pragma unroll
    for (int a = 0; a < kBlkM; ++a)
#pragma unroll
      for (int b = 0; b < kBlkN; ++b) part[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fk = (lane >> 4) * 8;
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
    // 4. scale the group's partial by 0.5 * s[n][g] (the weights were decoded as 2t)
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) {
      const int col = n_base + wn * kWN + 16 * b + fr;
      const float sc = col < n ? 0.5f * f16_to_f32(scales[(int64_t)col * groups + g]) : 0.f;
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(sc, part[a][b][r], acc[a][b][r]);
    }
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

// ---- skinny product: up to 32 activation rows, slot-2 codes ----------------------------------
//
// With few activation rows the tile kernel above has too few workgroups (n / 128) to fill the
// chip, and its LDS round trips sit on the critical path. Here a workgroup of W waves owns
// 16 * FB outputs and 16 * TB activation rows, and splits K across its waves: wave w takes
// scale groups [w * G / W, (w + 1) * G / W). Every wave builds its MFMA operands in
// registers: x fragments straight from memory, weights decoded from 8 bytes of codes per lane
// per group. Within each 16 consecutive k, both operands use the order 0,8,1,9,...,7,15 of the
// slot-2 decode, so the contraction is unchanged. Each group's partial is scaled in fp32; the W
// per-wave results are added through LDS in wave order (deterministic, no atomics).
// Every workgroup reads all of x for its outputs, so x traffic from L2 falls as FB grows: the
// few-row case uses FB = 4 and keeps the kernel within 128 VGPRs (two stages), so that 16 waves
// fit on a CU, rather than shrinking FB to get more workgroups.

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

// pairs 4H..4H+3 of interleave16 over 16 consecutive bf16 values in w[0..7]
template <int H>
__device__ __forceinline__ uint4 interleave4(const uint32_t* w) {
  if constexpr (H == 0)
    return make_uint4(pair16<0, 8>(w), pair16<1, 9>(w), pair16<2, 10>(w), pair16<3, 11>(w));
  else
    return make_uint4(pair16<4, 12>(w), pair16<5, 13>(w), pair16<6, 14>(w), pair16<7, 15>(w));
}

template <int TB, int kFB, int kWaves, int kStages>
__global__ __launch_bounds__(kWaves * 64) void gemm_skinny_kernel(const uint8_t* __restrict__ codes, int64_t stride,
                                                          const uint16_t* __restrict__ scales, int n, int k,
                                                          const uint16_t* __restrict__ x, int m,
                                                          float* __restrict__ y) {
  // kFB: 16-output blocks per workgroup; kWaves: K slices (waves) per workgroup; kStages: groups
  // of loads in flight per wave
  __shared__ float red[kWaves][TB * kFB * 4][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    code_off[fb] = row * (uint32_t)stride + 8u * (uint32_t)kq;
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
      const int off = live ? (int)(code_off[fb] + 32u * (uint32_t)g) : kOobOffset;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, off, 0, 0);
      st.cw[fb][0] = v[0];
      st.cw[fb][1] = v[1];
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
      for (int fb = 0; fb < kFB; ++fb)
        b[fb] = __builtin_bit_cast(bf16x8, (s & 1) ? decode4_slot2<1>(st.cw[fb][s >> 1])
                                                   : decode4_slot2<0>(st.cw[fb][s >> 1]));
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
  if (LAYOUT == TGS_LAYOUT_SLOT2 && m <= 32) {
    const int ni = (int)n, ki = (int)k, mi = (int)m;
    if (m <= 16) {
      // 64 outputs per workgroup; 16 K slices when that gives too few workgroups to fill the chip
      const dim3 grid((unsigned)((n + 63) / 64));
      if ((n + 63) / 64 >= 256)
        hipLaunchKernelGGL((gemm_skinny_kernel<1, 4, 8, 2>), grid, dim3(512), 0, stream, codes, stride, scales, ni,
                           ki, x, mi, y);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<1, 4, 16, 2>), grid, dim3(1024), 0, stream, codes, stride, scales, ni,
                           ki, x, mi, y);
    } else {
      // 16 outputs per block: the most (4, 2, 1) that still gives 512 workgroups
      const int64_t fb = (n + 63) / 64 >= 512 ? 4 : ((n + 31) / 32 >= 512 ? 2 : 1);
      const dim3 grid((unsigned)((n + 16 * fb - 1) / (16 * fb)), (unsigned)((m + 31) / 32));
      if (fb == 4)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 4, 8, 3>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
      else if (fb == 2)
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 2, 8, 3>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
      else
        hipLaunchKernelGGL((gemm_skinny_kernel<2, 1, 8, 3>), grid, dim3(512), 0, stream, codes, stride, scales, ni, ki,
                           x, mi, y);
    }
    return hipGetLastError();
  }
  const unsigned gx = (unsigned)((n + kBN - 1) / kBN);
  if (m <= 16) {
    hipLaunchKernelGGL((gemm_kernel<LAYOUT, 16>), dim3(gx, (unsigned)((m + 15) / 16)), dim3(kThreads), 0, stream,
                       codes, stride, scales, (int)n, (int)k, x, (int)m, y);
  } else if (m <= 64) {
    hipLaunchKernelGGL((gemm_kernel<LAYOUT, 64>), dim3(gx, (unsigned)((m + 63) / 64)), dim3(kThreads), 0, stream,
                       codes, stride, scales, (int)n, (int)k, x, (int)m, y);
  } else {
    hipLaunchKernelGGL((gemm_kernel<LAYOUT, 128>), dim3(gx, (unsigned)((m + 127) / 128)), dim3(kThreads), 0,
                       stream, codes, stride, scales, (int)n, (int)k, x, (int)m, y);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_launch(int32_t layout, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x_bf16, int64_t m, float* y, hipStream_t stream) {
  if (layout == TGS_LAYOUT_SLOT2)
    return launch_layout<TGS_LAYOUT_SLOT2>(codes, stride, scales, n, k, x_bf16, m, y, stream);
  return launch_layout<TGS_LAYOUT_BASE3>(codes, stride, scales, n, k, x_bf16, m, y, stream);
}

}  // namespace tgs
