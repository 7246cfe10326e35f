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
//   3. after a barrier the registers go to LDS: activations as loaded, weights decoded to bf16
//      2t in {-2, 0, +2} (exact; the factor 2 keeps the low byte of every bf16 zero, so one
//      v_perm table lookup makes two weights).
// Both tiles hold k in its natural order. Binary codes (t in {-1, +1}, one bit per weight) decode
// the same way into bf16 2t in {-2, +2}.
// Up to 32 activation rows of slot-2 or binary codes take the skinny kernel further below instead.
//
// K split across workgroups (both kernels). When a launch would leave CUs idle, some outputs are
// computed in P parts: part p walks the scale groups [p G / P, (p + 1) G / P). Part 0 writes y,
// part p > 0 writes its sums to a caller-supplied workspace, and a second kernel adds the parts
// into y in part order: y = ((y_0 + y_1) + y_2) + ... The sum is deterministic (fixed order, no
// atomics) and nothing is allocated. The skinny kernel splits every output ([m][n] workspace slice
// per part); the tiled kernel takes whole tiles first, for as many full rounds of workgroups as
// the tiles fill, and splits only the tiles left over for the last round ([tile][BM][BN] slices).
#include <algorithm>

#include "tgs_internal.h"

namespace tgs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 128;
constexpr int kPitch = kBK + 16;  // LDS row pitch in bf16 elements (32 bytes of padding: measured best of 132..168)
// K split across workgroups: the workgroups a launch of 64 x 64 tiles (4 waves each) aims for
constexpr int64_t kTileTarget = 640;
// ... and the fewest 128-groups a part keeps: with fewer, a wave has too few groups to stream
// (measured: 17408 x 5120, 40 groups, is slower in two parts at 16 and 128 rows)
constexpr int64_t kMinPartGroups = 32;
// skinny kernel, scales staged in LDS: b16 loads per thread (512 threads), so at most
// 512 * kSkinnyScaleLoads scales per workgroup take that path
constexpr int kSkinnyScaleLoads = 8;
// 128 x 128 tiles: workgroups resident at once (two per CU), and the fewest groups a part of a
// tail tile keeps
constexpr int64_t kTileSlots = 512;
constexpr int64_t kMinTailGroups = 8;

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Codes to bf16 weight pairs in natural k order (2 t_{2j} in the low half, 2 t_{2j+1} in the
// high half of word j). bf16(-2) = 0xC000, bf16(0) = 0, bf16(+2) = 0x4000: only the high byte
// differs. Two levels of v_perm, 19 VALU operations per 16 slot-2 codes:
//   1. spread: a shift and a mask put one code per byte (byte j of selector r: code 4j + r of a
//      slot-2 word, bit 8j + r of a binary word), and one v_perm per selector reads each byte's
//      high byte from a table; code 3, never written by the packer, reads as 0;
//   2. pair: one v_perm with a constant selector takes byte J of two spread words into bytes 1
//      and 3 of a word, with 0x0C (a constant zero) in bytes 0 and 2.
// word holding byte I of `lo` (in byte 1) and byte I of `hi` (in byte 3), zero low bytes
template <int I>
__device__ __forceinline__ uint32_t gather_pair(uint32_t hi, uint32_t lo) {
  constexpr uint32_t kSel = 0x0Cu | ((uint32_t)I << 8) | (0x0Cu << 16) | ((uint32_t)(4 + I) << 24);
  return __builtin_amdgcn_perm(hi, lo, kSel);
}

// byte j of d[r]: the bf16 high byte of code 4j + r of the 16 slot-2 codes in u (code i in
// bits 2i, 2i + 1)
// The table is a scalar register: v_perm may read one, and the compiler would otherwise keep
// the constant in a vector register, which the 128 x 128 tile kernel (at its 256-register limit)
// does not have to spare.
__device__ __forceinline__ uint32_t scalar_const(uint32_t v) {
  uint32_t r;
  __asm__("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}

__device__ __forceinline__ void spread_slot2(uint32_t u, uint32_t* d) {
  const uint32_t table = scalar_const(0x004000C0u);  // codes 0, 1, 2: t = -1, 0, +1
#pragma unroll
  for (int r = 0; r < 4; ++r) d[r] = __builtin_amdgcn_perm(0u, table, (u >> (2 * r)) & 0x03030303u);
}

// byte j of d[r]: the bf16 high byte of bit 8j + r of u (a set bit meaning t = +1)
__device__ __forceinline__ void spread_binary(uint32_t u, uint32_t* d) {
  const uint32_t table = scalar_const(0x000040C0u);  // bit 0, 1: t = -1, +1
#pragma unroll
  for (int r = 0; r < 8; ++r) d[r] = __builtin_amdgcn_perm(0u, table, (u >> r) & 0x01010101u);
}

// words 4H..4H+3 (codes 8H..8H+7) of a spread slot-2 word: word j pairs codes 2j and 2j + 1
template <int H>
__device__ __forceinline__ uint4 pairs4_slot2(const uint32_t* d) {
  return make_uint4(gather_pair<2 * H>(d[1], d[0]), gather_pair<2 * H>(d[3], d[2]),
                    gather_pair<2 * H + 1>(d[1], d[0]), gather_pair<2 * H + 1>(d[3], d[2]));
}

// words 4S..4S+3 (bits 8S..8S+7) of a spread binary word
template <int S>
__device__ __forceinline__ uint4 pairs4_binary(const uint32_t* d) {
  return make_uint4(gather_pair<S>(d[1], d[0]), gather_pair<S>(d[3], d[2]), gather_pair<S>(d[5], d[4]),
                    gather_pair<S>(d[7], d[6]));
}

__device__ __forceinline__ void put4(uint32_t* out, uint4 v) {
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}

// 16 slot-2 codes -> 8 words of bf16 pairs
__device__ __forceinline__ void decode16_slot2(uint32_t u, uint32_t* out) {
  uint32_t d[4];
  spread_slot2(u, d);
  put4(out, pairs4_slot2<0>(d));
  put4(out + 4, pairs4_slot2<1>(d));
}

// 32 binary codes -> 16 words of bf16 pairs
__device__ __forceinline__ void decode32_binary(uint32_t u, uint32_t* out) {
  uint32_t d[8];
  spread_binary(u, d);
  put4(out, pairs4_binary<0>(d));
  put4(out + 4, pairs4_binary<1>(d));
  put4(out + 8, pairs4_binary<2>(d));
  put4(out + 12, pairs4_binary<3>(d));
}

__device__ __forceinline__ uint16_t bf16_of_2t_digit(uint32_t digit) {
  // digit = t + 1 in {0, 1, 2} -> bf16(2t)
  return digit == 0 ? 0xC000u : (digit == 2 ? 0x4000u : 0u);
}

// Two waves per SIMD (at most 256 registers; slot-2), so that two workgroups share a CU and one's
// MFMAs run while the other waits on its loads (measured +40% at 2048 rows over one per CU).
// KS = 2 splits K between two halves of the workgroup (4 waves each, groups taken alternately,
// own LDS tiles); the second half's sums are added to the first's at the end, through LDS. It is
// used when the tiles alone give too few workgroups (KS parts of 4 waves, KS = 2 or 4).
template <int LAYOUT, int BM, int BN, int KS>
__global__ __launch_bounds__(kThreads * KS)
__attribute__((amdgpu_waves_per_eu(LAYOUT == TGS_LAYOUT_BASE3 ? 1 : 2, 8))) void gemm_tile_kernel(
    const uint8_t* __restrict__ codes, int64_t stride, const uint16_t* __restrict__ scales, int n, int k,
    const uint16_t* __restrict__ x, int m, float* __restrict__ y, float* __restrict__ part_sums, int n_tiles,
    int whole, int parts) {
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
  // Workgroups [0, whole) take tiles 0.. whole; workgroup whole + j * parts + p takes part p of
  // tile whole + j. Tile t is column tile t % n_tiles of row tile t / n_tiles.
  const int id = (int)blockIdx.x;
  const int j = id < whole ? 0 : (id - whole) / parts;
  const int tile = id < whole ? id : whole + j;
  const int part = id < whole ? 0 : id - whole - j * parts, nparts = id < whole ? 1 : parts;
  const int n_base = (tile % n_tiles) * BN, m_base = (tile / n_tiles) * BM;
  const int groups = k / 128;
  const int pg0 = part * groups / nparts, pg1 = (part + 1) * groups / nparts;
  // where the sums go: y, or this part's [BM][BN] slice for the tile in the workspace
  const int tail = (int)((gridDim.x - (unsigned)whole) / (unsigned)parts);
  float* __restrict__ slice = part > 0 ? part_sums + ((int64_t)(part - 1) * tail + j) * (BM * BN) : nullptr;

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
  // With 128-row tiles every thread issues the same loads whether or not it needs them (live
  // false, or a thread without a weight row: parked out of range), so that the compiler's wait
  // counts stay exact (see the group loop).
  auto load_stage = [&](int g, bool live) {
#pragma unroll
    for (int u = 0; u < kXUnits; ++u) {
      const int unit = tid + u * kThreads, r = unit >> 3, c16 = (unit & 7) * 16;
      const uint32_t off = ((uint32_t)(m_base + r) * (uint32_t)k + (uint32_t)(g * 128 + c16)) * 2u;
      const uint4 a = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? (int)off : kOobOffset, 0, 0));
      const uint4 b = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? (int)(off + 16u) : kOobOffset, 0, 0));
      xr[u][0] = a.x; xr[u][1] = a.y; xr[u][2] = a.z; xr[u][3] = a.w;
      xr[u][4] = b.x; xr[u][5] = b.y; xr[u][6] = b.z; xr[u][7] = b.w;
    }
    const bool code_live = live && tid < kCodeThreads;
    if (LAYOUT == TGS_LAYOUT_SLOT2 && (BM == 128 || tid < kCodeThreads)) {
      const uint32_t off = (uint32_t)(n_base + (tid >> 1)) * (uint32_t)stride + (uint32_t)(g * 32 + 16 * (tid & 1));
      cr = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, code_live ? (int)off : kOobOffset, 0, kStreamAux));
    }
    if (LAYOUT == TGS_LAYOUT_BINARY && (BM == 128 || tid < kCodeThreads)) {  // 64 codes are 8 bytes
      const uint32_t off = (uint32_t)(n_base + (tid >> 1)) * (uint32_t)stride + (uint32_t)(g * 16 + 8 * (tid & 1));
      const uint2 v = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(code_rsrc, code_live ? (int)off : kOobOffset, 0, kStreamAux));
      cr.x = v.x;
      cr.y = v.y;
    }
  };
  auto store_stage = [&](int g) {
#pragma unroll
    for (int u = 0; u < kXUnits; ++u) {
      const int unit = tid + u * kThreads, r = unit >> 3, c16 = (unit & 7) * 16;
      uint4* dst = reinterpret_cast<uint4*>(xs + r * kPitch + c16);
      dst[0] = make_uint4(xr[u][0], xr[u][1], xr[u][2], xr[u][3]);
      dst[1] = make_uint4(xr[u][4], xr[u][5], xr[u][6], xr[u][7]);
    }
    if (tid < kCodeThreads) {
      const int r = tid >> 1, h = tid & 1;
      // decoded a 16-code word (slot-2) or a 32-code word (binary) at a time, each stored as
      // soon as it is made, so that few decoded words are live at once
      uint4* dst = reinterpret_cast<uint4*>(ws + r * kPitch + 64 * h);
      const uint32_t cw[4] = {cr.x, cr.y, cr.z, cr.w};
      if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t d[4];
          spread_slot2(cw[q], d);
          dst[2 * q] = pairs4_slot2<0>(d);
          dst[2 * q + 1] = pairs4_slot2<1>(d);
        }
      } else if constexpr (LAYOUT == TGS_LAYOUT_BINARY) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t d[8];
          spread_binary(cw[q], d);
          dst[4 * q] = pairs4_binary<0>(d);
          dst[4 * q + 1] = pairs4_binary<1>(d);
          dst[4 * q + 2] = pairs4_binary<2>(d);
          dst[4 * q + 3] = pairs4_binary<3>(d);
        }
      } else {
        uint32_t out[32];
        // base-3: digit by digit from the packed bytes (not on a measured path)
        const int row = n_base + r;
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
          out[e / 2] = lo | (hi << 16);
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) dst[v] = make_uint4(out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]);
      }
    }
  };

  f32x4 acc[kBlkM][kBlkN];
#pragma unroll
  for (int a = 0; a < kBlkM; ++a)
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  // K part kh takes groups pg0 + kh, pg0 + kh + KS, ...; all KS parts run the same number of
  // iterations (the barriers are shared), and a group index past pg1 is loaded harmlessly (in
  // range, or beyond the buffer and read as zero) but not multiplied
  const int iters = (pg1 - pg0 + KS - 1) / KS;
  // (128-row tiles) a group's sums before its scale, and this lane's output columns' scales
  f32x4 gsum[kBlkM][kBlkN];
  uint32_t sraw[kBlkN];
  auto load_scales = [&](int g) {
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) {
      const uint32_t col = (uint32_t)(n_base + wn * kWN + 16 * b + fr);
      sraw[b] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)((col * (uint32_t)groups + (uint32_t)g) * 2u), 0, 0);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int a = 0; a < kBlkM; ++a)
#pragma unroll
      for (int b = 0; b < kBlkN; ++b) gsum[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
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
          gsum[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], gsum[a][b], 0, 0, 0);
    }
  };
  auto scale_add = [&]() {
#pragma unroll
    for (int b = 0; b < kBlkN; ++b) {
      const float sc = 0.5f * f16_to_f32((uint16_t)sraw[b]);  // the weights were decoded as 2t
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(sc, gsum[a][b][r], acc[a][b][r]);
    }
  };
  load_stage(pg0 + kh, true);
  store_stage(pg0 + kh);
  __syncthreads();
  if constexpr (BM == 128) {
    // Each iteration first issues the next stage's loads, then scales the previous group's sums
    // by its scales (loaded an iteration earlier), then loads this group's scales; the MFMAs
    // follow. The scheduling barrier keeps the compiler from sinking the scale loads below the
    // MFMAs, which leaves their latency in front of the next iteration's loads, and every stage
    // load is issued (parked past the end) so that the waits stay exact. (5120 x 17408 at 2048
    // rows: 477 -> 457 us on one box; with 64-row tiles this order was 2-7% slower.)
    bool prev_live = false;
    for (int i = 0; i < iters; ++i) {
      const int g = pg0 + i * KS + kh;
      const bool more = i + 1 < iters;
      load_stage(g + KS, more);
      if (prev_live) scale_add();
      load_scales(g);
      prev_live = KS == 1 || g < pg1;
      __builtin_amdgcn_sched_barrier(0);
      multiply();
      __syncthreads();
      if (more) {
        store_stage(g + KS);
        __syncthreads();
      }
    }
    if (prev_live) scale_add();
  } else {
    for (int i = 0; i < iters; ++i) {
      const int g = pg0 + i * KS + kh;
      const bool more = i + 1 < iters;
      if (more) load_stage(g + KS, true);
      // this lane's output columns: their scales, loaded ahead of the MFMAs
      uint32_t sr[kBlkN];
  #pragma unroll
      for (int b = 0; b < kBlkN; ++b) {
        const uint32_t col = (uint32_t)(n_base + wn * kWN + 16 * b + fr);
        sr[b] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)((col * (uint32_t)groups + (uint32_t)g) * 2u), 0, 0);
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
      if (KS == 1 || g < pg1) {
  #pragma unroll
        for (int b = 0; b < kBlkN; ++b) {
          const float sc = 0.5f * f16_to_f32((uint16_t)sr[b]);  // the weights were decoded as 2t
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
  }
  if constexpr (KS > 1) {
    // the other K parts hand their sums to the first, added in part order (deterministic). A part's
    // sums go to its own tiles, now free: rows of 256 floats, first in its activation tile, then
    // in its weight tile.
    constexpr int kE = kBlkM * kBlkN * 4;
    constexpr int kXsRows = BM * kPitch * 2 / 4 / 256, kWsRows = BN * kPitch * 2 / 4 / 256;
    static_assert(kE <= kXsRows + kWsRows, "the sums fit a part's tiles");
    auto slot = [&](int h, int e) -> float* {
      return e < kXsRows ? reinterpret_cast<float*>(xs_all[h]) + e * 256 + tid
                         : reinterpret_cast<float*>(ws_all[h]) + (e - kXsRows) * 256 + tid;
    };
    if (kh > 0) {
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int b = 0; b < kBlkN; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) *slot(kh, (a * kBlkN + b) * 4 + r) = acc[a][b][r];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int h = 1; h < KS; ++h)
#pragma unroll
      for (int a = 0; a < kBlkM; ++a)
#pragma unroll
        for (int b = 0; b < kBlkN; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[a][b][r] += *slot(h, (a * kBlkN + b) * 4 + r);
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
        if (row < m && col < n) {
          if (part == 0)
            y[(int64_t)row * n + col] = acc[a][b][r];
          else
            slice[(row - m_base) * BN + (col - n_base)] = acc[a][b][r];
        }
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
// per group. Both operands keep k in its natural order (the pair decode above), so the x
// fragments go to the MFMA as loaded. Each group's partial is scaled in fp32; the W per-wave
// results are added through LDS in wave order (deterministic, no atomics).
// Binary codes (BIN) take 4 bytes (32 weights) per lane per group and decode the same way.
// Every workgroup reads all of x for its outputs, so x traffic from L2 falls as FB grows. The
// host picks FB so that a launch is about one workgroup per CU (one round of workgroups) rather
// than shrinking FB to get more workgroups.

template <int TB, int kFB, int kWaves, int kStages, bool BIN, bool SL>
__global__ __launch_bounds__(kWaves * 64) void gemm_skinny_kernel(const uint8_t* __restrict__ codes, int64_t stride,
                                                          const uint16_t* __restrict__ scales, int n, int k,
                                                          const uint16_t* __restrict__ x, int m,
                                                          float* __restrict__ y, float* __restrict__ part_sums) {
  // kFB: 16-output blocks per workgroup; kWaves: K slices (waves) per workgroup; kStages: groups
  // of loads in flight per wave. SL: the scales of the workgroup's rows and K part go to LDS
  // (dynamic, [16 kFB][part groups] fp16) before the weight stream starts; otherwise each wave
  // loads its rows' scales with every group.
  __shared__ float red[kWaves][TB * kFB * 4][64];
  extern __shared__ __attribute__((aligned(16))) uint16_t sc_lds[];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int fr = lane & 15, kq = lane >> 4;  // fragment row and k quarter
  const int n_base = blockIdx.x * 16 * kFB, m_base = blockIdx.y * 16 * TB;
  const int groups = k / 128;
  // this workgroup's part of K: groups [pg0, pg0 + pgn); wave w takes pg0 + w, pg0 + w + W, ...,
  // so that the waves of a workgroup read every row front to back together
  const int part = (int)blockIdx.z, parts = (int)gridDim.z;
  const int pg0 = part * groups / parts, pgn = (part + 1) * groups / parts - pg0;
  float* __restrict__ out = part == 0 ? y : part_sums + (int64_t)(part - 1) * m * n;

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
    uint32_t sc[SL ? 1 : kFB];
    uint32_t xv[TB][16];
    int g;  // its scale group
  };
  // Every workgroup reads the same activations; if all started at the same group, hundreds of CUs
  // would request the same few L2 lines at once. Each workgroup walks its waves' groups in a
  // rotated order instead: a wave's i-th group is its ((i + rot) mod count)-th.
  const int count = (pgn - wave + kWaves - 1) / kWaves;
  const int rot = count > 0 ? (int)(blockIdx.x % (unsigned)count) : 0;
  auto load = [&](Stage& st, int i) {
    const bool live = i < count;
    int j = i + rot;
    if (j >= count) j -= count;
    const int g = pg0 + wave + kWaves * j;
    st.g = g;
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
      if constexpr (!SL)
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
    // Step s multiplies k = 32 kq + 8 s .. + 7 of the group (MFMA k slots 8 kq .. + 7), in natural
    // order on both sides: the lane's x load s as loaded, and weights 8 s .. 8 s + 7 of its codes.
    uint32_t d[kFB][8];  // spread codes (slot-2: one 16-code word at a time; binary: all 32)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 a[TB], b[kFB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        a[tb] = __builtin_bit_cast(
            bf16x8, make_uint4(st.xv[tb][4 * s], st.xv[tb][4 * s + 1], st.xv[tb][4 * s + 2], st.xv[tb][4 * s + 3]));
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) {
        if constexpr (BIN) {
          if (s == 0) spread_binary(st.cw[fb][0], d[fb]);
          const uint4 w = s == 0 ? pairs4_binary<0>(d[fb])
                          : s == 1 ? pairs4_binary<1>(d[fb])
                          : s == 2 ? pairs4_binary<2>(d[fb])
                                   : pairs4_binary<3>(d[fb]);
          b[fb] = __builtin_bit_cast(bf16x8, w);
        } else {
          if ((s & 1) == 0) spread_slot2(st.cw[fb][s >> 1], d[fb]);
          b[fb] = __builtin_bit_cast(bf16x8, (s & 1) ? pairs4_slot2<1>(d[fb]) : pairs4_slot2<0>(d[fb]));
        }
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
      const uint16_t sbits = SL ? sc_lds[(16 * fb + fr) * pgn + (st.g - pg0)] : (uint16_t)st.sc[SL ? 0 : fb];
      const float sc = 0.5f * f16_to_f32(sbits);  // the weights were decoded as 2t
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tb][fb][r] = fmaf(sc, part[tb][fb][r], acc[tb][fb][r]);
    }
  };

  // kStages groups of loads in flight; a stage is reloaded as soon as it has been multiplied
  // (loads past the wave's last group are parked out of range, so every load is unconditional
  // and the compiler's wait counts stay exact)
  // SL: the scales first, so that they do not wait behind the weight stream in the CU's memory
  // pipeline. Scale i of the block [16 kFB rows][pgn groups] is row i / pgn, group pg0 + i % pgn:
  // consecutive threads read consecutive scales of a row, so each load instruction touches one or
  // two cache lines (in the group loop a scale load touches 16). Rows past n read as zero.
  constexpr int kScaleLoads = SL ? kSkinnyScaleLoads : 1;
  uint32_t sv[kScaleLoads];
  const int sc_count = 16 * kFB * pgn;
  if constexpr (SL) {
    // (r, gl) of e = threadIdx.x + 512 i, advanced by 512 = q pgn + rem each step (no division per load)
    const int q = kWaves * 64 / pgn, rem = kWaves * 64 - q * pgn;
    int r = (int)threadIdx.x / pgn, gl = (int)threadIdx.x - r * pgn;
#pragma unroll
    for (int i = 0; i < kScaleLoads; ++i) {
      const int e = (int)threadIdx.x + kWaves * 64 * i;
      const int off = e < sc_count ? (int)(((uint32_t)(n_base + r) * (uint32_t)groups + (uint32_t)(pg0 + gl)) * 2u)
                                   : kOobOffset;
      sv[i] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, off, 0, 0);
      r += q;
      gl += rem;
      if (gl >= pgn) {
        gl -= pgn;
        ++r;
      }
    }
  }
  Stage st[kStages];
#pragma unroll
  for (int u = 0; u < kStages; ++u) load(st[u], u);
  if constexpr (SL) {
#pragma unroll
    for (int i = 0; i < kScaleLoads; ++i) {
      const int e = (int)threadIdx.x + kWaves * 64 * i;
      if (e < sc_count) sc_lds[e] = (uint16_t)sv[i];
    }
    __syncthreads();
  }
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
    if (row < m && col < n) out[(int64_t)row * n + col] = sum;
  }
}

// How one launch (at most a chunk of activation rows) is laid out.
struct GemmPlan {
  int kind;    // 0: skinny, up to 16 rows; 1: skinny, 17..32 rows (two blocks of 16); 2: tiled
  int fb;      // skinny: 16-output blocks per workgroup
  int bm, bn;  // tiled: tile shape
  int ks;      // tiled: K parts inside a workgroup
  int parts;   // K parts across workgroups (skinny: of every output; tiled: of the tail tiles)
  int64_t wgs; // workgroups of one part (skinny), tiles (tiled)
  int64_t whole, tail;  // tiled: tiles taken whole, then tiles split in `parts`
  int64_t n_tiles;      // tiled: column tiles
  bool sl;              // skinny: scales staged in LDS
  int64_t lds;          // ... the dynamic LDS bytes that takes
};

// compute units of the current device (256 on MI355X; 256 if the query fails)
int64_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 256;
  return cus;
}

GemmPlan plan_of(int32_t layout, int64_t n, int64_t k, int64_t m, bool split) {
  GemmPlan p{};
  const int64_t groups = k / 128;
  // parts for a launch of `wgs` tiles: enough to give the CUs about `target` workgroups, each part
  // keeping at least `min_groups` scale groups
  auto parts_for = [&](int64_t wgs, int64_t target, int64_t max_parts, int64_t min_groups) {
    if (!split) return 1;
    int64_t q = (target + wgs - 1) / wgs;
    q = std::min(q, max_parts);
    q = std::min(q, groups / min_groups);
    return (int)std::max<int64_t>(1, q);
  };
  if ((layout == TGS_LAYOUT_SLOT2 || layout == TGS_LAYOUT_BINARY) && m <= 32) {
    // 16 * FB outputs per workgroup of 8 waves (FB in 2..6) and one (m <= 16) or two blocks of 16
    // activation rows, in P parts of K (P in 1..4, each at least kMinPartGroups groups; P = 1
    // without a workspace): the most workgroups that still give no CU a second one, ties to the
    // larger FB. A CU streams this kernel's loads at a rate of its own, so a CU with two
    // workgroups doubles the launch (17408 x 5120: FB = 4, 272 workgroups, 30.9 us against 20.6 us
    // for FB = 5, 218); and every workgroup reads x for its part of K, so x's L2 traffic falls as
    // FB grows. 5120 x 17408: FB = 5 in four parts (256 workgroups) 22.0 us, FB = 6 in four (216)
    // 24.3 us, FB = 2 in three (480) 27.5 us. (Up to 32 rows once took FB = 4/2/1 for at least 512
    // workgroups: 50 / 78 us at 32 rows on these two shapes.)
    p.kind = m <= 16 ? 0 : 1;
    const int64_t cus = device_cus();
    const int64_t max_parts = split ? std::min<int64_t>(4, std::max<int64_t>(1, groups / kMinPartGroups)) : 1;
    // (two row blocks at FB = 6 spill with binary codes: FB <= 5 there)
    const int fb_max = m <= 16 ? 6 : 5;
    p.fb = fb_max, p.parts = 1;
    int64_t best = 0;
    for (int fb = fb_max; fb >= 2; --fb)
      for (int64_t q = 1; q <= max_parts; ++q) {
        const int64_t w = (n + 16 * fb - 1) / (16 * fb) * q;
        if (w <= cus && w > best) best = w, p.fb = fb, p.parts = (int)q;
      }
    p.wgs = (n + 16 * p.fb - 1) / (16 * p.fb);
    // the scales of a workgroup's rows and (largest) part in LDS, when one batch of loads covers them
    const int64_t sc = 16LL * p.fb * ((groups + p.parts - 1) / p.parts);
    p.sl = sc <= 512LL * kSkinnyScaleLoads;
    p.lds = p.sl ? sc * 2 : 0;
    return p;
  }
  // tiles: 128 x 128 for many activation rows, else 64 rows; 64 columns when 128 gives too few
  // tiles. With too few tiles even then, K is split: across workgroups when a workspace is given
  // (each part is a workgroup of its own, so the parts spread over all CUs), else inside the
  // workgroup (two or four parts of 4 waves, added through LDS).
  p.kind = 2;
  const int64_t cus = device_cus();
  p.bm = m > 128 ? 128 : 64;
  const int64_t m_tiles = (m + p.bm - 1) / p.bm;
  p.bn = (n + 127) / 128 * m_tiles >= 512 ? 128 : 64;
  p.n_tiles = (n + p.bn - 1) / p.bn;
  const int64_t tiles = p.n_tiles * m_tiles;
  p.wgs = tiles;
  p.parts = 1;
  p.whole = tiles;
  p.tail = 0;
  if (p.bm == 64 && p.bn == 64) {
    // few small tiles over a long K: every tile in parts
    p.parts = parts_for(tiles, kTileTarget, 4, kMinPartGroups);
    if (p.parts > 1) {
      p.whole = 0, p.tail = tiles;
    } else if (split && tiles > 2 * cus) {
      // otherwise two whole tiles per CU, and the tiles left over in up to 4 parts, so that no CU
      // takes a third whole tile (a CU's throughput is shared by its workgroups: 17408 x 5120 at
      // 128 rows, 544 tiles, 66.5 -> 62.5 us with 512 whole and 32 in four parts)
      const int64_t rem = tiles % (2 * cus);
      const int64_t q = rem > 0 ? std::min<int64_t>({4, 2 * cus / rem, groups / kMinTailGroups}) : 1;
      if (q > 1) p.parts = (int)q, p.whole = tiles - rem, p.tail = rem;
    }
  } else if (p.bm == 128 && p.bn == 128 && split) {
    // 128 x 128 tiles run two workgroups per CU (kTileSlots at a time): whole tiles for the full
    // rounds, and the tiles left over for a last, partly empty round in up to 4 parts that fill it
    const int64_t rem = tiles % kTileSlots;
    const int64_t q = rem > 0 ? std::min<int64_t>({4, kTileSlots / rem, groups / kMinTailGroups}) : 1;
    if (q > 1) p.parts = (int)q, p.whole = tiles - rem, p.tail = rem;
  }
  p.ks = 1;
  if (p.parts == 1) {
    const bool ks2 = tiles < 512 && groups >= 16;
    // four K parts for few 64 x 64 tiles over a long K: every part walks a quarter of the groups,
    // and each group iteration waits out about one HBM latency
    const bool ks4 = ks2 && p.bm == 64 && p.bn == 64 && tiles < 256 && groups >= 64;
    p.ks = ks4 ? 4 : (ks2 && p.bn == 64 ? 2 : 1);  // (128-column tiles come with >= 512 tiles)
  }
  return p;
}

// y[i] += ws[0][i] + ws[1][i] + ... (parts 1, 2, ... of a split launch), added in part order
__global__ __launch_bounds__(256) void gemm_parts_add_kernel(float* __restrict__ y, const float* __restrict__ ws,
                                                             int64_t count, int extra) {
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += step) {
    float v = y[i];
    for (int q = 0; q < extra; ++q) v += ws[q * count + i];
    y[i] = v;
  }
}

// the same for the split tiles of the tiled kernel: y over tail tile j += its slices of parts
// 1, 2, ... ([part - 1][j][BM][BN] in ws), in part order
__global__ __launch_bounds__(256) void gemm_tile_parts_add_kernel(float* __restrict__ y, const float* __restrict__ ws,
                                                                  int m, int n, int n_tiles, int whole, int tail,
                                                                  int extra, int bm, int bn) {
  const int64_t per = (int64_t)bm * bn, count = (int64_t)tail * per;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < count; e += step) {
    const int j = (int)(e / per), l = (int)(e - (int64_t)j * per);
    const int tile = whole + j;
    const int row = (tile / n_tiles) * bm + l / bn, col = (tile % n_tiles) * bn + l % bn;
    if (row >= m || col >= n) continue;
    float v = y[(int64_t)row * n + col];
    for (int q = 0; q < extra; ++q) v += ws[((int64_t)q * tail + j) * per + l];
    y[(int64_t)row * n + col] = v;
  }
}

template <int LAYOUT>
hipError_t launch_layout(const GemmPlan& p, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n,
                         int64_t k, const uint16_t* x, int64_t m, float* y, float* ws, hipStream_t stream) {
  constexpr bool kBin = LAYOUT == TGS_LAYOUT_BINARY;
  const int ni = (int)n, ki = (int)k, mi = (int)m;
  if (p.kind == 0) {
    if constexpr (LAYOUT == TGS_LAYOUT_SLOT2 || kBin) {
      const dim3 grid((unsigned)p.wgs, 1, (unsigned)p.parts);
#define TGS_SKINNY(FB_)                                                                                            \
  if (p.sl)                                                                                                        \
    hipLaunchKernelGGL((gemm_skinny_kernel<1, FB_, 8, 2, kBin, true>), grid, dim3(512), (size_t)p.lds, stream, codes, \
                       stride, scales, ni, ki, x, mi, y, ws);                                                      \
  else                                                                                                             \
    hipLaunchKernelGGL((gemm_skinny_kernel<1, FB_, 8, 2, kBin, false>), grid, dim3(512), 0, stream, codes, stride,   \
                       scales, ni, ki, x, mi, y, ws)
      switch (p.fb) {
        case 2: TGS_SKINNY(2); break;
        case 3: TGS_SKINNY(3); break;
        case 4: TGS_SKINNY(4); break;
        case 5: TGS_SKINNY(5); break;
        default: TGS_SKINNY(6); break;
      }
#undef TGS_SKINNY
    }
  } else if (p.kind == 1) {
    if constexpr (LAYOUT == TGS_LAYOUT_SLOT2 || kBin) {
      const dim3 grid((unsigned)p.wgs, 1, (unsigned)p.parts);
#define TGS_SKINNY2(FB_)                                                                                           \
  if (p.sl)                                                                                                        \
    hipLaunchKernelGGL((gemm_skinny_kernel<2, FB_, 8, 2, kBin, true>), grid, dim3(512), (size_t)p.lds, stream, codes, \
                       stride, scales, ni, ki, x, mi, y, ws);                                                      \
  else                                                                                                             \
    hipLaunchKernelGGL((gemm_skinny_kernel<2, FB_, 8, 2, kBin, false>), grid, dim3(512), 0, stream, codes, stride,   \
                       scales, ni, ki, x, mi, y, ws)
      switch (p.fb) {
        case 2: TGS_SKINNY2(2); break;
        case 3: TGS_SKINNY2(3); break;
        case 4: TGS_SKINNY2(4); break;
        default: TGS_SKINNY2(5); break;
      }
#undef TGS_SKINNY2
    }
  } else {
    const dim3 grid((unsigned)(p.whole + p.tail * p.parts));
#define TGS_TILE(BM_, BN_, KS_)                                                                           \
  hipLaunchKernelGGL((gemm_tile_kernel<LAYOUT, BM_, BN_, KS_>), grid, dim3(kThreads * KS_), 0, stream, codes, \
                     stride, scales, ni, ki, x, mi, y, ws, (int)p.n_tiles, (int)p.whole, p.parts)
    if (p.bm == 128 && p.bn == 128) {
      TGS_TILE(128, 128, 1);
    } else if (p.bm == 128) {
      if (p.ks == 2) TGS_TILE(128, 64, 2); else TGS_TILE(128, 64, 1);
    } else if (p.bn == 128) {
      TGS_TILE(64, 128, 1);
    } else {
      if (p.ks == 4) TGS_TILE(64, 64, 4); else if (p.ks == 2) TGS_TILE(64, 64, 2); else TGS_TILE(64, 64, 1);
    }
#undef TGS_TILE
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.parts == 1) return e;
  if (p.kind == 2) {
    const int64_t count = p.tail * p.bm * p.bn;
    const int64_t blocks = std::min<int64_t>(4096, (count + 255) / 256);
    hipLaunchKernelGGL(gemm_tile_parts_add_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, ws, mi, ni,
                       (int)p.n_tiles, (int)p.whole, (int)p.tail, p.parts - 1, p.bm, p.bn);
  } else {
    const int64_t count = m * n;
    const int64_t blocks = std::min<int64_t>(2048, (count + 255) / 256);
    hipLaunchKernelGGL(gemm_parts_add_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, y, ws, count, p.parts - 1);
  }
  return hipGetLastError();
}

// activation rows per launch: the kernels address x with 32-bit offsets (m * k * 2 < 2^31)
int64_t rows_per_launch(int64_t k) { return std::max<int64_t>(128, (kMaxDeviceCodeBytes / (2 * k)) / 128 * 128); }

}  // namespace

size_t gemm_workspace_bytes(int32_t layout, int64_t n, int64_t k, int64_t m) {
  const int64_t rows = rows_per_launch(k);
  size_t bytes = 0;
  // the full chunks and the last one (the only launch shapes)
  for (const int64_t mr : {std::min(rows, m), m % rows}) {
    if (mr <= 0) continue;
    const GemmPlan p = plan_of(layout, n, k, mr, true);
    const size_t per_part = p.kind == 2 ? (size_t)p.tail * p.bm * p.bn : (size_t)mr * (size_t)n;
    bytes = std::max(bytes, (size_t)(p.parts - 1) * per_part * sizeof(float));
  }
  return bytes;
}

hipError_t gemm_launch(int32_t layout, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n,
                       int64_t k, const uint16_t* x_bf16, int64_t m, float* y, float* ws, hipStream_t stream) {
  const int64_t max_rows = rows_per_launch(k);
  for (int64_t r0 = 0; r0 < m; r0 += max_rows) {
    const int64_t mr = std::min(max_rows, m - r0);
    const uint16_t* xr = x_bf16 + r0 * k;
    float* yr = y + r0 * n;
    const GemmPlan p = plan_of(layout, n, k, mr, ws != nullptr);
    const hipError_t e =
        layout == TGS_LAYOUT_SLOT2   ? launch_layout<TGS_LAYOUT_SLOT2>(p, codes, stride, scales, n, k, xr, mr, yr, ws, stream)
        : layout == TGS_LAYOUT_BASE3 ? launch_layout<TGS_LAYOUT_BASE3>(p, codes, stride, scales, n, k, xr, mr, yr, ws, stream)
                                     : launch_layout<TGS_LAYOUT_BINARY>(p, codes, stride, scales, n, k, xr, mr, yr, ws, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tgs
