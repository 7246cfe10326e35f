// Ternary group-scaled GEMV (M <= 8 activation rows) for gfx950.
//
// y[i][n] = sum_k s[n][k/128] * t[n][k] * xr[i][k], weights read once, in packed form.
// The weight definition w = s_g * t with one fp16 scale per 128 weights is the one of
// "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsection
// "Group-scaled ternary format"; xr = R x for rotated-basis weights per the same page,
// subsection "Block-wise Hadamard rotation" (block n = 128 here).
//
// Work split. A workgroup (4 waves) owns a block of rows and walks K in slices. In a slice
// each lane owns one 16-byte chunk of codes (64 slot-2 weights or 80 base-3 trits) at a fixed
// K position and keeps the matching activations in registers while it walks its rows, so x is
// read from LDS once per slice and reused for every row. `S` lanes share a row (16, 32 or 64);
// a wave covers 64/S rows per load instruction, and consecutive lanes read consecutive 16-byte
// chunks of a row, so every load instruction is a fully used, contiguous span.
//
// Decode without unpacking (slot-2). Codes q = t + 1 sit in 2-bit slots; a 32-bit word holds 16
// of them, element j in bits 2j..2j+1. Masking the word (or the word shifted by 4 or 6 bits)
// with 0x00300030, 0x00C000C0 or 0x03000300 keeps the codes of elements j and j+8 in mantissa
// bits 4..9 of the two fp16 halves: with a zero exponent field those halves are the fp16
// subnormals q * 2^(p-24), p in {4, 6, 8}, exactly. v_dot2_f32_f16 multiplies them by the
// activation pair (x_j, x_{j+8}) and adds into an fp32 accumulator, one accumulator per bit
// position p. Three shifted copies cover all 16 codes: two shifts, eight ANDs and eight dot2 per
// 16 weights. (Positions below bit 4 are avoided: measured on gfx950, dot2 with an fp16
// subnormal operand whose value is q * 2^-24 loses about 7 bits, while at bit 4 and above the
// error stays below 4e-7 of the sum.) At the end of a chunk the accumulators are combined with
// exact power-of-two factors into 2^-20 * sum_k q x.
//
// Since t = q - 1, sum_k t x = sum_k q x - sum_k x. The second sum is produced by running the
// identical decode-and-dot sequence on the code word of an all-zero row (every slot q = 1), once
// per slice: a row whose codes are all zero then cancels bit for bit and gives exactly 0.
//
// Base-3. Each byte holds five trits, byte = sum_j (t_j + 1) 3^j. A word is split into two
// 16-bit lanes (bytes 0,2 and bytes 1,3); each digit is peeled off both lanes at once with
// packed 16-bit integer ops (q = v * 171 >> 9 equals v / 3 for v < 256; digit = v - 3q) and
// shifted to bits 4..5 of its lane, where it is again an exact fp16 subnormal fed to dot2. A
// 16-byte chunk (80 trits) can straddle a 128-trit scale group, so each lane keeps two
// accumulators and masks its activation pairs by group once per slice. The same all-zero-row
// trick (byte 121 = five zero trits) supplies sum_k x.
//
// Scales are applied in fp32 per chunk, partial sums are reduced across the S lanes of a row
// with lane shuffles in a fixed order: results are identical run to run.
#include "tgs_internal.h"

namespace tgs {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format, no swizzle)
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Activation pair (element e1 in the low half, e2 in the high half) from fp16 words w[e/2].
template <int E1, int E2>
__device__ __forceinline__ uint32_t xpair(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

template <int LAYOUT>
struct Geo;
template <>
struct Geo<TGS_LAYOUT_SLOT2> {
  static constexpr int kElems = 64;  // weights per 16-byte chunk
  static constexpr int kPairs = 32;  // activation pairs per chunk
  static constexpr int kAccs = 1;    // scale groups a chunk can touch
};
template <>
struct Geo<TGS_LAYOUT_BASE3> {
  static constexpr int kElems = 80;
  static constexpr int kPairs = 40;
  static constexpr int kAccs = 2;
};

__host__ __device__ inline int chunks_per_row(int layout, int k) {
  if (layout == TGS_LAYOUT_SLOT2) return k / 64;
  int used = (k + 4) / 5;
  return (used + 15) / 16;
}

// ---- per-lane activation registers for one slice --------------------------------------

template <int LAYOUT, int MT>
struct XRegs;

template <int MT>
struct XRegs<TGS_LAYOUT_SLOT2, MT> {
  uint32_t p[MT][32];  // pairs: [dword d][position i] -> (x_{16d+i}, x_{16d+i+8})

  __device__ __forceinline__ void load(const uint16_t* lds_chunk, int token_stride, int /*boundary*/) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint4* src = reinterpret_cast<const uint4*>(lds_chunk + t * token_stride);
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // 16 activations per code word, built one word at a time
        const uint4 a = src[2 * d], b = src[2 * d + 1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        p[t][8 * d + 0] = xpair<0, 8>(w);
        p[t][8 * d + 1] = xpair<1, 9>(w);
        p[t][8 * d + 2] = xpair<2, 10>(w);
        p[t][8 * d + 3] = xpair<3, 11>(w);
        p[t][8 * d + 4] = xpair<4, 12>(w);
        p[t][8 * d + 5] = xpair<5, 13>(w);
        p[t][8 * d + 6] = xpair<6, 14>(w);
        p[t][8 * d + 7] = xpair<7, 15>(w);
      }
    }
  }
};

template <int MT>
struct XRegs<TGS_LAYOUT_BASE3, MT> {
  // pairs for each dword d and digit j: e = bytes (0,2) -> trits (20d+j, 20d+10+j),
  // o = bytes (1,3) -> trits (20d+5+j, 20d+15+j); [0] masked to the first scale group of
  // the chunk, [1] to the second.
  uint32_t e[2][MT][20];
  uint32_t o[2][MT][20];

  template <int D, int J>
  __device__ __forceinline__ void set(const uint32_t* w, int t, int boundary) {
    constexpr int e1 = 20 * D + J, e2 = 20 * D + 10 + J, o1 = 20 * D + 5 + J, o2 = 20 * D + 15 + J;
    uint32_t pe = xpair<e1, e2>(w), po = xpair<o1, o2>(w);
    uint32_t me = (e1 < boundary ? 0xFFFFu : 0u) | (e2 < boundary ? 0xFFFF0000u : 0u);
    uint32_t mo = (o1 < boundary ? 0xFFFFu : 0u) | (o2 < boundary ? 0xFFFF0000u : 0u);
    e[0][t][5 * D + J] = pe & me;
    e[1][t][5 * D + J] = pe & ~me;
    o[0][t][5 * D + J] = po & mo;
    o[1][t][5 * D + J] = po & ~mo;
  }

  template <int D>
  __device__ __forceinline__ void set_dword(const uint32_t* w, int t, int boundary) {
    set<D, 0>(w, t, boundary);
    set<D, 1>(w, t, boundary);
    set<D, 2>(w, t, boundary);
    set<D, 3>(w, t, boundary);
    set<D, 4>(w, t, boundary);
  }

  // boundary: index within the chunk of the first trit of the second scale group (>= 80: none)
  __device__ __forceinline__ void load(const uint16_t* lds_chunk, int token_stride, int boundary) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      uint32_t w[40];
      const uint4* src = reinterpret_cast<const uint4*>(lds_chunk + t * token_stride);
#pragma unroll
      for (int v = 0; v < 10; ++v) {
        uint4 q = src[v];
        w[4 * v + 0] = q.x;
        w[4 * v + 1] = q.y;
        w[4 * v + 2] = q.z;
        w[4 * v + 3] = q.w;
      }
      set_dword<0>(w, t, boundary);
      set_dword<1>(w, t, boundary);
      set_dword<2>(w, t, boundary);
      set_dword<3>(w, t, boundary);
    }
  }
};

// ---- per-row chunk products ------------------------------------------------------------

// Slot-2: 2^-20 * sum_k q_k x_k over the 64 weights of the chunk, per token.
template <int MT>
__device__ __forceinline__ void chunk_dot_slot2(const uint4& cw, const XRegs<TGS_LAYOUT_SLOT2, MT>& xr,
                                                float (&out)[MT]) {
  float a2[MT], a3[MT], a4[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) a2[t] = a3[t] = a4[t] = 0.f;
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = words[d], v = u << 4, w = u >> 6;
    // codes of elements (j, j+8) at fp16 mantissa bits 4-5 (a2), 6-7 (a3) or 8-9 (a4)
    const uint32_t c2 = u & 0x00300030u, c3 = u & 0x00C000C0u, c4 = u & 0x03000300u;  // j = 2, 3, 4
    const uint32_t c0 = v & 0x00300030u, c1 = v & 0x00C000C0u;                          // j = 0, 1
    const uint32_t c5 = w & 0x00300030u, c6 = w & 0x00C000C0u, c7 = w & 0x03000300u;  // j = 5, 6, 7
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint32_t* p = &xr.p[t][8 * d];
      a2[t] = dot2(c2, p[2], a2[t]);
      a3[t] = dot2(c3, p[3], a3[t]);
      a4[t] = dot2(c4, p[4], a4[t]);
      a2[t] = dot2(c0, p[0], a2[t]);
      a3[t] = dot2(c1, p[1], a3[t]);
      a2[t] = dot2(c5, p[5], a2[t]);
      a3[t] = dot2(c6, p[6], a3[t]);
      a4[t] = dot2(c7, p[7], a4[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) out[t] = fmaf(fmaf(a4[t], 0.25f, a3[t]), 0.25f, a2[t]);
}

// Base-3: 2^-20 * sum_k (t_k + 1) x_k for the (up to) two scale groups of the chunk, per token.
template <int MT>
__device__ __forceinline__ void chunk_dot_base3(const uint4& cw, const XRegs<TGS_LAYOUT_BASE3, MT>& xr,
                                                float (&out0)[MT], float (&out1)[MT]) {
  float a0[MT], a1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) a0[t] = a1[t] = 0.f;
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u16x2 ve = __builtin_bit_cast(u16x2, words[d] & 0x00FF00FFu);
    u16x2 vo = __builtin_bit_cast(u16x2, (words[d] >> 8) & 0x00FF00FFu);
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      u16x2 de, dd;
      if (j < 4) {
        u16x2 qe = (ve * (u16x2)171) >> (u16x2)9;
        u16x2 qo = (vo * (u16x2)171) >> (u16x2)9;
        de = ve - qe * (u16x2)3;
        dd = vo - qo * (u16x2)3;
        ve = qe;
        vo = qo;
      } else {
        de = ve;
        dd = vo;
      }
      // digit at bits 4..5: the fp16 subnormal digit * 2^-20
      const uint32_t be = __builtin_bit_cast(uint32_t, de << (u16x2)4);
      const uint32_t bo = __builtin_bit_cast(uint32_t, dd << (u16x2)4);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        a0[t] = dot2(be, xr.e[0][t][5 * d + j], a0[t]);
        a1[t] = dot2(be, xr.e[1][t][5 * d + j], a1[t]);
        a0[t] = dot2(bo, xr.o[0][t][5 * d + j], a0[t]);
        a1[t] = dot2(bo, xr.o[1][t][5 * d + j], a1[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    out0[t] = a0[t];
    out1[t] = a1[t];
  }
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// ---- staging one slice of activations into LDS -------------------------------------------

// Plain basis: copy x[m0 + t][k_begin .. k_begin + len) to lds[t][...], zero past K or M.
template <int MT>
__device__ __forceinline__ void stage_plain(uint16_t* lds, int len, const uint16_t* x, int k, int m, int m0,
                                            int k_begin) {
  const int vecs = len / 8;  // 8 halves per 16-byte vector; len and K are multiples of 8
  for (int idx = threadIdx.x; idx < MT * vecs; idx += kThreads) {
    const int t = idx / vecs, v = idx - t * vecs;
    const int kk = k_begin + 8 * v;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (m0 + t < m && kk < k) val = *reinterpret_cast<const uint4*>(x + (int64_t)(m0 + t) * k + kk);
    *reinterpret_cast<uint4*>(lds + t * len + 8 * v) = val;
  }
}

// Rotated basis: each wave rotates whole 128-blocks: x -> (1/sqrt(128)) H_128 diag(sign) x,
// H in natural Sylvester order, computed in fp32 with an in-register butterfly (lane l holds
// elements l and l + 64), then rounded once to fp16.
template <int MT>
__device__ __forceinline__ void stage_rotated(uint16_t* lds, int len, const uint16_t* x, const int8_t* sign,
                                              int k, int m, int m0, int k_begin) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blocks = len / 128;
  for (int idx = wave; idx < MT * blocks; idx += kWaves) {
    const int t = idx / blocks, b = idx - t * blocks;
    const int kb = k_begin + 128 * b;
    float v0 = 0.f, v1 = 0.f;
    if (m0 + t < m && kb < k) {
      const uint16_t* xb = x + (int64_t)(m0 + t) * k + kb;
      v0 = f16_to_f32(xb[lane]) * (float)sign[kb + lane];
      v1 = f16_to_f32(xb[lane + 64]) * (float)sign[kb + lane + 64];
    }
    float a = v0 + v1, c = v0 - v1;
    v0 = a;
    v1 = c;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      float p0 = __shfl_xor(v0, s), p1 = __shfl_xor(v1, s);
      const bool upper = (lane & s) != 0;
      v0 = upper ? (p0 - v0) : (v0 + p0);
      v1 = upper ? (p1 - v1) : (v1 + p1);
    }
    const float norm = 0.08838834764831845f;  // 1/sqrt(128)
    _Float16 h0 = (_Float16)(v0 * norm), h1 = (_Float16)(v1 * norm);
    lds[t * len + 128 * b + lane] = __builtin_bit_cast(uint16_t, h0);
    lds[t * len + 128 * b + lane + 64] = __builtin_bit_cast(uint16_t, h1);
  }
}

// ---- the kernel ----------------------------------------------------------------------

// Single-token slot-2 kernels must keep four waves per SIMD resident (at most 128 VGPRs; three for
// the rotated variant) to have enough loads in flight; the build fails if that ever forces a spill.
template <int LAYOUT, int MT, bool ROT>
constexpr int min_waves_per_eu() {
  return (LAYOUT == TGS_LAYOUT_SLOT2 && MT == 1) ? (ROT ? 3 : 4) : (MT == 1 ? 2 : 1);
}

template <int LAYOUT, int S, int MT, int ITER, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves_per_eu<LAYOUT, MT, ROT>(), 8)))
void gemv_kernel(const GemvArgs args) {
  using G = Geo<LAYOUT>;
  constexpr int kIter = ITER;
  constexpr int kRowsPerInstr = 64 / S;
  constexpr int kRowsPerWave = kIter * kRowsPerInstr;
  constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
  constexpr int kSliceElems = S * G::kElems;

  __shared__ __attribute__((aligned(16))) uint16_t xs[MT * kSliceElems];

  // find this workgroup's job (uniform; the table lives in the kernel arguments)
  int j = 0;
  while (j + 1 < args.count && (int)blockIdx.x >= args.job[j + 1].block0) ++j;
  const GemvJob& job = args.job[j];
  const int n = job.n, k = job.k, m = args.m;
  const int groups = k / 128;
  const int chunks = chunks_per_row(LAYOUT, k);
  const int slices = (chunks + S - 1) / S;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = lane % S;      // chunk lane within a row
  const int rslot = lane / S;   // row slot within an instruction
  const int row0 = ((int)blockIdx.x - job.block0) * kRowsPerBlock + wave * kRowsPerWave + rslot;

  constexpr int kBatch = kIter >= 2 ? 2 : 1;
  constexpr int kBatches = kIter / kBatch;
  constexpr int kRing = kBatches >= 4 ? 4 : 3;
  struct Batch {
    uint4 cw[kBatch];
    uint32_t s0[kBatch], s1[kBatch];  // raw fp16 scale bits: converted only when used, so a
                                      // prefetch never waits for its own loads
  };
  // Buffer resources: loads past the end of the codes or scales return 0 instead of faulting,
  // so rows past n need no branch and every load is issued unconditionally (which keeps the
  // wait counts exact and the prefetch pipelined). The host limits both arrays to < 2^31 bytes.
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.codes, 0, (int)((int64_t)n * job.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);
  // codes and the (up to two) group scales of rows b*kBatch .. b*kBatch+kBatch-1 of this lane
  // slot. A lane whose chunk lies past the row (last slice) reads some other in-bounds bytes; its
  // activations are zero and its scales are forced to zero when used, so it adds nothing.
  auto load_batch = [&](Batch& bt, int b, int c, bool chunk_ok, int g0, bool has_g1) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int row = row0 + (b * kBatch + i) * kRowsPerInstr;
      // unsigned arithmetic: an offset past the buffer simply reads as zero
      const uint32_t code_off = (uint32_t)row * (uint32_t)job.stride + (uint32_t)c * 16u;
      const uint32_t scale_off = ((uint32_t)row * (uint32_t)groups + (uint32_t)g0) * 2u;
      bt.cw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(code_rsrc, (int)code_off, 0, 0));
      bt.s0[i] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)scale_off, 0, 0);
      bt.s1[i] = 0;
      if (LAYOUT == TGS_LAYOUT_BASE3)
        bt.s1[i] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)(scale_off + 2u), 0, 0);
    }
  };

  for (int m0 = 0; m0 < m; m0 += MT) {
    float part[kIter][MT];
#pragma unroll
    for (int it = 0; it < kIter; ++it)
#pragma unroll
      for (int t = 0; t < MT; ++t) part[it][t] = 0.f;

    for (int ks = 0; ks < slices; ++ks) {
      const int k_begin = ks * kSliceElems;
      const int c = ks * S + cl;  // this lane's chunk
      const bool chunk_ok = c < chunks;
      // first trit of the second scale group, relative to the chunk (base-3 only)
      const int t0 = c * G::kElems;
      const int boundary = (LAYOUT == TGS_LAYOUT_BASE3) ? ((t0 / 128 + 1) * 128 - t0) : 1 << 20;
      const int g0 = (LAYOUT == TGS_LAYOUT_SLOT2) ? c / 2 : t0 / 128;
      const bool has_g1 = LAYOUT == TGS_LAYOUT_BASE3 && boundary < G::kElems && g0 + 1 < groups;

      // Codes and scales do not depend on the activations: start loading the first batches of
      // rows before the activation slice is staged, so the two latencies overlap.
      Batch ring[kRing];
#pragma unroll
      for (int b = 0; b < kRing - 1 && b < kBatches; ++b) load_batch(ring[b], b, c, chunk_ok, g0, has_g1);

      __syncthreads();  // the previous slice's activations are no longer read
      if constexpr (ROT)
        stage_rotated<MT>(xs, kSliceElems, job.x, job.signs, k, m, m0, k_begin);
      else
        stage_plain<MT>(xs, kSliceElems, job.x, k, m, m0, k_begin);
      __syncthreads();

      XRegs<LAYOUT, MT> xr;
      xr.load(xs + cl * G::kElems, kSliceElems, boundary);
      // chunk products of an all-zero row: the same decode-and-dot on its code word
      float ref0[MT], ref1[MT];
      if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
        chunk_dot_slot2<MT>(make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u), xr, ref0);
      } else {
        chunk_dot_base3<MT>(make_uint4(0x79797979u, 0x79797979u, 0x79797979u, 0x79797979u), xr, ref0, ref1);
      }

      // rows in batches; kRing - 1 batches are in flight while one is computed (a ring of register
      // sets, fully unrolled, so no copies)
#pragma unroll
      for (int b = 0; b < kBatches; ++b) {
        if (b + kRing - 1 < kBatches) load_batch(ring[(b + kRing - 1) % kRing], b + kRing - 1, c, chunk_ok, g0, has_g1);
        // keep the scheduler from hoisting later batches' loads: the ring bounds the registers
        __builtin_amdgcn_sched_barrier(0);
        const Batch& cur = ring[b % kRing];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int it = b * kBatch + i;
          const float sc0 = chunk_ok ? f16_to_f32((uint16_t)cur.s0[i]) : 0.f;
          if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
            float qx[MT];
            chunk_dot_slot2<MT>(cur.cw[i], xr, qx);
#pragma unroll
            for (int t = 0; t < MT; ++t) part[it][t] = fmaf(sc0, (qx[t] - ref0[t]) * 1048576.0f, part[it][t]);
          } else {
            const float sc1 = (chunk_ok && has_g1) ? f16_to_f32((uint16_t)cur.s1[i]) : 0.f;
            float q0[MT], q1[MT];
            chunk_dot_base3<MT>(cur.cw[i], xr, q0, q1);
#pragma unroll
            for (int t = 0; t < MT; ++t)
              part[it][t] = fmaf(sc1, (q1[t] - ref1[t]) * 1048576.0f,
                                 fmaf(sc0, (q0[t] - ref0[t]) * 1048576.0f, part[it][t]));
          }
        }
      }
    }

    // Reduce across the S lanes of each row, in a fixed order. Transposed: at each exchange step
    // a lane keeps half of its values and sends the other half to its partner, so the number of
    // values per lane halves until one is left; the remaining steps are plain butterflies. The
    // sum of row slot `it` ends in the lanes whose bits (within the S-lane group) match `it`.
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float v[kIter];
#pragma unroll
      for (int it = 0; it < kIter; ++it) v[it] = part[it][t];
      int count = kIter;
#pragma unroll
      for (int off = S / 2; off >= 1; off >>= 1) {
        const bool upper = (lane & off) != 0;
        if (count > 1) {
#pragma unroll
          for (int i = 0; i < kIter / 2; ++i) {
            if (2 * i + 1 < count) {
              const float keep = upper ? v[2 * i + 1] : v[2 * i];
              const float send = upper ? v[2 * i] : v[2 * i + 1];
              v[i] = keep + __shfl_xor(send, off);
            }
          }
          count /= 2;
        } else {
          v[0] += __shfl_xor(v[0], off);
        }
      }
      // after the exchanges, lane bit pattern (within its S-lane group) selects the row slot:
      // each exchange step with offset `off` (taken while count > 1) routes odd slots to the
      // lanes with that bit set
      int it_sel = 0, bit = 0;
#pragma unroll
      for (int off = S / 2, cnt = kIter; off >= 1 && cnt > 1; off >>= 1, cnt /= 2, ++bit)
        if (lane & off) it_sel |= 1 << bit;
      const int row = row0 + it_sel * kRowsPerInstr;
      // one lane per (row slot): the lowest lane whose exchange bits equal it_sel
      int low_bits = 0;
#pragma unroll
      for (int off = S / 2, cnt = kIter; off >= 1; off >>= 1, cnt = cnt > 1 ? cnt / 2 : 1)
        if (cnt <= 1) low_bits |= off;
      if ((cl & low_bits) == 0 && row < n && m0 + t < m) job.y[(int64_t)(m0 + t) * n + row] = v[0];
    }
  }
}

template <int LAYOUT, int S, int MT, int ITER, bool ROT>
hipError_t launch_one(GemvArgs& args, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_kernel<LAYOUT, S, MT, ITER, ROT>), dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

// rows per lane slot: 8 for large single-token launches (more work per workgroup), else 4;
// fewer when several tokens share the registers
template <int LAYOUT, int S, int MT>
hipError_t launch_rot(bool rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  if constexpr (MT == 1 && LAYOUT == TGS_LAYOUT_SLOT2) {
    if (iter == 8)
      return rot ? launch_one<LAYOUT, S, MT, 8, true>(args, blocks, stream)
                 : launch_one<LAYOUT, S, MT, 8, false>(args, blocks, stream);
    return rot ? launch_one<LAYOUT, S, MT, 4, true>(args, blocks, stream)
               : launch_one<LAYOUT, S, MT, 4, false>(args, blocks, stream);
  } else {
    constexpr int it = MT == 1 ? 4 : (MT == 2 ? 2 : 1);
    return rot ? launch_one<LAYOUT, S, MT, it, true>(args, blocks, stream)
               : launch_one<LAYOUT, S, MT, it, false>(args, blocks, stream);
  }
}

template <int LAYOUT, int S>
hipError_t launch_mt(int mt, bool rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
    switch (mt) {
      case 1: return launch_rot<LAYOUT, S, 1>(rot, iter, args, blocks, stream);
      case 2: return launch_rot<LAYOUT, S, 2>(rot, iter, args, blocks, stream);
      default: return launch_rot<LAYOUT, S, 4>(rot, iter, args, blocks, stream);
    }
  } else {
    return launch_rot<LAYOUT, S, 1>(rot, iter, args, blocks, stream);
  }
}

template <int LAYOUT>
hipError_t launch_s(int s, int mt, bool rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  switch (s) {
    case 16: return launch_mt<LAYOUT, 16>(mt, rot, iter, args, blocks, stream);
    case 32: return launch_mt<LAYOUT, 32>(mt, rot, iter, args, blocks, stream);
    default: return launch_mt<LAYOUT, 64>(mt, rot, iter, args, blocks, stream);
  }
}

}  // namespace

// Tokens per pass (compile-time width of the activation registers); larger m loops over passes.
static int tokens_per_pass(int32_t layout, int64_t m) {
  if (layout == TGS_LAYOUT_BASE3) return 1;
  return m >= 4 ? 4 : (m >= 2 ? 2 : 1);
}

GemvPlan gemv_plan(int32_t layout, int64_t k, int64_t m, int32_t rotated) {
  GemvPlan p;
  p.layout = layout;
  p.m = (int32_t)m;
  p.rotated = rotated;
  // lanes per row: the width in {16, 32, 64} that wastes the fewest chunk slots (ties: wider)
  const int chunks = chunks_per_row(layout, (int)k);
  int best = 64, best_waste = 1 << 30;
  for (int s : {64, 32, 16}) {
    int waste = (chunks + s - 1) / s * s - chunks;
    if (waste < best_waste) {
      best = s;
      best_waste = waste;
    }
  }
  p.lanes = best;
  const int mt = tokens_per_pass(layout, m);
  p.iter = mt == 1 ? 4 : (mt == 2 ? 2 : 1);
  p.rows_per_block = kWaves * p.iter * (64 / best);
  return p;
}

void gemv_plan_set_rows(GemvPlan& p, int64_t total_rows) {
  // single-token slot-2 launches with plenty of rows: 2x more rows per workgroup, still >= 2048
  // workgroups
  if (p.layout != TGS_LAYOUT_SLOT2 || tokens_per_pass(p.layout, p.m) != 1) return;
  const int64_t big_rows = (int64_t)kWaves * 8 * (64 / p.lanes);
  if ((total_rows + big_rows - 1) / big_rows >= 2048) {
    p.iter = 8;
    p.rows_per_block = (int32_t)big_rows;
  }
}

hipError_t gemv_launch(const GemvPlan& plan, GemvArgs& args, int32_t blocks, hipStream_t stream) {
  const int mt = tokens_per_pass(plan.layout, plan.m);
  const bool rot = plan.rotated != 0;
  if (plan.layout == TGS_LAYOUT_SLOT2)
    return launch_s<TGS_LAYOUT_SLOT2>(plan.lanes, mt, rot, plan.iter, args, blocks, stream);
  return launch_s<TGS_LAYOUT_BASE3>(plan.lanes, mt, rot, plan.iter, args, blocks, stream);
}

}  // namespace tgs
