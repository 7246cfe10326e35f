// Ternary group-scaled GEMV (M <= 8 activation rows), slot-2 and binary codes, for gfx950.
// (Base-3 codes take the matrix-core kernel in gemv_mfma.hip.)
//
// y[i][n] = sum_k s[n][k/128] * t[n][k] * xr[i][k], weights read once, in packed form.
// The weight definition w = s_g * t with one fp16 scale per 128 weights is the one of
// "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsection
// "Group-scaled ternary format"; xr = R x for rotated-basis weights per the same page,
// subsection "Block-wise Hadamard rotation" (block n = 128 here).
//
// Work split. A workgroup (4 waves) owns a block of rows and walks K in slices. In a slice each
// lane owns one 16-byte chunk of codes (64 weights) at a fixed K
// position and keeps the matching activations in registers while it walks its rows. `S` lanes
// share a row (16, 32 or 64); a wave covers 64/S rows per load instruction, and consecutive lanes
// read consecutive 16-byte chunks of a row, so every load instruction is a fully used,
// contiguous span. Codes and scales are read through buffer resources (reads past the end return
// zero), issued before the activation slice is staged and pipelined in a ring of register sets.
//
// Decode without unpacking (slot-2). Codes q = t + 1 sit in 2-bit slots; a 32-bit word holds 16
// of them, element j in bits 2j..2j+1. dot2 pairs elements (j, j+8): masking the word (or the
// word shifted right by 6 bits) with 3 << p in both 16-bit halves, p in {0, 2, 4, 6, 8}, keeps the
// codes of elements j and j+8 in mantissa bits p..p+1 of the two halves, and OR-ing in the bits of
// 1.0 makes each half the fp16 number 1 + q * 2^(p-10), exactly. One packed fp16 add of
// -(1 + 2^(p-10)) then leaves (q - 1) * 2^(p-10) = t * 2^(p-10) in each half, again exactly (both
// operands and the difference are representable). v_dot2_f32_f16 multiplies the pair by the
// activation pair (x_j, x_{j+8}) and adds into an fp32 accumulator, one accumulator per position p.
// Per 16 weights: one shift, eight AND-ORs, eight packed adds and eight dot2. The accumulators are
// combined with exact power-of-two factors into 2^-20 * sum_k t x.
//
// Every product is t * x itself (times a power of two): a zero code contributes exactly nothing,
// so the partial sums, and with them the rounding, are those of the nonzero terms only; a row with
// one nonzero code gives s * t * x_k exactly.
//
// Binary codes (t in {-1, +1}, one bit b = (t + 1) / 2 per weight; the two-level sibling format of
// "Bonsai 27B and how 1-bit survives" (velog.io), section "What ternary and binary are") use the
// same kernels with 8-byte chunks of 64 weights. A 32-bit word holds 32 weights, element j in bit
// j, and dot2 pairs elements (j, j + 16): masking the word with 0x00010001 << p keeps the bits of
// both in fp16 bit p of the two halves, exactly b * 2^(p-24) (a subnormal for p < 10, the
// smallest normals for p = 10 and 11). Bits 4..11 are used in place and bits 0..3 and 12..15 are
// moved there with one shift each (u << 4, u >> 4), so every position stays at bit 4 or above:
// two shifts, sixteen ANDs and sixteen dot2 per 32 weights, into one accumulator per bit
// position. Then sum_k t x = 2 sum_k b x - sum_k x, the second sum again from the identical
// sequence on an all-ones word.
//
// Shared per-slice work. The activation pairs of a chunk (and, for binary codes, its all-ones-row
// product) depend on the chunk only, not on the wave, so one thread per chunk builds them once per
// workgroup and stores them in LDS, laid out [16-byte granule][chunk] so that the waves' reads are
// conflict-free 16-byte accesses by consecutive lanes.
//
// Scales are applied in fp32 per chunk; partial sums are reduced across the S lanes of a row in
// a fixed order: results are identical run to run.
//
// With the RMSNorm prologue (a runtime flag of the launch; the single-token kernel does not take
// it), each pass of tokens first computes 1 / rms of its rows over all of K (rms_norm.h); the
// staging step then multiplies every activation by gamma and that factor in fp32, before the
// rotation (if any) and the one rounding to fp16.
#include <type_traits>

#include "lane_ops.h"
#include "rms_norm.h"
#include "tgs_internal.h"


namespace tgs {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// waves per workgroup: 4 for every variant (8 waves per workgroup measured slower on the large
// single-token launches, and 4 gives small matrices more workgroups)
template <int ITER>
constexpr int waves_for() {
  return 4;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Activation pair (element e1 in the low half, e2 in the high half) from fp16 words w[e/2].
template <int E1, int E2>
__device__ __forceinline__ uint32_t xpair(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

constexpr int kChunkElems = 64;   // weights per 16-byte chunk
constexpr int kChunkPairDw = 32;  // activation pair words per chunk and token

// ---- building the activation pairs of one chunk ------------------------------------------

// slot-2: p[8d + i] = (x_{16d+i}, x_{16d+i+8}) from the chunk's 64 fp16 activations (32 words)
__device__ __forceinline__ void build_pairs_slot2(const uint32_t* w, uint32_t* p) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    p[8 * d + 0] = xpair<0, 8>(w + 8 * d);
    p[8 * d + 1] = xpair<1, 9>(w + 8 * d);
    p[8 * d + 2] = xpair<2, 10>(w + 8 * d);
    p[8 * d + 3] = xpair<3, 11>(w + 8 * d);
    p[8 * d + 4] = xpair<4, 12>(w + 8 * d);
    p[8 * d + 5] = xpair<5, 13>(w + 8 * d);
    p[8 * d + 6] = xpair<6, 14>(w + 8 * d);
    p[8 * d + 7] = xpair<7, 15>(w + 8 * d);
  }
}

// ---- chunk products -------------------------------------------------------------------------

// The bits of fp16 1.0 in both halves, held in a vector register: with the mask in a scalar
// register, each pair then takes one v_and_or_b32 (with both operands as literal constants the
// compiler splits it into an AND and an OR, since these three-operand forms take no literals)
__device__ __forceinline__ uint32_t one_pair_bits() {
  uint32_t r;
  asm("v_mov_b32 %0, 0x3c003c00" : "=v"(r));
  return r;
}

// Two slot-2 codes as signed fp16 operands: the codes of elements j and j+8 sit in bits p..p+1 of
// the two 16-bit halves of `word`; returns t * 2^(p-10) in each half (see the file comment).
// `one` = one_pair_bits().
template <int P>
__device__ __forceinline__ uint32_t slot2_signed_pair(uint32_t word, uint32_t one) {
  constexpr uint32_t kMask = 0x00030003u << P;
  constexpr uint32_t kNegBias = (0xBC00u | (1u << P)) * 0x00010001u;  // -(1 + 2^(P-10)) in both halves
  const half2_t h = __builtin_bit_cast(half2_t, (word & kMask) | one);
  return __builtin_bit_cast(uint32_t, h + __builtin_bit_cast(half2_t, kNegBias));
}

// slot-2: 2^-20 * sum_k t_k x_k over the 64 weights of a chunk
__device__ __forceinline__ float chunk_dot_slot2(const uint4& cw, const uint32_t* p) {
  const uint32_t one = one_pair_bits();
  float a0 = 0.f, a2 = 0.f, a4 = 0.f, a6 = 0.f, a8 = 0.f;  // a_p: pairs at bit p, terms t x 2^(p-10)
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = words[d], w = u >> 6;
    const uint32_t* q = p + 8 * d;
    a0 = dot2(slot2_signed_pair<0>(u, one), q[0], a0);  // j = 0
    a2 = dot2(slot2_signed_pair<2>(u, one), q[1], a2);  // j = 1
    a4 = dot2(slot2_signed_pair<4>(u, one), q[2], a4);  // j = 2
    a6 = dot2(slot2_signed_pair<6>(u, one), q[3], a6);  // j = 3
    a8 = dot2(slot2_signed_pair<8>(u, one), q[4], a8);  // j = 4
    a4 = dot2(slot2_signed_pair<4>(w, one), q[5], a4);  // j = 5
    a6 = dot2(slot2_signed_pair<6>(w, one), q[6], a6);  // j = 6
    a8 = dot2(slot2_signed_pair<8>(w, one), q[7], a8);  // j = 7
  }
  // sum t x = 2^10 a0 + 2^8 a2 + 2^6 a4 + 2^4 a6 + 2^2 a8 = 4 r
  const float r = fmaf(fmaf(fmaf(fmaf(a0, 4.f, a2), 4.f, a4), 4.f, a6), 4.f, a8);
  return r * 0x1p-18f;
}

// binary: p[16d + i] = (x_{32d+i}, x_{32d+i+16}) from the chunk's 64 fp16 activations (32 words)
template <int I>
__device__ __forceinline__ void pairs_binary_word(const uint32_t* w, uint32_t* p) {
  if constexpr (I < 16) {
    p[I] = xpair<I, I + 16>(w);
    pairs_binary_word<I + 1>(w, p);
  }
}

__device__ __forceinline__ void build_pairs_binary(const uint32_t* w, uint32_t* p) {
  pairs_binary_word<0>(w, p);
  pairs_binary_word<0>(w + 16, p + 16);
}

// binary: 2^-20 * sum_k b_k x_k over the 64 weights of a chunk
__device__ __forceinline__ float chunk_dot_binary(const uint2& cw, const uint32_t* p) {
  float a[8];  // a[j]: pairs whose bits sit at fp16 bit 4 + j, each term b * x * 2^(j - 20)
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = 0.f;
  const uint32_t words[2] = {cw.x, cw.y};
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t u = words[d], lo = u << 4, hi = u >> 4;
    const uint32_t* q = p + 16 * d;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = dot2(u & (0x00100010u << j), q[4 + j], a[j]);  // bits 4..11
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = dot2(lo & (0x00100010u << j), q[j], a[j]);  // bits 0..3
#pragma unroll
    for (int j = 0; j < 4; ++j) a[4 + j] = dot2(hi & (0x01000100u << j), q[12 + j], a[4 + j]);  // bits 12..15
  }
  float r = a[7];
#pragma unroll
  for (int j = 6; j >= 0; --j) r = fmaf(r, 0.5f, a[j]);
  return r;
}

// ---- per-layout chunk operations (BIN: binary codes, else slot-2) --------------------------

template <bool BIN>
using ChunkCodes = typename std::conditional<BIN, uint2, uint4>::type;

template <bool BIN>
constexpr uint32_t chunk_bytes() {
  return BIN ? 8u : 16u;
}

template <bool BIN>
__device__ __forceinline__ ChunkCodes<BIN> load_chunk(__amdgpu_buffer_rsrc_t rsrc, int off) {
  if constexpr (BIN)
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, kStreamAux));
  else
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kStreamAux));
}

template <bool BIN>
__device__ __forceinline__ void build_pairs(const uint32_t* w, uint32_t* p) {
  if constexpr (BIN)
    build_pairs_binary(w, p);
  else
    build_pairs_slot2(w, p);
}

// Binary codes: 2^-20 * sum_k x_k over the chunk, by the same instruction sequence as the rows
// (all-ones codes have b = 1 everywhere). Slot-2 codes decode to signed operands and need none.
template <bool BIN>
__device__ __forceinline__ float chunk_ref(const uint32_t* p) {
  if constexpr (BIN)
    return chunk_dot_binary(make_uint2(0xFFFFFFFFu, 0xFFFFFFFFu), p);
  else
    return 0.f;
}

// 2^-20 * sum_k t_k x_k over the chunk (binary: given its reference sum; every binary weight is
// nonzero, so sum |x| over the chunk is also sum |t x|)
template <bool BIN>
__device__ __forceinline__ float chunk_value(const ChunkCodes<BIN>& cw, const uint32_t* p, float ref) {
  if constexpr (BIN)
    return fmaf(2.f, chunk_dot_binary(cw, p), -ref);
  else
    return chunk_dot_slot2(cw, p);
}

// ---- staging one slice of activations ----------------------------------------------------

// Rotated basis: each wave rotates whole 128-blocks into lds_x (fp16):
// x -> (1/sqrt(128)) H_128 diag(sign) x, H in natural Sylvester order, computed in fp32 with an
// in-register butterfly (lane l holds elements l and l + 64), then rounded once to fp16.
// With gamma set, each activation is first multiplied by gamma[k] and 1 / rms of its token
// (RMSNorm), computed from the per-wave sums of squares norm_part[t * WAVES + w] (LDS).
template <int MT, int WAVES, int BLOCK>
__device__ __forceinline__ void stage_rotated(uint16_t* lds, int len, const uint16_t* x, const int8_t* sign,
                                              int k, int m, int m0, int k_begin, const uint16_t* gamma,
                                              const float* norm_part, float eps) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  auto token_rinv = [&](int t) { return rms_inverse(norm_part, t, WAVES, k, eps); };
  if constexpr (BLOCK == 1024) {
    // 1024-element blocks (k and the slice are multiples of 1024): lane l holds elements
    // 16 l .. 16 l + 15; four butterfly stages inside the lane, six with lane l ^ s
    const int blocks = len / 1024;
    for (int idx = wave; idx < MT * blocks; idx += WAVES) {
      const int t = idx / blocks, b = idx - t * blocks;
      const int kb = k_begin + 1024 * b + 16 * lane;
      float v[16];
      uint4 q[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
      uint4 sg = make_uint4(0, 0, 0, 0);
      if (m0 + t < m && kb < k) {
        const uint4* xb = reinterpret_cast<const uint4*>(x + (int64_t)(m0 + t) * k + kb);
        q[0] = xb[0];
        q[1] = xb[1];
        sg = *reinterpret_cast<const uint4*>(sign + kb);
      }
      const uint32_t xw[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
      const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float xv = f16_to_f32((uint16_t)(xw[i / 2] >> (16 * (i & 1))));
        v[i] = xv * (float)(int8_t)(sw[i / 4] >> (8 * (i & 3)));
      }
      if (gamma) {
        const float r = token_rinv(t);
        uint4 g[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
        if (kb < k) {
          g[0] = reinterpret_cast<const uint4*>(gamma + kb)[0];
          g[1] = reinterpret_cast<const uint4*>(gamma + kb)[1];
        }
        const uint32_t gw[8] = {g[0].x, g[0].y, g[0].z, g[0].w, g[1].x, g[1].y, g[1].z, g[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[2 * i] *= bf16_lo(gw[i]) * r;
          v[2 * i + 1] *= bf16_hi(gw[i]) * r;
        }
      }
#pragma unroll
      for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((i & h) == 0) {
            const float a = v[i], c = v[i + h];
            v[i] = a + c;
            v[i + h] = a - c;
          }
      auto cross = [&](auto s_tag) {
        constexpr int S = decltype(s_tag)::value;
        const float sgn = (lane & S) ? -1.f : 1.f;  // the upper lane of a pair keeps partner - own
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], sgn, xor_lane<S>(v[i], lane));
      };
      cross(std::integral_constant<int, 1>{});
      cross(std::integral_constant<int, 2>{});
      cross(std::integral_constant<int, 4>{});
      cross(std::integral_constant<int, 8>{});
      cross(std::integral_constant<int, 16>{});
      cross(std::integral_constant<int, 32>{});
      uint32_t out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 lo = (_Float16)(v[2 * i] * 0.03125f), hi = (_Float16)(v[2 * i + 1] * 0.03125f);  // 1/sqrt(1024)
        out[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(lds + t * len + 1024 * b + 16 * lane);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    }
    return;
  }
  const int blocks = len / 128;
  for (int idx = wave; idx < MT * blocks; idx += WAVES) {
    const int t = idx / blocks, b = idx - t * blocks;
    const int kb = k_begin + 128 * b;
    float v0 = 0.f, v1 = 0.f;
    if (m0 + t < m && kb < k) {
      const uint16_t* xb = x + (int64_t)(m0 + t) * k + kb;
      v0 = f16_to_f32(xb[lane]) * (float)sign[kb + lane];
      v1 = f16_to_f32(xb[lane + 64]) * (float)sign[kb + lane + 64];
      if (gamma) {
        const float r = token_rinv(t);
        v0 *= __builtin_bit_cast(float, (uint32_t)gamma[kb + lane] << 16) * r;
        v1 *= __builtin_bit_cast(float, (uint32_t)gamma[kb + lane + 64] << 16) * r;
      }
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

// Single-token kernels must keep four waves per SIMD resident (at most 128 VGPRs; three for the
// rotated variant) to have enough loads in flight; the build fails if that ever forces a spill.
template <int MT, int ROT>
constexpr int min_waves_per_eu() {
  return MT == 1 ? (ROT ? 3 : 4) : 1;
}

// ROT: 0 for the plain basis, else the rotation block (128 or 1024). BIN: binary codes.
template <int S, int MT, int ITER, int ROT, bool BIN>
__global__ __launch_bounds__(64 * waves_for<ITER>())
__attribute__((amdgpu_waves_per_eu(min_waves_per_eu<MT, ROT>(), 8))) void gemv_kernel(const GemvArgs args) {
  constexpr int kWaves = waves_for<ITER>();
  constexpr int kThreads = 64 * kWaves;
  constexpr int kIter = ITER;
  constexpr int kRowsPerInstr = 64 / S;
  constexpr int kRowsPerWave = kIter * kRowsPerInstr;
  constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
  constexpr int kSliceElems = S * kChunkElems;
  constexpr int kGran = kChunkPairDw / 4;  // 16-byte granules of pair words per chunk and token

  __shared__ uint4 lds_pairs[MT * kGran * S];                                          // [t][granule][chunk]
  __shared__ float lds_ref[MT * S];                                                    // [t][chunk]
  __shared__ __attribute__((aligned(16))) uint16_t lds_x[ROT ? MT * kSliceElems : 8];  // rotated staging
  __shared__ float lds_norm[MT * kWaves];                                              // RMSNorm partial sums

  int m = 0;
  const GemvJob job = gemv_job_of_block(args, &m);  // uniform; m read with the job
  const int n = job.n, k = job.k;
  const int groups = k / 128;
  const int chunks = k / kChunkElems;
  const int slices = (chunks + S - 1) / S;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int cl = lane % S;     // chunk lane within a row
  const int rslot = lane / S;  // row slot within an instruction
  const int row0 = ((int)blockIdx.x - job.block0) * kRowsPerBlock + wave * kRowsPerWave + rslot;

  constexpr int kBatch = kIter >= 2 ? 2 : 1;
  constexpr int kBatches = kIter / kBatch;
  constexpr int kRing = kBatches >= 4 ? 4 : 3;
  struct Batch {
    ChunkCodes<BIN> cw[kBatch];
    uint32_t s0[kBatch];  // raw fp16 scale bits: converted only when used, so a prefetch never
                          // waits for its own loads
  };
  // Buffer resources: loads past the end of the codes or scales return 0 instead of faulting,
  // so rows past n need no branch and every load is issued unconditionally (which keeps the
  // wait counts exact and the prefetch pipelined). The host limits both arrays to < 2^31 bytes.
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.codes, 0, (int)((int64_t)n * job.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);
  // codes and the group scale of rows b*kBatch .. b*kBatch+kBatch-1 of this lane slot. A lane whose chunk lies past the row (last slice) reads some other in-bounds bytes; its
  // activations are zero and its scales are forced to zero when used, so it adds nothing.
  auto load_batch = [&](Batch& bt, int b, int c, int g0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int row = row0 + (b * kBatch + i) * kRowsPerInstr;
      // unsigned arithmetic: an offset past the buffer simply reads as zero. Rows, row strides
      // and group counts are below 2^24 (checked on the host), so the full-rate 24-bit multiply
      // gives the exact low 32 bits.
      const uint32_t code_off = __umul24((uint32_t)row, (uint32_t)job.stride) + (uint32_t)c * chunk_bytes<BIN>();
      const uint32_t scale_off = (__umul24((uint32_t)row, (uint32_t)groups) + (uint32_t)g0) * 2u;
      bt.cw[i] = load_chunk<BIN>(code_rsrc, (int)code_off);
      bt.s0[i] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, (int)scale_off, 0, 0);
    }
  };

  for (int m0 = 0; m0 < m; m0 += MT) {
    // RMSNorm: the sums of squares of this pass's rows, read by the staging steps below (the
    // previous pass's last reads of lds_norm came before its last barrier)
    if (args.norm) {
      rms_partials<MT>(job.x, k, m, m0, lds_norm, kThreads);
      __syncthreads();
    }
    float part[kIter][MT];
#pragma unroll
    for (int it = 0; it < kIter; ++it)
#pragma unroll
      for (int t = 0; t < MT; ++t) part[it][t] = 0.f;

    for (int ks = 0; ks < slices; ++ks) {
      const int k_begin = ks * kSliceElems;
      const int c = ks * S + cl;  // this lane's chunk
      const bool chunk_ok = c < chunks;
      const int g0 = c / 2;  // two chunks per scale group

      // Codes and scales do not depend on the activations: start loading the first batches of
      // rows before the activation slice is staged, so the two latencies overlap.
      Batch ring[kRing];
#pragma unroll
      for (int b = 0; b < kRing - 1 && b < kBatches; ++b) load_batch(ring[b], b, c, g0);

      // ---- stage: pairs (and binary reference products) of the slice's chunks, once per workgroup
      __syncthreads();  // the previous slice's pairs are no longer read
      if constexpr (ROT) {
        stage_rotated<MT, kWaves, ROT>(lds_x, kSliceElems, job.x, job.signs, k, m, m0, k_begin,
                                       args.norm ? job.gamma : nullptr, lds_norm, args.eps);
        __syncthreads();
      }
      for (int u = tid; u < MT * S; u += kThreads) {
        const int t = u / S, bc = u - t * S;  // token, chunk within the slice
        const int bt0 = (ks * S + bc) * kChunkElems;
        uint32_t w[kChunkElems / 2];
#pragma unroll
        for (int v = 0; v < kChunkElems / 8; ++v) {
          uint4 q = make_uint4(0, 0, 0, 0);
          const int kk = bt0 + 8 * v;  // K and chunk starts are multiples of 8
          if constexpr (ROT) {
            q = *reinterpret_cast<const uint4*>(lds_x + t * kSliceElems + bc * kChunkElems + 8 * v);
          } else {
            if (m0 + t < m && kk < k) {
              q = *reinterpret_cast<const uint4*>(job.x + (int64_t)(m0 + t) * k + kk);
              if (args.norm) {
                const float r = rms_inverse(lds_norm, t, kWaves, k, args.eps);
                const uint4 g = *reinterpret_cast<const uint4*>(job.gamma + kk);
                q = make_uint4(norm_word(q.x, g.x, r), norm_word(q.y, g.y, r), norm_word(q.z, g.z, r),
                               norm_word(q.w, g.w, r));
              }
            }
          }
          w[4 * v + 0] = q.x;
          w[4 * v + 1] = q.y;
          w[4 * v + 2] = q.z;
          w[4 * v + 3] = q.w;
        }
        uint32_t p[kChunkPairDw];
        build_pairs<BIN>(w, p);
        if constexpr (BIN) lds_ref[t * S + bc] = chunk_ref<BIN>(p);
#pragma unroll
        for (int g = 0; g < kGran; ++g)
          lds_pairs[(t * kGran + g) * S + bc] = make_uint4(p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]);
      }
      __syncthreads();

      // ---- this lane's pairs and reference products
      uint32_t xp[MT][kChunkPairDw];
      float ref0[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int g = 0; g < kGran; ++g) {
          const uint4 q = lds_pairs[(t * kGran + g) * S + cl];
          xp[t][4 * g + 0] = q.x;
          xp[t][4 * g + 1] = q.y;
          xp[t][4 * g + 2] = q.z;
          xp[t][4 * g + 3] = q.w;
        }
        ref0[t] = BIN ? lds_ref[t * S + cl] : 0.f;
      }

      // rows in batches; kRing - 1 batches are in flight while one is computed (a ring of register
      // sets, fully unrolled, so no copies)
#pragma unroll
      for (int b = 0; b < kBatches; ++b) {
        if (b + kRing - 1 < kBatches) load_batch(ring[(b + kRing - 1) % kRing], b + kRing - 1, c, g0);
        // keep the scheduler from hoisting later batches' loads: the ring bounds the registers
        __builtin_amdgcn_sched_barrier(0);
        const Batch& cur = ring[b % kRing];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int it = b * kBatch + i;
          const float sc0 = chunk_ok ? f16_to_f32((uint16_t)cur.s0[i]) : 0.f;
#pragma unroll
          for (int t = 0; t < MT; ++t)
            part[it][t] = fmaf(sc0, chunk_value<BIN>(cur.cw[i], xp[t], ref0[t]), part[it][t]);
        }
      }
    }

    // Reduce across the S lanes of each row, in a fixed order. Transposed: at each exchange step
    // a lane keeps half of its values and sends the other half to its partner, so the number of
    // values per lane halves until one is left; the remaining steps are plain butterflies.
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
      // Each exchange step with offset `off` routes odd row slots to the lanes with that bit set,
      // so those bits of the lane index name the row slot it now holds.
      int it_sel = 0, bit = 0;
#pragma unroll
      for (int off = S / 2, cnt = kIter; off >= 1 && cnt > 1; off >>= 1, cnt /= 2, ++bit)
        if (lane & off) it_sel |= 1 << bit;
      const int row = row0 + it_sel * kRowsPerInstr;
      // one writer per row slot: the lane whose butterfly-step bits are zero
      int low_bits = 0;
#pragma unroll
      for (int off = S / 2, cnt = kIter; off >= 1; off >>= 1, cnt = cnt > 1 ? cnt / 2 : 1)
        if (cnt <= 1) low_bits |= off;
      // the chunk products carry a factor 2^-20, undone here (an exact power of two)
      if ((cl & low_bits) == 0 && row < n && m0 + t < m) job.y[(int64_t)(m0 + t) * n + row] = v[0] * 1048576.0f;
    }
  }
}

// ---- single-token kernel: slot-2 codes, one activation row, plain basis --------------------
//
// The decode case that carries most of the traffic. A workgroup owns a block of rows and has one
// wave per K slice of S chunks (64 weights each). Each lane owns one chunk of every row of its
// wave, so the lane that turns its 64 activations into dot2 pairs (and, for binary codes, their
// all-ones-row product) is the only one that ever uses them: they stay in registers, with no LDS staging and
// no barrier before the weight stream. Per wave:
//   1. its activation loads (8 x 16 B per lane) go out first, then the first four 2-row batches
//      of codes and scales, so for small matrices all of a wave's loads are in flight at once;
//   2. the pairs are built while the weights are in flight (vector-memory waits retire in issue
//      order, so this waits only for the activations);
//   3. batches are consumed in groups of four; while a group is consumed, the next group's loads
//      go out into the slots just freed. Every load of a group is issued unconditionally, so the
//      compiler's wait counts are exact;
//   4. each batch is reduced across its lanes right away (lane-half swaps and DPP rotations, no
//      LDS). With one slice the sums go straight to y; otherwise each wave writes its slice sums
//      to LDS and, after one barrier, every row adds its slices in a fixed order.

// Sum of v0 over the S lanes of each row group goes to the group's lanes holding slot 0, and of
// v1 to those holding slot 1. Returns the sum this lane holds and sets `slot` to which one it is.
template <int S>
__device__ __forceinline__ float reduce_pair(float v0, float v1, int lane, int& slot) {
  if constexpr (S == 64) {
    // lanes 0..31 end with v0[l] + v0[l + 32], lanes 32..63 with v1[l - 32] + v1[l]
    swap_halves32(v0, v1);
    float s = v0 + v1;
    // each lane adds the lane 16 away in its 32-lane half
    float t = s;
    swap_rows16(s, t);
    s += t;
    s += dpp<kDppRor8>(s);
    s += dpp<kDppRor4>(s);
    s += dpp<kDppRor2>(s);
    s += dpp<kDppRor1>(s);
    slot = lane >> 5;
    return s;
  } else if constexpr (S == 32) {
    // within each 32-lane half: lanes 0..15 end with v0 of rows 0 and 1, lanes 16..31 with v1
    swap_rows16(v0, v1);
    float s = v0 + v1;
    s += dpp<kDppRor8>(s);
    s += dpp<kDppRor4>(s);
    s += dpp<kDppRor2>(s);
    s += dpp<kDppRor1>(s);
    slot = (lane >> 4) & 1;
    return s;
  } else {
    static_assert(S == 16, "lanes per row must be 16, 32 or 64");
    // within each 16-lane group: lanes 0..7 keep slot 0, lanes 8..15 slot 1
    const bool upper = (lane & 8) != 0;
    const float keep = upper ? v1 : v0, send = upper ? v0 : v1;
    float s = keep + dpp<kDppRor8>(send);
    s += dpp<kDppHalfMirror>(s);  // lane i with lane 7 - i of its 8-lane half
    s += dpp<kDppQuadSwap2>(s);
    s += dpp<kDppQuadSwap1>(s);
    slot = (lane >> 3) & 1;
    return s;
  }
}

// XS (64 lanes per row, at most 4 K slices): the activations are read with coalesced 16-byte
// loads (lane l takes unit 64 v + l of the wave's 8 KB slice) and handed to their lanes through
// the wave's own 8 KB of LDS. Read directly, each of the 8 loads would touch 64 different cache
// lines (lane l wants bytes 128 l ..), which measured 12% slower over the 8B set in layer order.
// Only the wave itself uses its region and one wave's LDS accesses complete in order, so no
// barrier is needed. Unit U is stored at slot U ^ ((U >> 3) & 7) of 16-byte slots: in every group
// of 8 lanes, both the writes and the reads then touch 8 different slots of a 128-byte row.
// W row waves (W = 4, for launches whose rows span one K slice) share the slice's activations:
// the workgroup holds W waves, each with its own rows; they load the 8 KB together (2 loads per
// lane) and meet at one barrier before reading their lanes' bytes, so x is read once per W waves.
// NORM: the RMSNorm prologue. The lane's 64 activations are in its registers, so the sum of
// squares costs a few FMAs per lane; the waves' sums meet in LDS after one barrier (by then every
// wave's first weight loads are in flight), and each lane scales its activations by gamma and
// 1 / rms before building its dot2 pairs. At most 8 waves (K <= 32768) in this variant.
template <int S, int G, bool BIN, bool NORM, bool XS, int W>
__global__ __launch_bounds__(1024)  // (also with NORM, whose workgroups are smaller: 128 registers
                                    // keep 4 waves per SIMD)
void gemv_wave_kernel(const GemvArgs args) {
  static_assert(!XS || S == 64, "activation staging is for 64 lanes per row");
  static_assert(W == 1 || (XS && W == kWaveKernelRowWaves), "row waves share activations through LDS only");
  constexpr int kRowsPerInstr = 64 / S;
  constexpr int kRing = G;  // batches per group: 4, or 1-2 for waves of 2-4 rows
  // dynamic LDS: XS: [slices][512] 16-byte units of activations (normalised, with NORM); then
  // [slices][rows of the workgroup] slice sums, when slices > 1
  extern __shared__ __attribute__((aligned(16))) char lds_dyn[];
  __shared__ float norm_part[NORM ? 8 : 1];  // RMSNorm: each wave's sum of squares

  int R = 0;  // row slots per wave: 2 * G * (number of groups), read with the job
  const GemvJob job = gemv_job_of_block(args, nullptr, &R);  // a copy: the fields stay in scalar registers
  const int n = job.n, k = job.k;
  const int groups = k / 128;
  const int chunks = k / 64;
  const int slices = (chunks + S - 1) / S;  // waves per workgroup: slices * W
  const int batches = R / 2;
  const int rows_wave = R * kRowsPerInstr;
  const int rows_wg = W * rows_wave;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
  const int ks = wave % slices, rw = wave / slices;  // K slice and row wave
  const int cl = lane % S, rslot = lane / S;
  const int c = ks * S + cl;  // this lane's chunk
  const bool lane_live = c < chunks;
  const int block_row0 = ((int)blockIdx.x - job.block0) * rows_wg;
  const int row0 = block_row0 + rw * rows_wave + rslot;
  uint4* lds_x = reinterpret_cast<uint4*>(lds_dyn);
  float* lds_acc = reinterpret_cast<float*>(lds_dyn + (XS ? slices * 8192 : 0));

  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)job.x, 0, k * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.codes, 0, (int)((int64_t)n * job.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);

  // 1. activations of this lane's chunk (reads past K return zero), and their norm weights
  // (XS: this wave's share of the slice's coalesced loads, units 64 v + lane for v = rw, rw + W, ..)
  uint32_t xw[32];
#pragma unroll
  for (int i = 0; i < 8 / W; ++i) {
    const int v = XS ? rw + W * i : i;
    const int xoff = XS ? ks * 8192 + 1024 * v + 16 * lane : c * 128 + 16 * v;
    const uint4 q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xoff, 0, 0));
    xw[4 * i + 0] = q.x;
    xw[4 * i + 1] = q.y;
    xw[4 * i + 2] = q.z;
    xw[4 * i + 3] = q.w;
  }
  uint32_t gw[NORM ? 32 : 1];
  if constexpr (NORM) {
    const __amdgpu_buffer_rsrc_t g_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)job.gamma, 0, k * 2, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
      const int v = XS ? rw + W * i : i;
      const int goff = XS ? ks * 8192 + 1024 * v + 16 * lane : c * 128 + 16 * v;
      const uint4 q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(g_rsrc, goff, 0, 0));
      gw[4 * i + 0] = q.x;
      gw[4 * i + 1] = q.y;
      gw[4 * i + 2] = q.z;
      gw[4 * i + 3] = q.w;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order

  struct Batch {
    ChunkCodes<BIN> cw[2];
    uint32_t s[2];
  };
  // batch b -> rows row0 + (2b + i) * kRowsPerInstr. Rows past the matrix read as zero; a lane
  // past the row's last chunk parks its loads out of range (no traffic, zero data).
  const uint32_t code_col = (uint32_t)c * chunk_bytes<BIN>(), scale_col = (uint32_t)(c >> 1) * 2u;
  auto load_batch = [&](Batch& bt, int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t row = (uint32_t)(row0 + (2 * b + i) * kRowsPerInstr);
      const uint32_t code_off = __umul24(row, (uint32_t)job.stride) + code_col;
      const uint32_t scale_off = __umul24(row, (uint32_t)groups) * 2u + scale_col;
      bt.cw[i] = load_chunk<BIN>(code_rsrc, lane_live ? (int)code_off : kOobOffset);
      bt.s[i] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, lane_live ? (int)scale_off : kOobOffset, 0, 0);
    }
  };
  Batch ring[kRing];
#pragma unroll
  for (int u = 0; u < kRing; ++u) load_batch(ring[u], u);
  __builtin_amdgcn_sched_barrier(0);  // every load is out before anything waits

  if constexpr (XS) {
    if constexpr (NORM) {
      // RMSNorm while staging: every unit of x is held by exactly one thread of the workgroup, so
      // each thread adds the squares of its own units, the waves' sums meet in LDS, and each
      // thread scales its units by gamma / rms before storing them (once per workgroup, not once
      // per wave)
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < 4 * (8 / W); ++i) sq = add_squares(xw[i], sq);
      sq = wave_sum(sq, lane);
      if (lane == 0) norm_part[wave] = sq;
      __syncthreads();
      float total = 0.f;
      for (int q = 0; q < slices * W; ++q) total += norm_part[q];
      const float r = rms_scale(total, k, args.eps);
#pragma unroll
      for (int i = 0; i < 4 * (8 / W); ++i) xw[i] = norm_word(xw[i], gw[i], r);
    }
    uint4* region = lds_x + ks * 512;
#pragma unroll
    for (int i = 0; i < 8 / W; ++i) {
      const int u = 64 * (rw + W * i) + lane;
      region[u ^ ((u >> 3) & 7)] = make_uint4(xw[4 * i], xw[4 * i + 1], xw[4 * i + 2], xw[4 * i + 3]);
    }
    if constexpr (W > 1) __syncthreads();  // the slice's other units come from the other row waves
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = 8 * lane + j;
      const uint4 q = region[u ^ ((u >> 3) & 7)];
      xw[4 * j + 0] = q.x;
      xw[4 * j + 1] = q.y;
      xw[4 * j + 2] = q.z;
      xw[4 * j + 3] = q.w;
    }
  }
  if constexpr (NORM && !XS) {
    // the row's sum of squares: each chunk once (lanes of row slot 0), wave by wave in LDS
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sq = add_squares(xw[i], sq);
    sq = wave_sum(rslot == 0 ? sq : 0.f, lane);
    if (lane == 0) norm_part[ks] = sq;
    __syncthreads();
    float total = 0.f;
    for (int q = 0; q < slices; ++q) total += norm_part[q];
    const float r = rms_scale(total, k, args.eps);
#pragma unroll
    for (int i = 0; i < 32; ++i) xw[i] = norm_word(xw[i], gw[i], r);
  }

  // 2. dot2 pairs (and, for binary codes, the all-ones-row product) of this lane's chunk
  uint32_t xp[32];
  build_pairs<BIN>(xw, xp);
  const float ref = chunk_ref<BIN>(xp);

  constexpr int kSlotLanes = S == 64 ? 32 : (S == 32 ? 16 : 8);
  const bool writer = (lane & (kSlotLanes - 1)) == 0;
  auto consume = [&](const Batch& cur, int b) {
    const float v0 = f16_to_f32((uint16_t)cur.s[0]) * chunk_value<BIN>(cur.cw[0], xp, ref);
    const float v1 = f16_to_f32((uint16_t)cur.s[1]) * chunk_value<BIN>(cur.cw[1], xp, ref);
    int slot;
    const float sum = reduce_pair<S>(v0, v1, lane, slot);
    if (writer) {
      const int local = rw * rows_wave + (2 * b + slot) * kRowsPerInstr + rslot;  // one writer per (row, slice)
      if (slices == 1) {
        const int row = block_row0 + local;
        if (row < n) job.y[row] = sum * 1048576.0f;
      } else {
        lds_acc[ks * rows_wg + local] = sum;
      }
    }
  };
  // 3. groups of G batches; the next group's loads reuse the slots as they are freed
  const int n_groups = batches / kRing;
  for (int g = 0; g + 1 < n_groups; ++g) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      consume(ring[u], kRing * g + u);
      load_batch(ring[u], kRing * (g + 1) + u);
    }
  }
#pragma unroll
  for (int u = 0; u < kRing; ++u) consume(ring[u], kRing * (n_groups - 1) + u);

  // 4. rows spanning several slices: add the slice sums in slice order
  if (slices > 1) {
    __syncthreads();
    for (int r = threadIdx.x; r < rows_wg; r += (int)blockDim.x) {
      float acc = 0.f;
      for (int q = 0; q < slices; ++q) acc += lds_acc[q * rows_wg + r];
      const int row = block_row0 + r;
      if (row < n) job.y[row] = acc * 1048576.0f;
    }
  }
}

template <int S, bool BIN, bool NORM, bool XS, int W>
hipError_t launch_wave_xs(GemvArgs& args, int blocks, int rows_per_wave, int slices, hipStream_t stream) {
  const size_t lds = (slices > 1 ? (size_t)slices * W * rows_per_wave * (64 / S) * sizeof(float) : 0) +
                     (XS ? (size_t)slices * 8192 : 0);
  args.rows_per_wave = rows_per_wave;
  const dim3 block(64 * slices * W);
  if (rows_per_wave >= 8)
    hipLaunchKernelGGL((gemv_wave_kernel<S, 4, BIN, NORM, XS, W>), dim3(blocks), block, lds, stream, args);
  else if (rows_per_wave >= 4)
    hipLaunchKernelGGL((gemv_wave_kernel<S, 2, BIN, NORM, XS, W>), dim3(blocks), block, lds, stream, args);
  else
    hipLaunchKernelGGL((gemv_wave_kernel<S, 1, BIN, NORM, XS, W>), dim3(blocks), block, lds, stream, args);
  return hipGetLastError();
}

// activations staged through LDS (XS) with 64 lanes per row and at most 4 K slices (32 KB), shared
// by row_waves waves per slice
template <int S, bool BIN, bool NORM>
hipError_t launch_wave(GemvArgs& args, int blocks, int rows_per_wave, int slices, int row_waves,
                       hipStream_t stream) {
  if constexpr (S == 64) {
    if (slices == 1 && row_waves == kWaveKernelRowWaves)
      return launch_wave_xs<S, BIN, NORM, true, kWaveKernelRowWaves>(args, blocks, rows_per_wave, slices, stream);
    if (slices <= 4) return launch_wave_xs<S, BIN, NORM, true, 1>(args, blocks, rows_per_wave, slices, stream);
  }
  return launch_wave_xs<S, BIN, NORM, false, 1>(args, blocks, rows_per_wave, slices, stream);
}

template <bool BIN, bool NORM>
hipError_t launch_wave_s(const GemvPlan& plan, GemvArgs& args, int blocks, hipStream_t stream) {
  switch (plan.lanes) {
    case 16: return launch_wave<16, BIN, NORM>(args, blocks, plan.iter, plan.slices, 1, stream);
    case 32: return launch_wave<32, BIN, NORM>(args, blocks, plan.iter, plan.slices, 1, stream);
    default: return launch_wave<64, BIN, NORM>(args, blocks, plan.iter, plan.slices, plan.row_waves, stream);
  }
}

template <int S, int MT, int ITER, int ROT, bool BIN>
hipError_t launch_one(GemvArgs& args, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_kernel<S, MT, ITER, ROT, BIN>), dim3(blocks), dim3(64 * waves_for<ITER>()), 0, stream,
                     args);
  return hipGetLastError();
}

template <int S, int MT, int ITER, bool BIN>
hipError_t launch_block(int rot, GemvArgs& args, int blocks, hipStream_t stream) {
  if (rot == 1024) return launch_one<S, MT, ITER, 1024, BIN>(args, blocks, stream);
  if (rot) return launch_one<S, MT, ITER, 128, BIN>(args, blocks, stream);
  return launch_one<S, MT, ITER, 0, BIN>(args, blocks, stream);
}

// rows per lane slot: 8 for large single-token launches (more work per workgroup), else 4;
// fewer when several tokens share the registers. rot: 0, 128 or 1024 (the rotation block)
template <int S, int MT, bool BIN>
hipError_t launch_rot(int rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  if constexpr (MT == 1) {
    if (iter == 8) return launch_block<S, MT, 8, BIN>(rot, args, blocks, stream);
    return launch_block<S, MT, 4, BIN>(rot, args, blocks, stream);
  } else {
    constexpr int it = MT == 2 ? 2 : 1;
    return launch_block<S, MT, it, BIN>(rot, args, blocks, stream);
  }
}

template <int S, bool BIN>
hipError_t launch_mt(int mt, int rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  switch (mt) {
    case 1: return launch_rot<S, 1, BIN>(rot, iter, args, blocks, stream);
    case 2: return launch_rot<S, 2, BIN>(rot, iter, args, blocks, stream);
    default: return launch_rot<S, 4, BIN>(rot, iter, args, blocks, stream);
  }
}

template <bool BIN>
hipError_t launch_s(int s, int mt, int rot, int iter, GemvArgs& args, int blocks, hipStream_t stream) {
  switch (s) {
    case 16: return launch_mt<16, BIN>(mt, rot, iter, args, blocks, stream);
    case 32: return launch_mt<32, BIN>(mt, rot, iter, args, blocks, stream);
    default: return launch_mt<64, BIN>(mt, rot, iter, args, blocks, stream);
  }
}

}  // namespace

// Tokens per pass (compile-time width of the activation registers); larger m loops over passes.
static int tokens_per_pass(int64_t m) { return m >= 4 ? 4 : (m >= 2 ? 2 : 1); }

GemvPlan gemv_plan(int32_t layout, int64_t k, int64_t m, int32_t rotated, bool norm) {
  GemvPlan p;
  p.layout = layout;
  p.m = (int32_t)m;
  p.rotated = rotated;
  p.norm = norm ? 1 : 0;
  p.row_waves = 1;
  p.slices = 0;
  p.mfma = 0;
  // base-3: decode once, multiply all tokens on the matrix cores
  if (layout == TGS_LAYOUT_BASE3) {
    p.mfma = 1;
    p.stream = 0;
    p.lanes = 64;
    p.iter = 1;
    p.rows_per_block = gemv_b3_mfma_rows((int32_t)m);
    return p;
  }
  // single-token slot-2 in the plain basis: on the matrix cores when K fits
  if (layout == TGS_LAYOUT_SLOT2 && m == 1 && !rotated && gemv_s2_mfma_fits(k)) {
    p.mfma = 2;
    p.stream = 1;
    p.lanes = 64;
    p.iter = 1;
    p.slices = gemv_s2_mfma_waves(k);
    p.rows_per_block = 16;
    return p;
  }
  // slot-2 and binary from here on (both in chunks of 64 weights). The single-token kernel: one wave per K slice of 64 chunks, up to 16
  // waves per workgroup
  const int chunks = (int)(k / kChunkElems);
  // (with the RMSNorm prologue: at most 8 waves per workgroup, K <= 32768)
  p.stream = (m == 1 && !rotated && k <= (norm ? kMaxWaveKernelK / 2 : kMaxWaveKernelK)) ? 1 : 0;
  if (p.stream) {
    // rows shorter than one full slice: 32 or 16 lanes per row, several rows per instruction
    p.lanes = chunks > 32 ? 64 : (chunks > 16 ? 32 : 16);
    p.slices = (chunks + p.lanes - 1) / p.lanes;
    p.iter = 8;
    p.rows_per_block = 8 * (64 / p.lanes);
    return p;
  }
  // lanes per row: the width in {16, 32, 64} that wastes the fewest chunk slots (ties: wider)
  int best = 64, best_waste = 1 << 30;
  for (int s : {64, 32, 16}) {
    int waste = (chunks + s - 1) / s * s - chunks;
    if (waste < best_waste) {
      best = s;
      best_waste = waste;
    }
  }
  p.lanes = best;
  const int mt = tokens_per_pass(m);
  p.iter = mt == 1 ? 4 : (mt == 2 ? 2 : 1);
  p.rows_per_block = 4 * p.iter * (64 / best);  // 4 waves per workgroup at these sizes
  return p;
}

void gemv_plan_set_rows(GemvPlan& p, int64_t total_rows) {
  if (p.mfma) return;
  if (p.stream) {
    // rows per wave: as many (4..64) as still give kWaveKernelTargetWaves waves in all. Small
    // launches get 4 or 8 rows per wave, which puts every load of a wave in flight at once.
    // (Measured on the 8B set: a floor of 4 rows beat 8 by 1.5% in layer order and 3.7% as a set;
    // 2 rows, or twice the target waves, lost 10-22%: every wave re-reads the activations.)
    const int64_t rows_per_instr = 64 / p.lanes;
    int r = 64;
    while (r > 4 && (total_rows + r * rows_per_instr - 1) / (r * rows_per_instr) * p.slices < kWaveKernelTargetWaves)
      r /= 2;
    p.iter = r;
    // row waves sharing the activations (64 lanes per row, one K slice), for launches of
    // up to kWaveKernelShareRows rows. Measured on the 8B set: 4 row waves +9% in layer order;
    // 8 row waves, or sharing in the 3-slice launches, or in launches of a whole set, were slower.
    p.row_waves = 1;
    if (p.lanes == 64 && p.slices == 1 && total_rows <= kWaveKernelShareRows)
      p.row_waves = kWaveKernelRowWaves;
    p.rows_per_block = (int32_t)(r * rows_per_instr * p.row_waves);
    return;
  }
  // single-token slot-2 launches with plenty of rows: twice the rows per workgroup (8 rows per lane
  // slot) while that still leaves >= 2048 workgroups
  if (tokens_per_pass(p.m) != 1) return;
  const int64_t big_rows = (int64_t)waves_for<8>() * 8 * (64 / p.lanes);
  if ((total_rows + big_rows - 1) / big_rows >= 2048) {
    p.iter = 8;
    p.rows_per_block = (int32_t)big_rows;
  }
}

hipError_t gemv_launch(const GemvPlan& plan, GemvArgs& args, int32_t blocks, hipStream_t stream) {
  if (plan.mfma == 2) {
    int64_t max_k = 0;
    for (int i = 0; i < args.count; ++i) max_k = args.job[i].k > max_k ? args.job[i].k : max_k;
    return gemv_s2_mfma_launch(args, blocks, max_k, plan.norm != 0, stream);
  }
  if (plan.mfma)
    return gemv_b3_mfma_launch(args, blocks, plan.m, (int)rotation_block(plan.rotated), plan.norm != 0, stream);
  const bool bin = plan.layout == TGS_LAYOUT_BINARY;
  if (plan.stream) {
    if (plan.norm)
      return bin ? launch_wave_s<true, true>(plan, args, blocks, stream)
                 : launch_wave_s<false, true>(plan, args, blocks, stream);
    return bin ? launch_wave_s<true, false>(plan, args, blocks, stream)
               : launch_wave_s<false, false>(plan, args, blocks, stream);
  }
  const int rot = (int)rotation_block(plan.rotated), mt = tokens_per_pass(plan.m);
  return bin ? launch_s<true>(plan.lanes, mt, rot, plan.iter, args, blocks, stream)
             : launch_s<false>(plan.lanes, mt, rot, plan.iter, args, blocks, stream);
}

}  // namespace tgs
