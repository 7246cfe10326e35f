// Base-3 GEMV (1..8 tokens) on the matrix cores.
//
// y[i][j] = sum_k s[j][k/128] * t[j][k] * xr[i][k], with xr = x or, for weights stored in the
// rotated basis, xr = R x, R = blockdiag((1/sqrt(n)) H_n S) with n = 128 or 1024 ("Ternary Bonsai 2
// 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr), subsections "Group-scaled ternary format"
// and "Block-wise Hadamard rotation"). A dot2 decode would repeat the whole base-3 digit extraction
// for every token; here the codes are decoded once and v_mfma_f32_16x16x32_f16 multiplies them by
// all tokens at once (tokens are the 16 rows of the A operand, padded with zeros). Even for one token this measured faster than the dot2 decode: the
// matrix cores take the multiply-adds and the decode is a few packed integer ops per digit.
//
// Work split. A workgroup of 8 waves owns 16 * FB output rows and splits the scale
// groups of K across its waves; each wave walks its groups one at a time:
//   - Codes. A group's 128 trits start in byte B0 = floor(128 g / 5) at digit off0 = 128 g - 5 B0
//     and end within the 32 bytes from B0. Lane (r, q) of a row block (r = lane % 16, q = lane / 16)
//     reads bytes B0 + 8q .. B0 + 8q + 7 of row r (three aligned dwords and a funnel shift) and
//     peels their digits with packed 16-bit integer ops (q = v * 171 >> 9 equals v / 3 for
//     v < 256; digit = v - 3q), five per byte. MFMA step j (0..4) takes
//     digit j of all eight bytes, paired (byte 0, byte 2), (1, 3), (4, 6), (5, 7). A digit d in
//     the low byte of a 16-bit half becomes the fp16 weight t = d - 1 (-1.0, 0 or +1.0) with one
//     byte lookup (v_perm): the digit, shifted into the high byte of the selector, picks the high
//     byte of the fp16 value from the table {0xBC, 0x00, 0x3C}, and the low byte is a constant
//     zero. So every product is t * x exactly, and a zero weight adds nothing: the partial sums
//     and their rounding are those of the nonzero terms, and a row with a single nonzero weight
//     gives s * t * x exactly.
//   - Activations. The wave writes the group's activations (rotated when the weights are: sign
//     flip, the natural-order Sylvester butterfly over the 128-block, 1/sqrt(128), one rounding to
//     fp16) into a private LDS tile laid out [q][j][8] in exactly the order of the weight operand,
//     so each MFMA step reads its A fragment with one 16-byte load. The 32 slots of the 160-trit
//     window that lie outside the group hold zeros: the trits there (neighbouring groups, or
//     bytes past the row) multiply zero, and every MFMA step stays within one scale group.
//   - 1024-element rotation blocks span eight groups, so they are rotated once per workgroup (16
//     elements per lane: 4 butterfly stages in the lane, 6 across lanes). When the MT rotated rows
//     fit in 48 KB of LDS (PRE), the workgroup rotates all of them before its weight stream, and the
//     waves then walk contiguous group slices as in the plain basis. Otherwise wave w < MT rotates
//     token w's block b + 1 into one half of a double-buffered LDS array while every wave
//     multiplies its group 8 b + w of block b from the other half, with one barrier per block.
//   - Only the MT live rows of each A tile are kept in LDS; lanes of the padding rows MT..15 read
//     their fragments from one shared zero row, so every lane issues the same unconditional read.
//   - RMSNorm prologue (NORM): the workgroup first computes 1 / rms of each token over all of K
//     (rms_norm.h; its loads are issued before the first weights are needed), and every
//     activation is multiplied by gamma[k] and that factor in fp32 before the sign flip, the
//     butterfly and the one rounding to fp16.
//   - Each group's 16 x 16 partial is scaled by its fp16 scale in fp32 and added to the running
//     sum; at the end the 8 waves' sums are added through LDS in wave order (deterministic).
#include <type_traits>

#include "lane_ops.h"
#include "rms_norm.h"
#include "tgs_internal.h"

namespace tgs {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;       // K slices per workgroup
// 16-row blocks per workgroup, measured best: 1 for a single token (more workgroups for the small
// launches of a decode step), 2 for several tokens (the 27B rotated set with 8 tokens: 618 GB/s,
// against 477 with 1 and 490 with 4)
constexpr int kMfmaFB1 = 1;
constexpr int kMfmaFBMulti = 2;
constexpr int kRowPitch = 168;  // halves per token row of the activation tile: 160 slots + 8 (bank spread)

// window position rel (0..159) of a group's trit -> its slot in the [q][j][8] tile
__device__ __forceinline__ int tile_slot(int rel) {
  const int b = (rel * 205) >> 10;  // rel / 5 for rel < 160
  const int j = rel - 5 * b;
  const int q = b >> 3, bl = b & 7;
  const int pos = (bl & 4) | ((bl & 1) << 1) | ((bl >> 1) & 1);  // byte order 0,2,1,3,4,6,5,7
  return (q * 5 + j) * 8 + pos;
}

// Weight operand of two digits: d (0..2) in the low byte of each 16-bit half -> fp16 t = d - 1 in
// each half. The selector holds the digits in bytes 1 and 3 and 0x0C (constant zero) in bytes 0
// and 2; the table's bytes 0..2 are the high bytes of fp16 -1.0, 0 and +1.0.
__device__ __forceinline__ uint32_t digits_to_weights(u16x2 d) {
  constexpr uint32_t kTable = 0x003C00BCu;
  return __builtin_amdgcn_perm(0u, kTable, (__builtin_bit_cast(uint32_t, d) << 8) | 0x000C000Cu);
}

__device__ __forceinline__ u16x2 peel(u16x2& v) {  // next base-3 digit of both halves
  const u16x2 q = (v * (u16x2)171) >> (u16x2)9;
  const u16x2 d = v - q * (u16x2)3;
  v = q;
  return d;
}

// Element of the group that entry e = kE p + i of a lane's slot list holds after the rotation:
// e itself, except in 128-element blocks for one token and for eight on the matrix cores (MROT).
// One token: the two lane-half butterfly stages pair the lane's own two elements (a swap of one
// register's half with the other's, then a sum and a difference), which leaves element bit 0 on
// lane bit 4, bits 1..4 on lane bits 0..3, bit 5 on lane bit 5 and bit 6 on the register.
// Eight tokens (MROT): entry j = 8 h + 4 i + r of p = cb + 2 eq is element 4 eq + r of 16-element
// chunk 4 h + 2 i + cb (the layout the rotation's products leave, below).
template <int MT, int ROT, bool MROT>
__host__ __device__ constexpr int rotated_element(int e) {
  if (MROT) {
    const int p = e >> 4, j = e & 15;
    return 64 * (j >> 3) + 32 * ((j >> 2) & 1) + 16 * (p & 1) + 4 * (p >> 1) + (j & 3);
  }
  if (MT != 1 || ROT != 128) return e;
  const int p = e >> 1, reg = e & 1;
  return ((p >> 4) & 1) | ((p & 15) << 1) | (((p >> 5) & 1) << 5) | (reg << 6);
}

// Rotation of eight tokens' 128-element groups on the matrix cores. Sylvester's H_128 is
// H_8 (x) H_16 over the 16-element chunks c of the group: y[16 c' + e] = sum_c H_8[c'][c]
// (H_16 x_c)[e]. One v_mfma_f32_16x16x32_f16 takes H_16 on both halves of its A operand (rows e)
// and, as the B operand's 16 columns, eight tokens times two chunk parities cb: column
// tok + 8 cb holds chunk pp = 2 i + cb in its k rows 0..15 and chunk pp + 4 in rows 16..31. With
// [H_16 | H_16] it yields H_16 (x_pp + x_pp+4), with [H_16 | -H_16] H_16 (x_pp - x_pp+4): the
// product and the H_8 stage on chunk bit 2. The stage on chunk bit 1 (i) is a sum and a difference
// in the lane, the one on bit 0 (cb, lane bit 3) one DPP exchange with the lane 8 apart. Products
// of +-1 and fp16 values are exact and the sums are fp32, as in the butterfly; the one rounding to
// fp16 follows 1/sqrt(128).
// v[j] += v[j] of lane (lane ^ 8) * sp for the 16 values, each one v_fmac_f32 reading the partner
// through DPP (row_ror:8 is lane ^ 8 within a 16-lane row). The compiler emits a separate DPP move
// for this form, so it is written out; the s_nop gives the two wait states a DPP read needs after
// a VALU write of its source (every later source was written before the first), and each
// instruction reads its partner's value before any lane's result is written.
__device__ __forceinline__ void fmac_partner8x16(float (&v)[16], float sp) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %8, %8, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %9, %9, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %10, %10, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %11, %11, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %12, %12, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %13, %13, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %14, %14, %16 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %15, %15, %16 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
        "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15])
      : "v"(sp));
}

// A operand of lane (e = lane % 16, k rows 8 (lane / 16) ..): H_16[e][k mod 16], negated in rows
// k >= 16 when `minus`
__device__ __forceinline__ half8 hadamard16_operand(int lane, bool minus) {
  const int e = lane & 15, k0 = 8 * ((lane >> 4) & 1);
  const bool neg = minus && (lane >> 5);
  half8 h;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bool odd = (__builtin_popcount((unsigned)(e & (k0 + t))) & 1) != 0;
    h[t] = (odd != neg) ? (_Float16)-1.f : (_Float16)1.f;
  }
  return h;
}

// pipeline depth of the group loop (plain and 128-block bases): stages of loads per wave. Two
// measured best: on the 8B base-3 set with one token, 3, 4 and 6 stages ran at 838, 815 and
// 748 GB/s in layer order against 860 (1362, 1289, 1127 against 1429 as a set), and 3 stages with
// 8 tokens at 505 against 602 GB/s on the 27B rotated set.
constexpr int kStagesOneToken = 2, kStagesTokens = 2;

template <int MT, int kFB, int ROT, bool NORM, bool PRE>
__global__ __launch_bounds__(kWaves * 64) void gemv_b3_mfma_kernel(const GemvArgs args) {
  static_assert(ROT == 0 || ROT == 128 || ROT == 1024, "rotation block is 0 (none), 128 or 1024");
  static_assert(!PRE || ROT == 1024, "whole-row rotation is for 1024-element blocks");
  // eight tokens' 128-element groups rotate on the matrix cores (rotated_element); with the RMSNorm
  // prologue the normalized activations are fp32, which that product's fp16 operand would round
  constexpr bool MROT = MT == 8 && ROT == 128 && !NORM;
  // the waves' A tiles (MT rows each), and afterwards the waves' sums
  constexpr int kTileBytes = kWaves * MT * kRowPitch * 2, kRedBytes = kWaves * kFB * 4 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
  // byte offsets of tile slots for each start digit off0 (0..4): the group's 128 activations in
  // K order, then the 32 window positions outside the group
  __shared__ __attribute__((aligned(16))) uint16_t slot_tab[5][128];
  __shared__ __attribute__((aligned(16))) uint16_t zero_tab[5][32];
  // the A operand's padding rows MT..15: every lane reads a fragment, those lanes from this zero
  // row (one address per k quarter, so the reads broadcast)
  __shared__ __attribute__((aligned(16))) _Float16 zero_row[160];
  // rotated 1024-blocks of the MT tokens, double-buffered: [buffer][token][1024]
  __shared__ __attribute__((aligned(16))) _Float16 blk[ROT == 1024 && !PRE ? 2 * MT * 1024 : 8];
  // PRE: the MT rows rotated, [MT][k] (dynamic LDS, MT * k * 2 bytes)
  extern __shared__ __attribute__((aligned(16))) _Float16 xrot[];
  __shared__ float norm_part[NORM ? MT * kWaves : 1];  // RMSNorm: per-wave sums of squares

  int m = 0;
  const GemvJob job = gemv_job_of_block(args, &m);  // m read with the job, kept in a register
  const int n = job.n, k = job.k;
  const int groups = k / 128;

  // the wave index is the same in every lane; read it as such so that each wave's group range,
  // loop counters and load offsets stay in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, kq = lane >> 4;
  const int n_base = ((int)blockIdx.x - job.block0) * 16 * kFB;
  const int g_begin = wave * groups / kWaves, g_end = (wave + 1) * groups / kWaves;
  const int blocks = k / 1024;  // used with 1024-element rotation blocks only (k % 1024 == 0)

  // activations: kL lanes per token, each with kE consecutive elements of the group. With eight
  // tokens a token's lanes are those with equal lane bits 2, 4 and 5 (p from bits 0, 1 and 3), so
  // the rotation's three cross-lane butterfly stages pair lanes 1, 2 and 8 apart: each a single
  // DPP move (lanes 4 apart would take two masked moves and a copy)
  // MROT: token lane % 8, p = cb + 2 eq from lane bits 3 and 4..5 (rotated_element)
  constexpr int kL = 64 / MT, kE = 2 * MT;
  const int tok = MROT ? lane & 7 : MT == 8 ? ((lane >> 2) & 1) | ((lane >> 3) & 6) : lane / kL;
  const int p = MROT ? ((lane >> 3) & 1) | ((lane >> 4) << 1) : MT == 8 ? (lane & 3) | ((lane >> 1) & 4) : lane % kL;
  // MROT: the lane's B operand elements of the group, for i = 0 (+ 32 for i = 1): chunk
  // cb + 4 (k quarter >> 1), half (k quarter & 1); and the two A operands
  const int mrot_e = 16 * ((lane >> 3) & 1) + 64 * (lane >> 5) + 8 * ((lane >> 4) & 1);
  const half8 h_plus = MROT ? hadamard16_operand(lane, false) : half8{};
  const half8 h_minus = MROT ? hadamard16_operand(lane, true) : half8{};

  // rows < MT of this wave's A tile, rewritten for every group
  _Float16* tile = reinterpret_cast<_Float16*>(smem) + wave * MT * kRowPitch;
  const _Float16* a_row = fr < MT ? tile + fr * kRowPitch : zero_row;
  // the zero row and the slot tables; the plain basis writes them after its first loads are issued
  auto init_tables = [&]() {
    for (int i = threadIdx.x; i < 160; i += kWaves * 64) zero_row[i] = (_Float16)0.f;
    for (int i = threadIdx.x; i < 5 * 160; i += kWaves * 64) {
      const int o = i / 160, e = i - 160 * o;
      if (e < 128)
        slot_tab[o][e] = (uint16_t)(2 * tile_slot(o + rotated_element<MT, ROT, MROT>(e)));
      else  // rel in [0, o) and [o + 128, 160)
        zero_tab[o][e - 128] = (uint16_t)(2 * tile_slot(e - 128 < o ? e - 128 : e));
    }
    if constexpr (!NORM) __syncthreads();  // the tables (with the norm: at the barrier of norm_factors)
  };
  if constexpr (PRE || ROT == 1024) init_tables();
  // RMSNorm factors: of this lane's token (group staging) and of token `wave` (block staging).
  // Every thread calls norm_factors once, before its first multiply; its barrier also publishes
  // the tables. The plain-basis loop calls it after its first loads are issued, so the rows'
  // extra read overlaps the first weights.
  float rinv_tok = 1.f, rinv_wave = 1.f;
  auto norm_factors = [&]() {
    if constexpr (NORM) {
      rms_partials<MT>(job.x, k, m, 0, norm_part, kWaves * 64);
      __syncthreads();
      rinv_tok = rms_inverse(norm_part, tok, kWaves, k, args.eps);
      rinv_wave = rms_inverse(norm_part, wave < MT ? wave : 0, kWaves, k, args.eps);
    }
  };

  // reads past each buffer return zero: rows >= n, tokens >= m (their outputs are not stored)
  const __amdgpu_buffer_rsrc_t code_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.codes, 0, (int)((int64_t)n * job.stride), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t scale_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.scales, 0, (int)((int64_t)n * groups * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.x, 0, (int)((int64_t)m * k * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t sign_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.signs, 0, ROT ? k : 0, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t gamma_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)job.gamma, 0, NORM ? k * 2 : 0, kRsrcWord3);

  // offsets are unsigned: n * stride < 2^31 and 64 rows more add less than 2^31
  uint32_t row_off[kFB], scale_row[kFB];
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb) {
    const uint32_t row = (uint32_t)(n_base + 16 * fb + fr);
    row_off[fb] = row * (uint32_t)job.stride;
    scale_row[fb] = row * (uint32_t)groups * 2u;
  }

  struct Stage {
    uint32_t c[kFB][3];          // three aligned dwords of codes per row block
    uint32_t s[kFB];             // raw fp16 scale bits
    uint32_t x[MT];              // this lane's kE fp16 activations of the group, in pairs
    uint32_t sg[(kE + 3) / 4];   // their sign bytes
    uint32_t bx[ROT == 1024 ? 8 : 1];  // 1024-blocks: 16 fp16 activations of the next block
    uint32_t bs[ROT == 1024 ? 4 : 1];  // and their sign bytes
    uint32_t gm[NORM && ROT != 1024 ? MT : 1];  // RMSNorm weights (bf16 pairs) of x's elements
    uint32_t bg[NORM && ROT == 1024 ? 8 : 1];   // and of bx's
  };
  auto load_codes = [&](Stage& st, int g, bool live) {
    const uint32_t byte0 = (uint32_t)((128 * g) / 5 + 8 * kq);
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      const int off = live ? (int)(row_off[fb] + (byte0 & ~3u)) : kOobOffset;
      const auto v = __builtin_amdgcn_raw_buffer_load_b96(code_rsrc, off, 0, 0);
      st.c[fb][0] = v[0];
      st.c[fb][1] = v[1];
      st.c[fb][2] = v[2];
      st.s[fb] = __builtin_amdgcn_raw_buffer_load_b16(scale_rsrc, live ? (int)(scale_row[fb] + 2u * g) : kOobOffset,
                                                     0, 0);
    }
  };
  // group g of the contiguous split: codes, scales and this lane's activations (and signs)
  auto load = [&](Stage& st, int g) {
    const bool live = g < g_end;
    load_codes(st, g, live);
    if constexpr (MROT) {
      // x[0..3] and sg[0..1]: the lane's B operand of product i = 0, x[4..7] and sg[2..3]: of i = 1
      const int xo = live ? (tok * k + 128 * g + mrot_e) * 2 : kOobOffset;
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo, 0, 0);
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? xo + 64 : kOobOffset, 0, 0);
      const int so = live ? 128 * g + mrot_e : kOobOffset;
      const auto sa = __builtin_amdgcn_raw_buffer_load_b64(sign_rsrc, so, 0, 0);
      const auto sb = __builtin_amdgcn_raw_buffer_load_b64(sign_rsrc, live ? so + 32 : kOobOffset, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.x[i] = a[i];
        st.x[4 + i] = b[i];
      }
      st.sg[0] = sa[0];
      st.sg[1] = sa[1];
      st.sg[2] = sb[0];
      st.sg[3] = sb[1];
      return;
    }
    const int xo = live ? (tok * k + 128 * g + kE * p) * 2 : kOobOffset;
    if constexpr (MT == 8) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo, 0, 0);
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? xo + 16 : kOobOffset, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.x[i] = a[i];
        st.x[4 + i] = b[i];
      }
    } else if constexpr (MT == 4) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.x[i] = a[i];
    } else if constexpr (MT == 2) {
      const auto a = __builtin_amdgcn_raw_buffer_load_b64(x_rsrc, xo, 0, 0);
      st.x[0] = a[0];
      st.x[1] = a[1];
    } else {
      st.x[0] = __builtin_amdgcn_raw_buffer_load_b32(x_rsrc, xo, 0, 0);
    }
    if constexpr (NORM && ROT != 1024) {  // (1024-blocks load their norm weights with the block)
      const int go = live ? (128 * g + kE * p) * 2 : kOobOffset;
      if constexpr (MT == 8) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(gamma_rsrc, go, 0, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b128(gamma_rsrc, live ? go + 16 : kOobOffset, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          st.gm[i] = a[i];
          st.gm[4 + i] = b[i];
        }
      } else if constexpr (MT == 4) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(gamma_rsrc, go, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.gm[i] = a[i];
      } else if constexpr (MT == 2) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(gamma_rsrc, go, 0, 0);
        st.gm[0] = a[0];
        st.gm[1] = a[1];
      } else {
        st.gm[0] = __builtin_amdgcn_raw_buffer_load_b32(gamma_rsrc, go, 0, 0);
      }
    }
    if constexpr (ROT == 128) {
      const int so = live ? 128 * g + kE * p : kOobOffset;
      if constexpr (MT == 8) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b128(sign_rsrc, so, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.sg[i] = a[i];
      } else if constexpr (MT == 4) {
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(sign_rsrc, so, 0, 0);
        st.sg[0] = a[0];
        st.sg[1] = a[1];
      } else if constexpr (MT == 2) {
        st.sg[0] = __builtin_amdgcn_raw_buffer_load_b32(sign_rsrc, so, 0, 0);
      } else {
        st.sg[0] = __builtin_amdgcn_raw_buffer_load_b16(sign_rsrc, so, 0, 0);
      }
    }
  };
  // 1024-blocks: token t's 16 activations 1024 bb + 16 lane .. and their signs (t < MT)
  auto load_block = [&](Stage& st, int bb, int t) {
    const bool live = bb < blocks && t < MT;
    const int e0 = 1024 * bb + 16 * lane;
    const int xo = live ? (t * k + e0) * 2 : kOobOffset;
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xo, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, live ? xo + 16 : kOobOffset, 0, 0);
    const auto sv = __builtin_amdgcn_raw_buffer_load_b128(sign_rsrc, live ? e0 : kOobOffset, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st.bx[i] = a[i];
      st.bx[4 + i] = b[i];
      st.bs[i] = sv[i];
    }
    if constexpr (NORM) {
      const auto ga = __builtin_amdgcn_raw_buffer_load_b128(gamma_rsrc, live ? 2 * e0 : kOobOffset, 0, 0);
      const auto gb = __builtin_amdgcn_raw_buffer_load_b128(gamma_rsrc, live ? 2 * e0 + 16 : kOobOffset, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st.bg[i] = ga[i];
        st.bg[4 + i] = gb[i];
      }
    }
  };
  // 1024-blocks: signs, the natural-order Sylvester butterfly over the block in fp32 (strides 1..8
  // inside the lane, 16..512 across lanes), 1/sqrt(1024), one rounding to fp16, into dst[0 .. 1024);
  // rn: the token's RMSNorm factor
  auto rotate_block = [&](const Stage& st, _Float16* dst_block, float rn) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t sel = (i & 1) ? 0x030C020Cu : 0x010C000Cu;  // sign bytes 2i, 2i + 1 -> bits 15, 31
      const uint32_t xd = st.bx[i] ^ (__builtin_amdgcn_perm(0u, st.bs[i >> 1], sel) & 0x80008000u);
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)xd);
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(xd >> 16));
      if constexpr (NORM) {
        v[2 * i] *= bf16_lo(st.bg[i]) * rn;
        v[2 * i + 1] *= bf16_hi(st.bg[i]) * rn;
      }
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
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
    // lane strides 16 and 32 (element bits 8 and 9): registers i and i + 8, then i and i + 4, are
    // paired by a lane-half swap, after which a lane holds both partners of one of them and a sum
    // and a difference finish the stage. Element bits 8 and 9 end on register bits 3 and 2, and
    // register bits 3 and 2 (element bits 3 and 2) on lane bits 4 and 5.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      swap_rows16(v[i], v[i + 8]);
      const float a = v[i], b = v[i + 8];
      v[i] = a + b;
      v[i + 8] = a - b;
    }
#pragma unroll
    for (int i = 0; i < 12; ++i)
      if ((i & 4) == 0) {
        swap_halves32(v[i], v[i + 4]);
        const float a = v[i], b = v[i + 4];
        v[i] = a + b;
        v[i + 4] = a - b;
      }
    // registers 4q .. 4q + 3 hold four consecutive elements: q's bits are element bits 9 and 8
    const int e0 = (((lane >> 5) & 1) << 2) | (((lane >> 4) & 1) << 3) | ((lane & 15) << 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(v[4 * q + 2 * h] * 0.03125f));
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(v[4 * q + 2 * h + 1] * 0.03125f));
        w[h] = lo | (hi << 16);
      }
      *reinterpret_cast<uint2*>(dst_block + e0 + 512 * (q & 1) + 256 * (q >> 1)) = make_uint2(w[0], w[1]);
    }
  };

  f32x4 acc[kFB];
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb) acc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  char* row_bytes = reinterpret_cast<char*>(tile + tok * kRowPitch);
  // group g: activations into the tile, decode, 5 MFMA steps, scale; `buf` is the LDS buffer that
  // holds g's rotated 1024-block
  auto compute = [&](const Stage& st, int g, int buf) {
    const int off0 = 128 * g - 5 * ((128 * g) / 5);  // digit of byte B0 where the group starts
    const uint32_t sh = (uint32_t)(((128 * g) / 5 + 8 * kq) & 3);
    // this lane's slots: kE consecutive entries of the table row for off0
    uint16_t slot[kE];
    {
      const uint16_t* src = &slot_tab[off0][kE * p];
      if constexpr (kE >= 8) {
#pragma unroll
        for (int h = 0; h < kE / 8; ++h) {
          const uint4 q = reinterpret_cast<const uint4*>(src)[h];
          const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            slot[8 * h + 2 * i] = (uint16_t)w[i];
            slot[8 * h + 2 * i + 1] = (uint16_t)(w[i] >> 16);
          }
        }
      } else if constexpr (kE == 4) {
        const uint2 q = *reinterpret_cast<const uint2*>(src);
        slot[0] = (uint16_t)q.x;
        slot[1] = (uint16_t)(q.x >> 16);
        slot[2] = (uint16_t)q.y;
        slot[3] = (uint16_t)(q.y >> 16);
      } else {
        const uint32_t q = *reinterpret_cast<const uint32_t*>(src);
        slot[0] = (uint16_t)q;
        slot[1] = (uint16_t)(q >> 16);
      }
    }
    // activations of this group -> tile row tok, in the weight operand's slot order
    _Float16 hv[kE];
    if constexpr (ROT == 1024) {
      // already rotated: kE consecutive fp16 values of token tok's block, at the group's place in it
      const _Float16* src = PRE ? xrot + tok * k + 128 * g + kE * p : blk + (buf * MT + tok) * 1024 + 128 * (g & 7) + kE * p;
      uint32_t w[MT];
      if constexpr (MT >= 4) {
#pragma unroll
        for (int h = 0; h < MT / 4; ++h) {
          const uint4 q = reinterpret_cast<const uint4*>(src)[h];
          w[4 * h] = q.x;
          w[4 * h + 1] = q.y;
          w[4 * h + 2] = q.z;
          w[4 * h + 3] = q.w;
        }
      } else if constexpr (MT == 2) {
        const uint2 q = *reinterpret_cast<const uint2*>(src);
        w[0] = q.x;
        w[1] = q.y;
      } else {
        w[0] = *reinterpret_cast<const uint32_t*>(src);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        hv[2 * i] = __builtin_bit_cast(_Float16, (uint16_t)w[i]);
        hv[2 * i + 1] = __builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
      }
    } else if constexpr (MROT) {
      // sign flip on the fp16 sign bits, then the rotation's products (rotated_element's layout)
      // (the columns of odd chunks, lane bit 3, are negated as well: see the last stage)
      const uint32_t odd_neg = (lane & 8) ? 0x80808080u : 0u;
      uint32_t xs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x030C020Cu : 0x010C000Cu;  // sign bytes 2i, 2i + 1 -> bits 15, 31
        xs[i] = st.x[i] ^ (__builtin_amdgcn_perm(0u, st.sg[i >> 1] ^ odd_neg, sel) & 0x80008000u);
      }
      f32x4 d[2][2];  // [chunk bit 2 of the output][i]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const half8 b = __builtin_bit_cast(half8, make_uint4(xs[4 * i], xs[4 * i + 1], xs[4 * i + 2], xs[4 * i + 3]));
        d[0][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_plus, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        d[1][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h_minus, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      }
      float v[16];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = d[h][0][r], b = d[h][1][r];
          v[8 * h + r] = a + b;      // chunk bit 1 clear
          v[8 * h + 4 + r] = a - b;  // chunk bit 1 set
        }
      // chunk bit 0: the even lane holds a, the odd one -b (its column was negated), so
      // own + partner * (-1 even, +1 odd) gives a + b and a - b: one multiply-add that takes the
      // partner through DPP
      const float sp = (lane & 8) ? 1.f : -1.f;
      fmac_partner8x16(v, sp);
#pragma unroll
      for (int j = 0; j < 16; ++j) hv[j] = (_Float16)(v[j] * 0.08838834764831845f);  // 1/sqrt(128)
    } else {
      // 128-blocks: sign flip (on the fp16 sign bits), the natural-order Sylvester butterfly over
      // the group in fp32 (strides below kE inside the lane, the rest across lanes), 1/sqrt(128),
      // one rounding to fp16
      float v[kE];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        uint32_t xd = st.x[i];
        if constexpr (ROT == 128) {
          // sign bytes of elements 2i and 2i + 1 -> bits 15 and 31
          const uint32_t sel = (i & 1) ? 0x030C020Cu : 0x010C000Cu;
          xd ^= __builtin_amdgcn_perm(0u, st.sg[i >> 1], sel) & 0x80008000u;
        }
        v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)xd);
        v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(xd >> 16));
        if constexpr (NORM) {
          v[2 * i] *= bf16_lo(st.gm[i]) * rinv_tok;
          v[2 * i + 1] *= bf16_hi(st.gm[i]) * rinv_tok;
        }
      }
      if constexpr (ROT == 128) {
#pragma unroll
        for (int h = 1; h < kE; h <<= 1)
#pragma unroll
          for (int i = 0; i < kE; ++i)
            if ((i & h) == 0) {
              const float a = v[i], b = v[i + h];
              v[i] = a + b;
              v[i + h] = a - b;
            }
        auto cross = [&](auto s_tag) {
          constexpr int S = decltype(s_tag)::value;       // stride in p
          constexpr int LS = (MT == 8 && S == 4) ? 8 : S;  // the same stride in lanes
          const float sgn = (p & S) ? -1.f : 1.f;  // the upper lane of a pair keeps partner - own
#pragma unroll
          for (int i = 0; i < kE; ++i) v[i] = fmaf(v[i], sgn, xor_lane<LS>(v[i], lane));
        };
        if constexpr (kL > 1) cross(std::integral_constant<int, 1>{});
        if constexpr (kL > 2) cross(std::integral_constant<int, 2>{});
        if constexpr (kL > 4) cross(std::integral_constant<int, 4>{});
        if constexpr (kL > 8) cross(std::integral_constant<int, 8>{});
        if constexpr (MT == 1) {
          // lane strides 16 and 32 (element bits 5 and 6): after each swap a lane holds both
          // partners of one of its elements, so a sum and a difference finish the stage (the slot
          // table follows the new places, rotated_element)
          swap_rows16(v[0], v[1]);
          float a = v[0], b = v[1];
          v[0] = a + b;
          v[1] = a - b;
          swap_halves32(v[0], v[1]);
          a = v[0];
          b = v[1];
          v[0] = a + b;
          v[1] = a - b;
        } else {
          if constexpr (kL > 16) cross(std::integral_constant<int, 16>{});
          if constexpr (kL > 32) cross(std::integral_constant<int, 32>{});
        }
#pragma unroll
        for (int i = 0; i < kE; ++i) v[i] *= 0.08838834764831845f;  // 1/sqrt(128)
      }
#pragma unroll
      for (int i = 0; i < kE; ++i) hv[i] = (_Float16)v[i];
    }
#pragma unroll
    for (int i = 0; i < kE; ++i) *reinterpret_cast<_Float16*>(row_bytes + slot[i]) = hv[i];
    // the 32 window slots outside the group meet zeros
    if constexpr (kL <= 32) {
      constexpr int kZ = 32 / kL;
#pragma unroll
      for (int z = 0; z < kZ; ++z) *reinterpret_cast<_Float16*>(row_bytes + zero_tab[off0][kZ * p + z]) = (_Float16)0.f;
    } else {
      if (p < 32) *reinterpret_cast<_Float16*>(row_bytes + zero_tab[off0][p]) = (_Float16)0.f;
    }
    __asm__ volatile("" ::: "memory");  // the tile writes precede the fragment reads (one wave, in order)

    // this lane's 8 bytes of each row block, then 5 MFMA steps
    u16x2 ve0[kFB], vo0[kFB], ve1[kFB], vo1[kFB];
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      const uint32_t w0 = __builtin_amdgcn_alignbyte(st.c[fb][1], st.c[fb][0], sh);
      const uint32_t w1 = __builtin_amdgcn_alignbyte(st.c[fb][2], st.c[fb][1], sh);
      ve0[fb] = __builtin_bit_cast(u16x2, w0 & 0x00FF00FFu);
      vo0[fb] = __builtin_bit_cast(u16x2, (w0 >> 8) & 0x00FF00FFu);
      ve1[fb] = __builtin_bit_cast(u16x2, w1 & 0x00FF00FFu);
      vo1[fb] = __builtin_bit_cast(u16x2, (w1 >> 8) & 0x00FF00FFu);
    }
    // part: sum x t per row block
    f32x4 part[kFB];
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) part[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const half8 a = *reinterpret_cast<const half8*>(a_row + (kq * 5 + j) * 8);
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) {
        const u16x2 de0 = j < 4 ? peel(ve0[fb]) : ve0[fb];
        const u16x2 do0 = j < 4 ? peel(vo0[fb]) : vo0[fb];
        const u16x2 de1 = j < 4 ? peel(ve1[fb]) : ve1[fb];
        const u16x2 do1 = j < 4 ? peel(vo1[fb]) : vo1[fb];
        const uint4 b4 = make_uint4(digits_to_weights(de0), digits_to_weights(do0), digits_to_weights(de1),
                                    digits_to_weights(do1));
        part[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, b4), part[fb], 0, 0, 0);
      }
    }
    __asm__ volatile("" ::: "memory");  // the fragment reads precede the next group's tile writes
    // D[i][j] (token i, output j) sits in lane 16 * (i / 4) + j, register i % 4
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)st.s[fb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[fb][r] = fmaf(sc, part[fb][r], acc[fb][r]);
    }
  };

  if constexpr (PRE) {
    // every block of every token rotated once (round robin over the waves), then contiguous group
    // slices per wave, as in the plain basis
    norm_factors();
    for (int idx = wave; idx < MT * blocks; idx += kWaves) {
      const int t = idx / blocks, bb = idx - t * blocks;
      Stage st;
      load_block(st, bb, t);
      const float rn = NORM ? rms_inverse(norm_part, t, kWaves, k, args.eps) : 1.f;
      rotate_block(st, xrot + t * k + 1024 * bb, rn);
    }
    __syncthreads();
    Stage st0, st1;
    load_codes(st0, g_begin, g_begin < g_end);
    for (int g = g_begin; g < g_end; g += 2) {
      load_codes(st1, g + 1, g + 1 < g_end);
      compute(st0, g, 0);
      if (g + 1 >= g_end) break;
      load_codes(st0, g + 2, g + 2 < g_end);
      compute(st1, g + 1, 0);
    }
  } else if constexpr (ROT == 1024) {
    // block b: waves < MT rotate block b + 1 into buffer (b + 1) & 1 while every wave multiplies
    // group 8 b + wave from buffer b & 1; the barrier closing block b orders both against block
    // b + 1 (every wave runs the same number of blocks, so all reach every barrier)
    auto step = [&](const Stage& st, int b) {
      if (wave < MT && b + 1 < blocks) rotate_block(st, blk + (((b + 1) & 1) * MT + wave) * 1024, rinv_wave);
      compute(st, 8 * b + wave, b & 1);
      __syncthreads();
    };
    norm_factors();
    {
      Stage st;
      load_block(st, 0, wave);
      if (wave < MT) rotate_block(st, blk + wave * 1024, rinv_wave);
    }
    __syncthreads();
    // stage b holds group 8 b + wave's codes and block b + 1's activations; two stages in flight
    Stage st0, st1;
    load_codes(st0, wave, 0 < blocks);
    load_block(st0, 1, wave);
    for (int b = 0; b < blocks; b += 2) {
      load_codes(st1, 8 * (b + 1) + wave, b + 1 < blocks);
      load_block(st1, b + 2, wave);
      step(st0, b);
      if (b + 1 >= blocks) break;
      load_codes(st0, 8 * (b + 2) + wave, b + 2 < blocks);
      load_block(st0, b + 3, wave);
      step(st1, b + 1);
    }
  } else {
    // kS - 1 groups of loads in flight ahead of the one being multiplied (a ring of kS stages);
    // loads past the wave's last group are parked out of range
    constexpr int kS = MT == 1 ? kStagesOneToken : kStagesTokens;
    Stage st[kS];
#pragma unroll
    for (int i = 0; i < kS - 1; ++i) load(st[i], g_begin + i);
    init_tables();
    norm_factors();
    for (int g = g_begin; g < g_end; g += kS) {
#pragma unroll
      for (int u = 0; u < kS; ++u) {
        if (g + u >= g_end) break;
        load(st[(u + kS - 1) % kS], g + u + kS - 1);
        compute(st[u], g + u, 0);
      }
    }
  }

  // add the waves' sums in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [wave][fb * 4 + r][lane]
  static_assert(kRedBytes <= sizeof(smem), "the wave sums fit in the tile memory");
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * kFB * 4 + fb * 4 + r) * 64 + lane] = acc[fb][r];
  __syncthreads();
  for (int e = threadIdx.x; e < kFB * 4 * 64; e += kWaves * 64) {
    const int idx = e >> 6, ln = e & 63;
    const int fb = idx >> 2, r = idx & 3;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[(w * kFB * 4 + idx) * 64 + ln];
    const int token = 4 * (ln >> 4) + r, row = n_base + 16 * fb + (ln & 15);
    if (token < m && row < n) job.y[(int64_t)token * n + row] = sum;
  }
}

// the whole rotated activation rows of a launch fit this much dynamic LDS
constexpr int kPreRotBytes = 48 * 1024;

template <int MT, int FB, bool NORM>
hipError_t launch_rot(GemvArgs& args, int blocks, int32_t block, hipStream_t stream) {
  int max_k = 0;
  for (int i = 0; i < args.count; ++i) max_k = args.job[i].k > max_k ? args.job[i].k : max_k;
  const size_t pre_bytes = (size_t)MT * (size_t)max_k * 2;
  if (block == 1024 && pre_bytes <= (size_t)kPreRotBytes)
    hipLaunchKernelGGL((gemv_b3_mfma_kernel<MT, FB, 1024, NORM, true>), dim3(blocks), dim3(kWaves * 64), pre_bytes,
                       stream, args);
  else if (block == 1024)
    hipLaunchKernelGGL((gemv_b3_mfma_kernel<MT, FB, 1024, NORM, false>), dim3(blocks), dim3(kWaves * 64), 0, stream,
                       args);
  else if (block)
    hipLaunchKernelGGL((gemv_b3_mfma_kernel<MT, FB, 128, NORM, false>), dim3(blocks), dim3(kWaves * 64), 0, stream,
                       args);
  else
    hipLaunchKernelGGL((gemv_b3_mfma_kernel<MT, FB, 0, NORM, false>), dim3(blocks), dim3(kWaves * 64), 0, stream,
                       args);
  return hipGetLastError();
}

template <int MT, int FB>
hipError_t launch_mt(GemvArgs& args, int blocks, int32_t block, bool norm, hipStream_t stream) {
  return norm ? launch_rot<MT, FB, true>(args, blocks, block, stream)
              : launch_rot<MT, FB, false>(args, blocks, block, stream);
}

}  // namespace

int gemv_b3_mfma_rows(int32_t m) { return 16 * (m == 1 ? kMfmaFB1 : kMfmaFBMulti); }

hipError_t gemv_b3_mfma_launch(GemvArgs& args, int32_t blocks, int32_t m, int32_t block, bool norm,
                               hipStream_t stream) {
  if (m <= 1) return launch_mt<1, kMfmaFB1>(args, blocks, block, norm, stream);
  if (m <= 2) return launch_mt<2, kMfmaFBMulti>(args, blocks, block, norm, stream);
  if (m <= 4) return launch_mt<4, kMfmaFBMulti>(args, blocks, block, norm, stream);
  return launch_mt<8, kMfmaFBMulti>(args, blocks, block, norm, stream);
}

}  // namespace tgs
