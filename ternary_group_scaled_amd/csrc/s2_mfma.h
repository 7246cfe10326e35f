// Matrix-core building blocks of the single-token slot-2 GEMV, shared by the one-launch kernel
// (gemv_s2_mfma.hip) and the step-chain kernel (gemv_chain.hip).
//
// The weight definition is the one of "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)"
// (discuss.pytorch.kr), subsection "Group-scaled ternary format": w = s_g * t, t in {-1, 0, +1},
// one fp16 scale per 128 consecutive weights of a row.
//
// Window. 512 weights of 16 output rows: lane (c, q) (c = lane % 16, q = lane / 16) owns group q of
// the window in row c (32 bytes of codes, two 16-byte loads; the four lanes of a row read its 128
// contiguous bytes). v_mfma_f32_16x16x32_f16 computes D[r][c] = sum over 32 k of A[r][k] B[k][c]:
// B holds 8 weights of lane (c, q) per step, 16 steps per window. A holds the activations: row r
// carries the window's group r, present only in lane (r, q = r) and zero elsewhere, so D[r][c] is
// the partial sum of group r for output row c, and lane c holds the four groups' partials in its
// four D registers.
//
// Decode. Codes q = t + 1 sit in 2-bit slots, element j of a little-endian 32-bit word in bits
// 2j..2j+1. The pair (j, j+8) sits in bits p..p+1 of both 16-bit halves of the word, or of the word
// shifted right by 6 (p in {0, 2, 4, 6, 8}). One v_and_or_b32 keeps those bits and sets the exponent
// field 25 - p, which makes each half the fp16 number 2^(10-p) + q exactly; one packed fp16 add of
// -(2^(10-p) + 1) leaves t = q - 1 (-1.0, 0 or +1.0) in each half, again exactly. Every product
// t * x is exact and a zero code adds nothing, so a row with one nonzero code gives s * t * x_k
// exactly.
//
// Activations in LDS. x is staged as dot2-style pairs (x_j, x_{j+8}) of every 16 elements, in the
// order of the weight operand: A fragment s of group g is 16 bytes at word 68 g + 4 s (64 words
// per group plus 4 of padding, so the four groups a step reads fall in different banks). Lanes
// whose A entries are zero read a 256-byte zero region instead, one shared address per step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rms_norm.h"

namespace tgs {
namespace s2 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWinK = 512;           // weights of a row per window: four scale groups
constexpr int kGroupPitch = 68;      // LDS words per group of activation pairs (64 + 4)
constexpr int kZeroBytes = 16 * 16;  // one 16-byte zero fragment per MFMA step
constexpr int kMaxK = 16384;         // largest K of the matrix-core single-token path

// A 32-bit constant in a vector register: the three-operand AND-OR takes no literal, and its other
// constant (the mask) goes in a scalar register.
template <uint32_t V>
__device__ __forceinline__ uint32_t vconst() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}

// exponent bits that give the code bits p..p+1 the weight 1: 2^(10-p) + q in each half
template <int P>
constexpr uint32_t kExpBits = ((uint32_t)(25 - P) << 10) * 0x00010001u;

struct ExpBits {
  uint32_t e0, e2, e4, e6, e8;
};

__device__ __forceinline__ ExpBits exp_bits() {
  return ExpBits{vconst<kExpBits<0>>(), vconst<kExpBits<2>>(), vconst<kExpBits<4>>(), vconst<kExpBits<6>>(),
                 vconst<kExpBits<8>>()};
}

// t in both fp16 halves from the codes in bits P..P+1 of each half of `word`; eb = the matching
// field of exp_bits()
template <int P>
__device__ __forceinline__ uint32_t signed_pair(uint32_t word, uint32_t eb) {
  constexpr uint32_t kMask = 0x00030003u << P;
  // -(2^(10-P) + 1) in both halves, exactly representable (11 significant bits at most)
  constexpr uint32_t kNeg = (0x8000u | ((uint32_t)(25 - P) << 10) | (1u << P)) * 0x00010001u;
  const half2v h = __builtin_bit_cast(half2v, (word & kMask) | eb);
  return __builtin_bit_cast(uint32_t, h + __builtin_bit_cast(half2v, kNeg));
}

// B operand of MFMA step s (0..15) of a window from the lane's 32 code bytes c[0], c[1]
__device__ __forceinline__ uint4 weights_of_step(const uint4* c, int s, const ExpBits& e) {
  const uint4& h = c[s >> 3];
  const uint32_t u = (s & 6) == 0 ? h.x : ((s & 6) == 2 ? h.y : ((s & 6) == 4 ? h.z : h.w));
  if ((s & 1) == 0)  // pairs j = 0..3: bits 0, 2, 4, 6 of u
    return make_uint4(signed_pair<0>(u, e.e0), signed_pair<2>(u, e.e2), signed_pair<4>(u, e.e4),
                      signed_pair<6>(u, e.e6));
  const uint32_t v = u >> 6;  // pairs j = 4..7: bit 8 of u, bits 4, 6, 8 of u >> 6
  return make_uint4(signed_pair<8>(u, e.e8), signed_pair<4>(v, e.e4), signed_pair<6>(v, e.e6),
                    signed_pair<8>(v, e.e8));
}

// NW windows as independent MFMA chains, interleaved step by step: d[i] += A(a_base[i]) B(cw[i])
template <int NW>
__device__ __forceinline__ void mfma_windows(const char* const* a_base, const uint4 (*cw)[2], f32x4* d,
                                             const ExpBits& e) {
#pragma unroll
  for (int s = 0; s < 16; ++s) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const half8 a = *reinterpret_cast<const half8*>(a_base[i] + 16 * s);
      const uint4 b = weights_of_step(cw[i], s, e);
      d[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8, b), d[i], 0, 0, 0);
    }
  }
}

// acc + the four groups' partials of a window times their fp16 scales (4 fp16 in sc), in fp32
__device__ __forceinline__ float scale_window(float acc, uint2 sc, const f32x4& d) {
  acc = fmaf(half_lo(sc.x), d[0], acc);
  acc = fmaf(half_hi(sc.x), d[1], acc);
  acc = fmaf(half_lo(sc.y), d[2], acc);
  acc = fmaf(half_hi(sc.y), d[3], acc);
  return acc;
}

// Activation pair (element e1 in the low half, e2 in the high half) from fp16 words w[e/2].
template <int E1, int E2>
__device__ __forceinline__ uint32_t xpair(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

// the pairs of staging unit u (16 consecutive fp16 activations, 8 words) into the LDS pair array
__device__ __forceinline__ void store_unit_pairs(uint32_t* pairs, int u, const uint32_t* xw) {
  uint4* dst = reinterpret_cast<uint4*>(pairs + (u >> 3) * kGroupPitch + (u & 7) * 8);
  dst[0] = make_uint4(xpair<0, 8>(xw), xpair<1, 9>(xw), xpair<2, 10>(xw), xpair<3, 11>(xw));
  dst[1] = make_uint4(xpair<4, 12>(xw), xpair<5, 13>(xw), xpair<6, 14>(xw), xpair<7, 15>(xw));
}

// LDS bytes of the pair array for K (the zero region follows it)
__host__ __device__ constexpr int pair_bytes(int k) { return (k / 128) * kGroupPitch * 4; }

}  // namespace s2
}  // namespace tgs
