// Cross-lane moves within a 64-lane wave on gfx950, shared by the GEMV kernels: DPP row and quad
// patterns, and the lane-half swaps.
#pragma once

#include <hip/hip_runtime.h>

namespace tgs {

// 32-bit lane moves within 16-lane rows (DPP): rotate right by N, or fixed quad/half patterns
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppRor1 = 0x121, kDppRor2 = 0x122, kDppRor4 = 0x124, kDppRor8 = 0x128, kDppRor12 = 0x12C;
constexpr int kDppHalfMirror = 0x141, kDppQuadSwap2 = 0x4E, kDppQuadSwap1 = 0xB1;

// Lane-half swaps, as inline asm: with the swap builtins (ROCm 7.2 hipcc), an expression that
// uses both results reads the first one twice, so the operands are passed read-write here. Each
// s_nop 1 gives the two wait states a VALU write needs before a swap reads the register, and the
// same after, before the next VALU reads the result.
__device__ __forceinline__ void swap_halves32(float& a, float& b) {  // a's lanes 32..63 <-> b's 0..31
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows16(float& a, float& b) {  // a's odd 16-lane rows <-> b's even
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// v of lane (lane ^ S), S a power of two below 64
template <int S>
__device__ __forceinline__ float xor_lane(float v, int lane) {
  if constexpr (S == 1) {
    return dpp<kDppQuadSwap1>(v);
  } else if constexpr (S == 2) {
    return dpp<kDppQuadSwap2>(v);
  } else if constexpr (S == 4) {
    // lanes with bit 2 clear (banks 0 and 2 of each row) take lane + 4, the others lane - 4
    const int b = __builtin_bit_cast(int, v);
    int r = __builtin_amdgcn_update_dpp(b, b, kDppRor12, 0xF, 0x5, false);  // banks 1, 3: written next
    r = __builtin_amdgcn_update_dpp(r, b, kDppRor4, 0xF, 0xA, false);
    return __builtin_bit_cast(float, r);
  } else if constexpr (S == 8) {
    return dpp<kDppRor8>(v);
  } else if constexpr (S == 16) {
    float a = v, b = v;
    swap_rows16(a, b);
    return (lane & 16) ? a : b;
  } else {
    static_assert(S == 32, "xor distance must be a power of two below 64");
    float a = v, b = v;
    swap_halves32(a, b);
    return (lane & 32) ? a : b;
  }
}

}  // namespace tgs
