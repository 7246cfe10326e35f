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
// of them, element j in bits 2j..2j+1. ANDing the word with 0x00030003 << 2i keeps the codes of
// elements i and i+8 in the low mantissa bits of the two fp16 halves: with a zero exponent
// field those halves are the fp16 subnormals q * 4^i * 2^-24, exactly. v_dot2_f32_f16 then
// multiplies them by the activation pair (x_i, x_{i+8}) and adds into an fp32 accumulator:
// products of an 11-bit significand by q * 4^i are exact, so each position i (i < 5) keeps
// its own accumulator, and positions 5..7 reuse the accumulators of 0..2 after one 10-bit shift
// of the word. At the end of a chunk the five accumulators are rescaled by 2^24 / 4^i (exact
// powers of two) and sum_k q x - sum_k x = sum_k t x. That is one AND and one dot2 per two
// weights plus one shift per word, instead of a shift/mask/convert/FMA per weight.
//
// Base-3. Each byte holds five trits, byte = sum_j (t_j + 1) 3^j. A word is split into two
// 16-bit lanes (bytes 0,2 and bytes 1,3); each digit is peeled off both lanes at once with
// packed 16-bit integer ops (q = v * 171 >> 9 equals v / 3 for v < 256; digit = v - 3q). The
// digit, 0..2, in a 16-bit lane is again an fp16 subnormal, fed to dot2 as above. A 16-byte
// chunk (80 trits) can straddle a 128-trit scale group, so each lane keeps two accumulators and
// masks its activation pairs by group once per slice.
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
constexpr int kIter = 4;  // rows per lane slot per workgroup

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Activation pair (element e1 in the low half, e2 in the high half) from fp16 words w[e/2].
template <int E1, int E2>
__device__ __forceinline__ uint32_t xpair(const uint32_t* w) {
  constexpr uint32_t sel = ((E1 & 1) ? 0x0302u : 0x0100u) | (((E2 & 1) ? 0x0706u : 0x0504u) << 16);
  return __builtin_amdgcn_perm(w[E2 / 2], w[E1 / 2], sel);
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w)[0];
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(half2_t, w)[1];
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
  float sum[MT];       // sum of the chunk's 64 activations

  __device__ __forceinline__ void load(const uint16_t* lds_chunk, int token_stride, int /*boundary*/) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      uint32_t w[32];
      const uint4* src = reinterpret_cast<const uint4*>(lds_chunk + t * token_stride);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        uint4 q = src[v];
        w[4 * v + 0] = q.x;
        w[4 * v + 1] = q.y;
        w[4 * v + 2] = q.z;
        w[4 * v + 3] = q.w;
      }
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 32; ++v) s += half_lo(w[v]) + half_hi(w[v]);
      sum[t] = s;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        p[t][8 * d + 0] = xpair<0, 8>(w + 8 * d);
        p[t][8 * d + 1] = xpair<1, 9>(w + 8 * d);
        p[t][8 * d + 2] = xpair<2, 10>(w + 8 * d);
        p[t][8 * d + 3] = xpair<3, 11>(w + 8 * d);
        p[t][8 * d + 4] = xpair<4, 12>(w + 8 * d);
        p[t][8 * d + 5] = xpair<5, 13>(w + 8 * d);
        p[t][8 * d + 6] = xpair<6, 14>(w + 8 * d);
        p[t][8 * d + 7] = xpair<7, 15>(w + 8 * d);
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
  float sum[2][MT];

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
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int v = 0; v < 40; ++v) {
        float a = half_lo(w[v]), b = half_hi(w[v]);
        if (2 * v < boundary) s0 += a; else s1 += a;
        if (2 * v + 1 < boundary) s0 += b; else s1 += b;
      }
      sum[0][t] = s0;
      sum[1][t] = s1;
      set_dword<0>(w, t, boundary);
      set_dword<1>(w, t, boundary);
      set_dword<2>(w, t, boundary);
      set_dword<3>(w, t, boundary);
    }
  }
};

// ---- per-row chunk products ------------------------------------------------------------

// Slot-2: returns sum_k t_k x_k over the 64 weights of the chunk for each token.
template <int MT>
__device__ __forceinline__ void chunk_dot_slot2(const uint4& cw, const XRegs<TGS_LAYOUT_SLOT2, MT>& xr,
                                                float (&out)[MT]) {
  float a[MT][5];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 5; ++i) a[t][i] = 0.f;
  const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t u = words[d];
    const uint32_t u10 = u >> 10;
    const uint32_t m0 = u & 0x00030003u, m1 = u & 0x000C000Cu, m2 = u & 0x00300030u, m3 = u & 0x00C000C0u,
                   m4 = u & 0x03000300u, m5 = u10 & 0x00030003u, m6 = u10 & 0x000C000Cu, m7 = u10 & 0x00300030u;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint32_t* p = &xr.p[t][8 * d];
      a[t][0] = dot2(m0, p[0], a[t][0]);
      a[t][1] = dot2(m1, p[1], a[t][1]);
      a[t][2] = dot2(m2, p[2], a[t][2]);
      a[t][3] = dot2(m3, p[3], a[t][3]);
      a[t][4] = dot2(m4, p[4], a[t][4]);
      a[t][0] = dot2(m5, p[5], a[t][0]);
      a[t][1] = dot2(m6, p[6], a[t][1]);
      a[t][2] = dot2(m7, p[7], a[t][2]);
    }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    // sum q x = 2^24 * (a0 + a1/4 + a2/16 + a3/64 + a4/256); every factor is a power of two
    float h = fmaf(fmaf(fmaf(fmaf(a[t][4], 0.25f, a[t][3]), 0.25f, a[t][2]), 0.25f, a[t][1]), 0.25f, a[t][0]);
    out[t] = fmaf(h, 16777216.0f, -xr.sum[t]);
  }
}

// Base-3: sums for the (up to) two scale groups of the chunk, per token.
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
      const uint32_t be = __builtin_bit_cast(uint32_t, de), bo = __builtin_bit_cast(uint32_t, dd);
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
    out0[t] = fmaf(a0[t], 16777216.0f, -xr.sum[0][t]);
    out1[t] = fmaf(a1[t], 16777216.0f, -xr.sum[1][t]);
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

template <int LAYOUT, int S, int MT, bool ROT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvArgs args) {
  using G = Geo<LAYOUT>;
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

  for (int m0 = 0; m0 < m; m0 += MT) {
    float part[kIter][MT];
#pragma unroll
    for (int it = 0; it < kIter; ++it)
#pragma unroll
      for (int t = 0; t < MT; ++t) part[it][t] = 0.f;

    for (int ks = 0; ks < slices; ++ks) {
      const int k_begin = ks * kSliceElems;
      __syncthreads();  // the previous slice's activations are no longer read
      if constexpr (ROT)
        stage_rotated<MT>(xs, kSliceElems, job.x, job.signs, k, m, m0, k_begin);
      else
        stage_plain<MT>(xs, kSliceElems, job.x, k, m, m0, k_begin);
      __syncthreads();

      const int c = ks * S + cl;  // this lane's chunk
      const bool chunk_ok = c < chunks;
      // first trit of the second scale group, relative to the chunk (base-3 only)
      const int t0 = c * G::kElems;
      const int boundary = (LAYOUT == TGS_LAYOUT_BASE3) ? ((t0 / 128 + 1) * 128 - t0) : 1 << 20;

      XRegs<LAYOUT, MT> xr;
      xr.load(xs + cl * G::kElems, kSliceElems, boundary);

      uint4 cw[kIter];
#pragma unroll
      for (int it = 0; it < kIter; ++it) {
        const int row = row0 + it * kRowsPerInstr;
        cw[it] = make_uint4(0, 0, 0, 0);
        if (chunk_ok && row < n)
          cw[it] = *reinterpret_cast<const uint4*>(job.codes + (int64_t)row * job.stride + (int64_t)c * 16);
      }
      if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
        float sc[kIter];
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
          const int row = row0 + it * kRowsPerInstr;
          sc[it] = (chunk_ok && row < n) ? f16_to_f32(job.scales[(int64_t)row * groups + c / 2]) : 0.f;
        }
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
          float tx[MT];
          chunk_dot_slot2<MT>(cw[it], xr, tx);
#pragma unroll
          for (int t = 0; t < MT; ++t) part[it][t] = fmaf(sc[it], tx[t], part[it][t]);
        }
      } else {
        const int g0 = t0 / 128;
        const bool has_g1 = boundary < G::kElems && g0 + 1 < groups;
        float sc0[kIter], sc1[kIter];
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
          const int row = row0 + it * kRowsPerInstr;
          const bool ok = chunk_ok && row < n;
          sc0[it] = ok ? f16_to_f32(job.scales[(int64_t)row * groups + g0]) : 0.f;
          sc1[it] = (ok && has_g1) ? f16_to_f32(job.scales[(int64_t)row * groups + g0 + 1]) : 0.f;
        }
#pragma unroll
        for (int it = 0; it < kIter; ++it) {
          float tx0[MT], tx1[MT];
          chunk_dot_base3<MT>(cw[it], xr, tx0, tx1);
#pragma unroll
          for (int t = 0; t < MT; ++t) part[it][t] = fmaf(sc1[it], tx1[t], fmaf(sc0[it], tx0[t], part[it][t]));
        }
      }
    }

    // reduce across the S lanes of each row, fixed order
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        float v = part[it][t];
#pragma unroll
        for (int off = S / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        part[it][t] = v;
      }
    }
    if (cl == 0) {
#pragma unroll
      for (int it = 0; it < kIter; ++it) {
        const int row = row0 + it * kRowsPerInstr;
        if (row < n) {
#pragma unroll
          for (int t = 0; t < MT; ++t)
            if (m0 + t < m) job.y[(int64_t)(m0 + t) * n + row] = part[it][t];
        }
      }
    }
  }
}

template <int LAYOUT, int S, int MT, bool ROT>
hipError_t launch_one(GemvArgs& args, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL((gemv_kernel<LAYOUT, S, MT, ROT>), dim3(blocks), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

template <int LAYOUT, int S, int MT>
hipError_t launch_rot(bool rot, GemvArgs& args, int blocks, hipStream_t stream) {
  return rot ? launch_one<LAYOUT, S, MT, true>(args, blocks, stream)
             : launch_one<LAYOUT, S, MT, false>(args, blocks, stream);
}

template <int LAYOUT, int S>
hipError_t launch_mt(int mt, bool rot, GemvArgs& args, int blocks, hipStream_t stream) {
  if constexpr (LAYOUT == TGS_LAYOUT_SLOT2) {
    switch (mt) {
      case 1: return launch_rot<LAYOUT, S, 1>(rot, args, blocks, stream);
      case 2: return launch_rot<LAYOUT, S, 2>(rot, args, blocks, stream);
      case 4: return launch_rot<LAYOUT, S, 4>(rot, args, blocks, stream);
      default: return launch_rot<LAYOUT, S, 8>(rot, args, blocks, stream);
    }
  } else {
    return mt == 1 ? launch_rot<LAYOUT, S, 1>(rot, args, blocks, stream)
                   : launch_rot<LAYOUT, S, 2>(rot, args, blocks, stream);
  }
}

template <int LAYOUT>
hipError_t launch_s(int s, int mt, bool rot, GemvArgs& args, int blocks, hipStream_t stream) {
  switch (s) {
    case 16: return launch_mt<LAYOUT, 16>(mt, rot, args, blocks, stream);
    case 32: return launch_mt<LAYOUT, 32>(mt, rot, args, blocks, stream);
    default: return launch_mt<LAYOUT, 64>(mt, rot, args, blocks, stream);
  }
}

}  // namespace

// Tokens per pass (compile-time width of the activation registers).
static int tokens_per_pass(int32_t layout, int64_t m) {
  if (layout == TGS_LAYOUT_BASE3) return m >= 2 ? 2 : 1;
  int mt = 1;
  while (mt < m) mt *= 2;
  return mt;
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
  p.rows_per_block = kWaves * kIter * (64 / best);
  return p;
}

hipError_t gemv_launch(const GemvPlan& plan, GemvArgs& args, int32_t blocks, hipStream_t stream) {
  const int mt = tokens_per_pass(plan.layout, plan.m);
  const bool rot = plan.rotated != 0;
  if (plan.layout == TGS_LAYOUT_SLOT2)
    return launch_s<TGS_LAYOUT_SLOT2>(plan.lanes, mt, rot, args, blocks, stream);
  return launch_s<TGS_LAYOUT_BASE3>(plan.lanes, mt, rot, args, blocks, stream);
}

}  // namespace tgs
