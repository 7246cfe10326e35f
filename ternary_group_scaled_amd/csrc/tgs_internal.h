// Internal declarations shared by the host entry points (tgs_host.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgs.h"

namespace tgs {

constexpr int kMaxJobs = TGS_MAX_BATCH;
// Largest code plane of one matrix on the device. Kernels read through 32-bit buffer offsets and
// park loads they do not need at kOobOffset, which must lie past every valid range.
constexpr int64_t kMaxDeviceCodeBytes = (1LL << 31) - (1LL << 20);
constexpr int kOobOffset = 0x7FFFFFF0;
// cache policy of a weight stream read once: non-temporal
constexpr int kStreamAux = 2;
// word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format, no swizzle); reads
// past the resource's size return zero
constexpr int kRsrcWord3 = 0x00020000;
// The single-token kernel runs one wave per 4096 weights of K, at most 16 per workgroup.
constexpr int kMaxWaveKernelK = 16 * 4096;
// and aims for at least this many waves per launch when choosing rows per wave
constexpr int kWaveKernelTargetWaves = 4096;

// One matrix of a batched GEMV launch. All pointers are device pointers.
struct GemvJob {
  const uint8_t* codes;    // [n][stride]
  const uint16_t* scales;  // [n][k/128] fp16 bits
  const uint16_t* x;       // [m][k] fp16 bits
  const int8_t* signs;     // [k] or nullptr (plain basis)
  float* y;                // [m][n]
  int64_t stride;          // bytes between rows of codes
  int32_t n;
  int32_t k;
  int32_t block0;          // first workgroup of this job in the launch
  int32_t row_blocks;      // workgroups for this job
};

struct GemvArgs {
  GemvJob job[kMaxJobs];
  int32_t count;
  int32_t m;
};

// Shape class of a GEMV launch: every job in one launch shares these.
struct GemvPlan {
  int32_t layout;     // TGS_LAYOUT_*
  int32_t lanes;      // lanes per row (16, 32 or 64)
  int32_t m;          // activation rows
  int32_t rotated;    // 0 or 1
  int32_t stream;     // 1: the single-token kernel (slot-2, plain basis, m = 1)
  int32_t slices;     // single-token kernel: K slices of 64 chunks = waves per workgroup
  int32_t mfma;       // 1: base-3, on the matrix cores (gemv_mfma.hip)
  int32_t iter;       // rows per lane slot
  int32_t rows_per_block;
};

// Launch helpers implemented in the .hip files. They only queue work; all argument checks
// happen in tgs_host.cpp before they are called.
GemvPlan gemv_plan(int32_t layout, int64_t k, int64_t m, int32_t rotated);
// after the jobs of a launch are known: pick rows per workgroup from their total row count
void gemv_plan_set_rows(GemvPlan& p, int64_t total_rows);
hipError_t gemv_launch(const GemvPlan& plan, GemvArgs& args, int32_t blocks, hipStream_t stream);
// base-3 on the matrix cores: rows of y per workgroup for m tokens
int gemv_b3_mfma_rows(int32_t m);
hipError_t gemv_b3_mfma_launch(GemvArgs& args, int32_t blocks, int32_t m, bool rotated, hipStream_t stream);

hipError_t gemm_launch(int32_t layout, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x_bf16, int64_t m, float* y, hipStream_t stream);

hipError_t hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, const int8_t* signs, void* y,
                           int32_t y_dtype, hipStream_t stream);

}  // namespace tgs
