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
// and, with 64 lanes per row and one K slice, this many row waves share the activations, in
// launches of up to kWaveKernelShareRows rows
constexpr int kWaveKernelRowWaves = 4;
constexpr int64_t kWaveKernelShareRows = 65536;

// One matrix of a batched GEMV launch. All pointers are device pointers.
struct GemvJob {
  const uint8_t* codes;    // [n][stride]
  const uint16_t* scales;  // [n][k/128] fp16 bits
  const uint16_t* x;       // [m][k] fp16 bits
  const int8_t* signs;     // [k] or nullptr (plain basis)
  const uint16_t* gamma;   // [k] bf16 bits of the RMSNorm weight, or nullptr (no norm)
  float* y;                // [m][n]
  int64_t stride;          // bytes between rows of codes
  int32_t n;
  int32_t k;
  int32_t block0;          // first workgroup of this job in the launch
  int32_t row_blocks;      // workgroups for this job
};

// Kernel argument block of a batched GEMV launch. The header comes first so that a wave can read
// it, the start table and job 0 in one batch of scalar loads; only a workgroup of a later job
// waits for a second load (its job's fields).
struct GemvArgs {
  int32_t count;
  int32_t m;
  int32_t rows_per_wave;     // single-token kernel only
  int32_t norm;              // 1: RMS-normalise x with each job's gamma first (the jobs' gammas are set)
  float eps;                 // the norm's epsilon
  int32_t reserved;
  int32_t start[kMaxJobs];   // == job[i].block0 for i < count; INT32_MAX past the last job
  GemvJob job[kMaxJobs];
};

// The job of this workgroup: the last one whose first workgroup is at or before blockIdx.x.
// m_out, rpw_out (optional): the header's m and rows_per_wave, taken from the same batch (asm
// outputs, so that the compiler keeps them in registers rather than loading them again later)
__device__ __forceinline__ GemvJob gemv_job_of_block(const GemvArgs& a, int* m_out = nullptr, int* rpw_out = nullptr) {
  const int b = (int)blockIdx.x;
  GemvJob job = a.job[0];
  // job 0, the job count and the header in one batch of scalar loads (job 0 not as a select of
  // two addresses); a launch of one job, as every launch in layer order is, needs nothing else
  const int32_t count = a.count;
  int32_t m = a.m, rpw = a.rows_per_wave;
  __asm__ volatile("" : "+s"(m), "+s"(rpw) : "s"(count), "s"(job.codes), "s"(job.scales), "s"(job.x), "s"(job.signs),
                   "s"(job.y), "s"(job.stride), "s"(job.n), "s"(job.k), "s"(job.block0));
  if (m_out) *m_out = m;
  if (rpw_out) *rpw_out = rpw;
  if (count == 1) return job;
  // starts increase and are >= 1 past job 0: start - 1 - b is negative exactly when b >= start
  int32_t st[kMaxJobs];
#pragma unroll
  for (int i = 1; i < kMaxJobs; ++i) st[i] = a.start[i];
  // the whole table, and the header, in the same batch of loads
  __asm__ volatile("" ::"s"(a.m), "s"(a.rows_per_wave), "s"(st[1]), "s"(st[2]), "s"(st[3]), "s"(st[4]), "s"(st[5]),
                   "s"(st[6]), "s"(st[7]), "s"(st[8]), "s"(st[9]), "s"(st[10]), "s"(st[11]), "s"(st[12]), "s"(st[13]),
                   "s"(st[14]), "s"(st[15]), "s"(st[16]));
  __asm__ volatile("" ::"s"(st[17]), "s"(st[18]), "s"(st[19]), "s"(st[20]), "s"(st[21]), "s"(st[22]), "s"(st[23]),
                   "s"(st[24]), "s"(st[25]), "s"(st[26]), "s"(st[27]), "s"(st[28]), "s"(st[29]), "s"(st[30]),
                   "s"(st[31]));
  uint32_t j = 0;
#pragma unroll
  for (int i = 1; i < kMaxJobs; ++i) j += (uint32_t)(st[i] - 1 - b) >> 31;
  if (j != 0) job = a.job[j];
  return job;
}

// Shape class of a GEMV launch: every job in one launch shares these.
struct GemvPlan {
  int32_t layout;     // TGS_LAYOUT_*
  int32_t lanes;      // lanes per row (16, 32 or 64)
  int32_t m;          // activation rows
  int32_t rotated;    // 0 (plain), 1 (128-element rotation blocks) or 1024
  int32_t stream;     // 1: the single-token kernel (slot-2, plain basis, m = 1)
  int32_t slices;     // single-token kernel: K slices of 64 chunks = waves per workgroup
  int32_t mfma;       // 1: base-3, on the matrix cores (gemv_mfma.hip); 2: single-token slot-2 on the
                      // matrix cores (gemv_s2_mfma.hip)
  int32_t iter;       // rows per lane slot
  int32_t rows_per_block;
  int32_t norm;       // 1: RMSNorm prologue
  int32_t row_waves;  // single-token kernel: waves per K slice sharing the activations
};

// Launch helpers implemented in the .hip files. They only queue work; all argument checks
// happen in tgs_host.cpp before they are called.
GemvPlan gemv_plan(int32_t layout, int64_t k, int64_t m, int32_t rotated, bool norm = false);
// after the jobs of a launch are known: pick rows per workgroup from their total row count
void gemv_plan_set_rows(GemvPlan& p, int64_t total_rows);
hipError_t gemv_launch(const GemvPlan& plan, GemvArgs& args, int32_t blocks, hipStream_t stream);
// single-token slot-2 on the matrix cores: whether K fits (a multiple of 512, at most 16384), waves
// per workgroup for K, and the launch (16 rows per workgroup; LDS sized for the largest K of the jobs)
bool gemv_s2_mfma_fits(int64_t k);
int gemv_s2_mfma_waves(int64_t k);
hipError_t gemv_s2_mfma_launch(GemvArgs& args, int32_t blocks, int64_t max_k, bool norm, hipStream_t stream);
// base-3 on the matrix cores: rows of y per workgroup for m tokens
int gemv_b3_mfma_rows(int32_t m);
// block: 0 for plain-basis weights, else the rotation block (128 or 1024)
hipError_t gemv_b3_mfma_launch(GemvArgs& args, int32_t blocks, int32_t m, int32_t block, bool norm,
                               hipStream_t stream);

// GEMV step chain (gemv_chain.hip): up to kChainMaxSteps single-token slot-2 steps in one launch,
// run in order with a wait between consecutive steps. Device pointers throughout.
constexpr int kChainMaxSteps = 16;
constexpr int kChainMaxMats = 3;
struct ChainMat {
  const uint8_t* codes;    // [n][stride]
  const uint16_t* scales;  // [n][k/128] fp16 bits
  float* y;                // [n]
  int32_t n;
  int32_t stride;
  int32_t rb0;             // first 16-row block of this matrix in the step's numbering
  int32_t reserved;
};
struct ChainStep {
  const void* x;           // [k] fp16, or fp32 (x_f32) rounded to fp16 when staged
  const uint16_t* gamma;   // [k] bf16 bits when norm
  ChainMat mat[kChainMaxMats];
  int32_t k;
  int32_t count;           // matrices of the step
  int32_t x_f32;
  int32_t norm;
  int32_t rbs;             // 16-row blocks of the step, all matrices
  float eps;
};
struct ChainArgs {
  uint32_t* flags;         // workspace: [grid] completed-step counts, then one error word
  int32_t count;
  int32_t reserved;
  ChainStep step[kChainMaxSteps];
};
// workgroups of a chain launch on the current device (one per compute unit), or -1
int chain_grid();
// 16-row blocks one workgroup may own in a step
constexpr int kChainMaxRbsPerWg = 16;
hipError_t chain_launch(const ChainArgs& args, int32_t grid, hipStream_t stream);
// The library-owned chain workspace of the current device (kChainStaticWords words, found once
// per device), for the entry point that allocates nothing; chain_clear zero-fills words of it.
constexpr int kChainStaticMaxGrid = 1024;
constexpr int kChainStaticWords = kChainStaticMaxGrid + 1;
hipError_t chain_static_workspace(uint32_t** ptr);
hipError_t chain_clear(uint32_t* words, int32_t count, hipStream_t stream);

// Code flips: one pair of matrices of a batched launch (device pointers).
struct FlipJob {
  const uint8_t* a;
  const uint8_t* b;
  uint32_t* rows;   // [n] or nullptr
  uint64_t* total;  // one counter or nullptr
  int64_t stride_a;
  int64_t stride_b;
  int32_t n;
  int32_t row_bytes;  // minimum row length of the layout: the bytes compared
  int32_t block0;     // first workgroup of this pair in the launch
  int32_t reserved;
};

struct FlipArgs {
  FlipJob job[kMaxJobs];
  int32_t count;
  int32_t layout;
};

int code_flip_rows_per_block();
hipError_t code_flip_launch(FlipArgs& args, int32_t blocks, hipStream_t stream);

// ws: NULL (no K split across workgroups), or gemm_workspace_bytes of device memory
hipError_t gemm_launch(int32_t layout, const uint8_t* codes, int64_t stride, const uint16_t* scales, int64_t n, int64_t k,
                       const uint16_t* x_bf16, int64_t m, float* y, float* ws, hipStream_t stream);
size_t gemm_workspace_bytes(int32_t layout, int64_t n, int64_t k, int64_t m);

hipError_t hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block, const int8_t* signs,
                           void* y, int32_t y_dtype, hipStream_t stream);
// the same rotation after RMSNorm of each row (gamma: bf16 bits [k]); one workgroup per row
hipError_t rmsnorm_hadamard_launch(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                                   const uint16_t* gamma, float eps, const int8_t* signs, void* y, int32_t y_dtype,
                                   hipStream_t stream);

// streaming-read probe: workgroups of 256 threads in the launch, and the launch
int stream_read_grid();
hipError_t stream_read_launch(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);

// rotation block of a descriptor's `rotated` field: 0 (plain basis), 128 or 1024
inline int64_t rotation_block(int32_t rotated) { return rotated == 0 ? 0 : (rotated == 1024 ? 1024 : 128); }

}  // namespace tgs
