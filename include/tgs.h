/*
 * tgs.h — C ABI of the ternary group-scaled matmul library for AMD Instinct MI355X (gfx950).
 *
 * The library multiplies activations by weights w = s_g * t, where each code t is -1, 0 or +1
 * and every group of 128 consecutive weights along K shares one fp16 scale s_g. The weights stay
 * packed in device memory and are decoded inside the kernels; no fp16 copy of W is ever made.
 *
 * Page references (titles as given by the sites):
 *   [P3] "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)", discuss.pytorch.kr
 *   [P2] "Bonsai 27B and how 1-bit survives", velog.io
 *   [P1] "Fine-tuning the ternary Bonsai-8B on Metal", molayo1419.me
 *
 * Conventions for every entry point:
 *   - Every call returns a tgs_status. Nothing is thrown across the ABI. After a failure,
 *     tgs_last_error() returns a message for the calling thread.
 *   - The caller owns every buffer it passes in. Pointers documented as "device" must be
 *     device memory of the current HIP device; "host" pointers must be host memory.
 *   - Arguments are checked on the host before any device work is queued. A rejected call
 *     queues nothing and leaves every output untouched.
 *   - Device calls run asynchronously on the given HIP stream (NULL = the default stream).
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - All calls are thread-safe. The library allocates no device memory and keeps no state
 *     between calls.
 */
#ifndef TGS_H
#define TGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TGS_MAGIC 0x31534754u /* "TGS1" */
#define TGS_VERSION 1u
#define TGS_GROUP 128          /* weights per fp16 scale, along K */
#define TGS_MAX_M_GEMV 8       /* activation rows accepted by ternary_gemv */
#define TGS_MAX_BATCH 32       /* matrices per ternary_gemv_batched call */

typedef enum {
  TGS_OK = 0,
  TGS_E_NULL = 1,     /* a required pointer is NULL */
  TGS_E_SHAPE = 2,    /* K % 128 != 0, N < 1, M out of range, row stride too small ... */
  TGS_E_ALIGN = 3,    /* a buffer is not aligned as documented */
  TGS_E_CODE = 4,     /* invalid code: trit outside {-1,0,1}, slot value 3, base-3 byte > 242,
                         non-canonical padding (host arrays only: device signs are not read) */
  TGS_E_LAYOUT = 5,   /* bad descriptor magic/version, unknown layout or rotation block */
  TGS_E_BASIS = 6,    /* weights in the rotated basis without signs, or signs for plain weights */
  TGS_E_SIZE = 7,     /* an output buffer is too small */
  TGS_E_DTYPE = 8,    /* unsupported activation/output dtype for this call */
  TGS_E_DEVICE = 9    /* a HIP runtime call failed */
} tgs_status;

/*
 * Packed layouts. [P3] section "Two packings: PTQ1_0 and PQ2_0" describes one layout with each
 * ternary value in its own 2-bit slot (scale plus codes = 34 bytes per 128 weights) and one that
 * packs ternary values densely. The pages fix neither bit order; these are the library's:
 *
 * TGS_LAYOUT_SLOT2: code q = t + 1 (0 -> -1, 1 -> 0, 2 -> +1; 3 is invalid). Element k of a row is
 *   held in bits 2*(k%4) and 2*(k%4)+1 of byte k/4, so a little-endian 32-bit word holds 16
 *   consecutive codes, element j in bits 2j..2j+1. Minimum row length K/4 bytes.
 * TGS_LAYOUT_BASE3: five trits per byte: byte b of a row = sum_{j<5} (t[5b+j] + 1) * 3^j, so
 *   valid bytes are 0..242. Positions past K in the last used byte hold t = 0. A row holds
 *   ceil(K/5) bytes followed by pad bytes of value 121 (five zero trits) up to a multiple of
 *   16 bytes: minimum row length round_up(ceil(K/5), 16) bytes.
 *
 * TGS_LAYOUT_BINARY: the two-level sibling format, t in {-1, +1} ([P2] "What ternary and binary
 *   are": two levels, 1.125 bits per weight with the group scales). One bit per weight: element
 *   k of a row is bit k%8 of byte k/8, set for t = +1 and clear for t = -1 (t = 0 cannot be
 *   stored). Minimum row length K/8 bytes; every byte is valid.
 *
 * All layouts keep the scales in a separate fp16 array [N][K/128], row-major, one per group of
 * 128 consecutive weights of a row ([P3] "Group-scaled ternary format": w_i = s_g * t_i with one
 * FP16 scale per 128 weights; [P2] "What the format is").
 */
typedef enum { TGS_LAYOUT_SLOT2 = 1, TGS_LAYOUT_BASE3 = 2, TGS_LAYOUT_BINARY = 3 } tgs_layout;

/* Activation / output element types (IEEE binary16, bfloat16, binary32). */
typedef enum { TGS_F16 = 1, TGS_BF16 = 2, TGS_F32 = 3 } tgs_dtype;

/*
 * A packed weight matrix W [n][k] (n output features, k input features).
 *   magic, version  TGS_MAGIC, TGS_VERSION (tgs_matrix_init fills them)
 *   layout          a tgs_layout
 *   rotated         0: plain basis. 1 or 1024: the codes are weights of the rotated basis, so the
 *                   layer computes y = W (R x), R = blockdiag_n((1/sqrt(n)) H_n S) with H_n the
 *                   natural-order Sylvester Hadamard matrix and S = diag(signs) ([P3] section
 *                   "Block-wise Hadamard rotation": R = H_n S / sqrt(n), f(x) = W(Rx)). 1 means
 *                   n = 128, one rotation block per scale group; 1024 means n = 1024, the size that
 *                   section names (a block spans 8 scale groups; k % 1024 == 0). tgs_matrix_init
 *                   also accepts 128 and stores it as 1. The packed model declares its basis and
 *                   the runtime must either apply the transform or refuse ([P3], same section):
 *                   calls on rotated weights require signs, calls on plain weights reject them.
 *   n, k            n >= 1, k >= 128, k % 128 == 0
 *   code_row_stride bytes between consecutive rows of codes: a multiple of 16 and at least
 *                   tgs_code_row_bytes(layout, k)
 *   codes           [n][code_row_stride] bytes, 16-byte aligned
 *   scales          [n][k/128] fp16 bit patterns, 2-byte aligned. Any fp16 value is accepted;
 *                   NaN and Inf propagate.
 */
typedef struct tgs_matrix {
  uint32_t magic;
  uint32_t version;
  int32_t layout;
  int32_t rotated;
  int64_t n;
  int64_t k;
  int64_t code_row_stride;
  const void* codes;
  const uint16_t* scales;
} tgs_matrix;

/* Minimum bytes per row of codes for the layout, or 0 if layout/k is invalid. */
size_t tgs_code_row_bytes(int32_t layout, int64_t k);

/* Fill a descriptor with magic/version and the minimum row stride. Returns TGS_E_SHAPE for an
 * invalid shape and TGS_E_LAYOUT for an unknown layout or a `rotated` value other than 0, 1, 128
 * and 1024, the same status every device call returns for such a descriptor (the descriptor is
 * then left zeroed). */
tgs_status tgs_matrix_init(tgs_matrix* w, int32_t layout, int32_t rotated, int64_t n, int64_t k,
                           const void* codes, const uint16_t* scales);

/*
 * pack_ternary (host): encode trits into the packed layout.
 *   trits      host [n][k] int8 in {-1, 0, +1} ({-1, +1} for TGS_LAYOUT_BINARY)
 *   scales     host [n][k/128] fp16 bits, copied to scales_out (both may be NULL to skip)
 *   codes_out  host buffer of codes_bytes >= n * tgs_code_row_bytes(layout, k); rows are
 *              written at the minimum stride
 * A native-ternary checkpoint is exactly scale x {-1, 0, +1}, so this re-encoding is lossless
 * ([P1] opening section on what these models are); unpack_ternary inverts it bit-exactly.
 * Returns TGS_E_CODE for a trit outside {-1, 0, +1} (or a 0 for the binary layout); codes_out may
 * then be partly written.
 */
tgs_status pack_ternary(int32_t layout, const int8_t* trits, const uint16_t* scales, int64_t n,
                        int64_t k, void* codes_out, size_t codes_bytes, uint16_t* scales_out);

/*
 * unpack_ternary (host): decode a host-resident packed matrix back to trits (and copy its
 * scales): the exact inverse of pack_ternary for either packing of [P3] "Two packings: PTQ1_0 and
 * PQ2_0" (and the binary layout), so a native-ternary checkpoint survives the round trip bit for
 * bit ([P1] opening section: re-encoding such a checkpoint is lossless). Every byte is checked:
 * slot value 3, base-3 bytes above 242, nonzero trits past K and pad bytes other than 121 give
 * TGS_E_CODE. trits_out is [n][k] int8; scales_out may be NULL.
 */
tgs_status unpack_ternary(const tgs_matrix* w, int8_t* trits_out, uint16_t* scales_out);

/*
 * ternary_gemv (device): y[i][j] = sum_k s[j][k/128] * t[j][k] * xr[i][k] for i < m, j < n,
 * with xr = x, or xr = R x when w->rotated (the rotation, with the descriptor's block size, is
 * computed inside the kernel). The weight of row j, column k is w = s_g * t with one fp16 scale
 * per 128-weight group ([P3] "Group-scaled ternary format"; [P2] "What the format is"); rotated
 * codes are weights of the basis R x ([P3] "Block-wise Hadamard rotation": the layer computes
 * W (R x)). The packed codes are read as they are, never expanded in memory ([P3] "Low-bit
 * kernels for hybrid attention": the kernels consume the packed weights directly).
 *   w       descriptor (host memory) of device-resident codes and scales
 *   x       device [m][k] activations of x_dtype; only TGS_F16 is accepted; 16-byte aligned
 *   m       1 .. TGS_MAX_M_GEMV (decode, or a small verify batch)
 *   signs   device [k] int8 in {-1, +1}, 16-byte aligned, when w->rotated, else NULL. The values
 *           live in device memory and are not read by the host (checking them would take a
 *           synchronous copy on every call); another value v multiplies its activation by v.
 *   y       device [m][n] fp32, 4-byte aligned
 *   stream  hipStream_t or NULL
 * Arithmetic: codes are decoded in registers; each 128-group is accumulated in fp32 and scaled
 * by its fp16 scale in fp32. Rotated activations are rounded once to fp16 after the transform,
 * so |R x| must stay below 65504. Results are deterministic run to run (no float atomics).
 * Rotated weights: the rotation is fused, and every workgroup that reads a group of K rotates it
 * again. A caller with a buffer for R x can instead rotate once with hadamard_rotate (fp16
 * output, the same rounding) and multiply with a plain-basis descriptor (rotated = 0) of the same
 * codes and scales; for several tokens that is the faster schedule.
 * Device limits (all device calls): n, k and the row stride below 2^24, and n * row stride at
 * most 2^31 - 2^20 bytes; larger matrices give TGS_E_SHAPE.
 */
tgs_status ternary_gemv(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m,
                        const int8_t* signs, float* y, void* stream);

/*
 * ternary_gemv_batched (device): count independent ternary_gemv calls (1..TGS_MAX_BATCH) that
 * share m and x_dtype, issued as few kernel launches as possible. ws is a host array of count
 * descriptors; xs, signs and ys are host arrays of count device pointers (signs may be NULL if
 * no matrix is rotated). Matrices may share an input (e.g. the q/k/v projections of one token).
 * Same rules and errors as ternary_gemv; all descriptors are checked before anything is queued.
 */
tgs_status ternary_gemv_batched(const tgs_matrix* ws, int32_t count, const void* const* xs,
                                int32_t x_dtype, int64_t m, const int8_t* const* signs,
                                float* const* ys, void* stream);

/*
 * ternary_gemm (device): the same product for m >= 1 rows of activations (prefill). The codes
 * are decoded tile by tile into LDS as bf16 and multiplied on the matrix cores (MFMA) with fp32
 * accumulation; each 128-group's partial product is scaled by its fp16 scale in fp32 ([P3]
 * section "Low-bit kernels for hybrid attention": unpack and group scale fused into the GEMM).
 *   x       device [m][k], TGS_BF16 only, 16-byte aligned; k at most 8384512 (the kernels address
 *           128 activation rows with 32-bit byte offsets), else TGS_E_SHAPE
 *   signs   must be NULL: this product is provided for plain-basis weights only, and rotated
 *           weights are refused with TGS_E_BASIS rather than multiplied in the wrong basis
 *   y       device [m][n] fp32, 4-byte aligned
 * Rotated weights (prefill): rotate the activations once with hadamard_rotate or
 * rmsnorm_hadamard_rotate into a bf16 buffer (y_dtype TGS_BF16) and multiply that buffer with a
 * plain-basis descriptor (rotated = 0) of the same codes and scales. That is the product of
 * bf16(R x): every rotated activation is rounded once to bf16 (unit roundoff 2^-8), so against
 * the unrounded rotation the result holds |y - y_exact| <= (2^-8 + 1e-3 (1 + 2^-8)) B + 1e-6
 * with B = sum |s t (R x)|, not the 1e-3 B + 1e-6 of the fused single-token route.
 */
tgs_status ternary_gemm(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m,
                        const int8_t* signs, float* y, void* stream);

/*
 * ternary_gemm_ws (device): ternary_gemm with a workspace, which lets a launch that would leave
 * compute units idle (few output tiles over a long K: e.g. the 5120 x 17408 down projection at
 * m <= 128) split K across workgroups: part p of P walks the 128-groups [p G / P, (p+1) G / P),
 * part 0 writes y, every other part writes its own [m][n] fp32 slice of the workspace, and a
 * second kernel on `stream` adds the parts into y in part order (deterministic: fixed order, no
 * atomics; the sum differs from ternary_gemm's only by fp32 rounding order). Nothing is allocated.
 *   w, x, x_dtype, m, signs, y, stream   as for ternary_gemm (same checks, same statuses)
 *   workspace        device memory, 4-byte aligned, not overlapping x or y, or NULL: then this is
 *                    ternary_gemm
 *   workspace_bytes  its size; below ternary_gemm_workspace_size(w, m) (and workspace not NULL):
 *                    TGS_E_SIZE
 * The workspace holds no state between calls; calls that overlap in time (different streams)
 * need workspaces of their own.
 */
tgs_status ternary_gemm_ws(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m,
                           const int8_t* signs, float* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * ternary_gemm_workspace_size (host): the bytes of workspace ternary_gemm_ws uses for this matrix
 * and m (0: that product is not split and needs none). Depends on w's layout, n and k, on m, and
 * on the current device's compute-unit count (256 when no device is visible), as the launch plan
 * does. Returns 0 for a descriptor that ternary_gemm would refuse, or m < 1.
 */
size_t ternary_gemm_workspace_size(const tgs_matrix* w, int64_t m);

/*
 * hadamard_rotate_g128 (device): y[i][b*128 + r] = (1/sqrt(128)) * sum_c H[r][c] * signs[b*128+c]
 * * x[i][b*128+c] for every row i < m and 128-block b: the block rotation R of [P3] "Block-wise
 * Hadamard rotation" with n = 128 and H the natural-order Sylvester matrix, signs applied first.
 *   x        device [m][k], x_dtype TGS_F16, TGS_BF16 or TGS_F32; 16-byte aligned
 *   k        multiple of 128
 *   signs    device [k] int8 in {-1, +1}, 16-byte aligned
 *   y        device [m][k], y_dtype TGS_F16, TGS_BF16 or TGS_F32; 16-byte aligned; must not
 *            overlap x
 * Computed in fp32 with a fast Walsh-Hadamard butterfly; fp16 and bf16 output is rounded once
 * from fp32, to nearest with ties to even.
 */
tgs_status hadamard_rotate_g128(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                const int8_t* signs, void* y, int32_t y_dtype, void* stream);

/*
 * ternary_code_flips (device): how many weights changed code between two packed matrices of the
 * same layout, shape and basis, per row and in total. A code flip is a weight whose ternary code
 * changes between checkpoints, e.g. 0 -> +1 or +1 -> -1: the only way training changes what a
 * native-ternary model computes, as opposed to nudging the shared scales ([P1] opening section;
 * its closing advice is to record the flips of every checkpoint).
 *   a, b        descriptors (host memory) of device-resident codes: same layout, rotated, n and k;
 *               the row strides may differ. Scales are not read.
 *   row_counts  device [n] uint32, 4-byte aligned, or NULL: flips of each row
 *   total       device uint64, 8-byte aligned, or NULL: flips of the whole matrix
 *               (at least one of row_counts and total is required)
 * The codes must be valid (unpack_ternary would accept them): pad trits and pad bytes are
 * compared as stored, and are equal in valid matrices. Counts are exact integers, identical run
 * to run. Both code planes are read once (the call is bound by HBM bandwidth for slot-2).
 */
tgs_status ternary_code_flips(const tgs_matrix* a, const tgs_matrix* b, uint32_t* row_counts, uint64_t* total,
                              void* stream);

/*
 * ternary_code_flips_batched (device): count pairs (1..TGS_MAX_BATCH) of one layout in one
 * launch (plus a small one that clears the totals). as and bs are host arrays of count
 * descriptors; row_counts and totals are host arrays of count device pointers (either array,
 * or entries of it, may be NULL as above, but every pair needs one of the two).
 */
tgs_status ternary_code_flips_batched(const tgs_matrix* as, const tgs_matrix* bs, int32_t count,
                                      uint32_t* const* row_counts, uint64_t* const* totals, void* stream);

/*
 * hadamard_rotate (device): the same rotation for blocks of `block` elements, 128 or 1024 (k a
 * multiple of block; [P3] "Block-wise Hadamard rotation" names n = 1024). Same arguments and
 * rules as hadamard_rotate_g128, which is this call with block = 128.
 */
tgs_status hadamard_rotate(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                           const int8_t* signs, void* y, int32_t y_dtype, void* stream);

/*
 * ternary_gemv_rmsnorm (device): ternary_gemv of the RMS-normalised activation,
 *   y[i][j] = sum_k s[j][k/128] * t[j][k] * xr[i][k],   xr = R xhat (rotated weights) or xhat,
 *   xhat[i][k] = gamma[k] * x[i][k] / sqrt((1/K) sum_c x[i][c]^2 + eps).
 * [P3] section "Running in the browser with WebGPU": the BlockHadamard operation has a variant
 * fused with RMSNorm; section "The 0.0976% kept at high precision": the norm weights
 * (input/post-attention layernorm) stay in bf16, neither rotated nor quantised. The pages do not
 * write the norm out; this is the usual root-mean-square normalisation over each row.
 *   gamma   device [k] bf16 bit patterns, 16-byte aligned
 *   eps     > 0 and finite, else TGS_E_SHAPE
 *   other arguments, rules and errors as ternary_gemv.
 * Each workgroup computes the rows' sums of squares itself (fp32, fixed order, so results stay
 * identical run to run); xhat (rotated or not) is rounded once to fp16.
 */
tgs_status ternary_gemv_rmsnorm(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m,
                                const uint16_t* gamma, float eps, const int8_t* signs, float* y,
                                void* stream);

/*
 * ternary_gemv_rmsnorm_batched (device): count ternary_gemv_rmsnorm calls sharing m, x_dtype and
 * eps, as in ternary_gemv_batched; gammas is a host array of count device pointers (none NULL).
 */
tgs_status ternary_gemv_rmsnorm_batched(const tgs_matrix* ws, int32_t count, const void* const* xs,
                                        int32_t x_dtype, int64_t m, const uint16_t* const* gammas,
                                        float eps, const int8_t* const* signs, float* const* ys,
                                        void* stream);

/*
 * rmsnorm_hadamard_rotate (device): y = R xhat with xhat the RMSNorm of each row of x as in
 * ternary_gemv_rmsnorm and R the block rotation of hadamard_rotate: the BlockHadamard variant
 * fused with RMSNorm of [P3] "Running in the browser with WebGPU".
 *   gamma   device [k] bf16 bit patterns, 16-byte aligned
 *   eps     > 0 and finite
 *   k       a multiple of block below 2^24; m below 2^31
 *   other arguments and rules as hadamard_rotate. One workgroup per row.
 */
tgs_status rmsnorm_hadamard_rotate(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                                   const uint16_t* gamma, float eps, const int8_t* signs, void* y,
                                   int32_t y_dtype, void* stream);

/*
 * ternary_gemv_chain (device): up to TGS_CHAIN_MAX_STEPS single-token GEMV steps run in order by
 * one launch. Step s computes, for each of its matrices i,
 *   y_i[j] = sum_k s_i[j][k/128] * t_i[j][k] * xh[k],
 * where xh is the step's input x in fp16 (an fp32 input is rounded to fp16, to nearest even),
 * RMS-normalised first when norm is set (xh <- gamma * xh / sqrt(mean xh^2 + eps), as in
 * ternary_gemv_rmsnorm): exactly what ternary_gemv (or ternary_gemv_rmsnorm) computes on that
 * fp16 vector ([P3] "Group-scaled ternary format"). Step s multiplies only after step s - 1 is
 * complete, so a step may read the output of any earlier step (an fp32 y, converted on the way in):
 * the steps of a decode pass in layer order ([P3] "Throughput: the two packings swap order by
 * hardware": batch-1 decode pays for every launch). The weights of step s are read while the
 * launch waits for step s - 1.
 *   steps      host array of count step descriptors (1 <= count <= TGS_CHAIN_MAX_STEPS)
 *     .count   matrices sharing the step's input, 1..TGS_CHAIN_MAX_MATRICES
 *     .x_dtype TGS_F16 or TGS_F32; .x device [k], 16-byte aligned
 *     .norm    0 or 1; with 1, .gamma device [k] bf16 bits (16-byte aligned) and .eps > 0, finite
 *     .w[i]    descriptors of device matrices: TGS_LAYOUT_SLOT2, plain basis, one k per step with
 *              k % 512 == 0 and k <= 16384; at most 16 * 16 * (compute units) rows in a step
 *     .y[i]    device [n_i] fp32, 4-byte aligned; must not overlap any step's input or weights
 *   workspace  device uint32 [tgs_chain_workspace_bytes() / 4], 4-byte aligned, zero-filled by the
 *              caller before its first use. A chain leaves it consistent for the next chain on the
 *              same device (its words count completed steps); it must be zero-filled again after a
 *              call whose error word (the last word) came back nonzero. Calls that use one
 *              workspace must not run concurrently.
 * The launch needs every compute unit (one workgroup each). Each wait between steps is bounded:
 * if the workgroups cannot all run at once (another kernel holds compute units), the waits give
 * up, the outputs are garbage and the workspace's last word becomes nonzero.
 */
#define TGS_CHAIN_MAX_STEPS 16
#define TGS_CHAIN_MAX_MATRICES 3
typedef struct tgs_chain_step {
  int32_t count;
  int32_t x_dtype;
  int32_t norm;
  float eps;
  const void* x;
  const uint16_t* gamma;
  tgs_matrix w[TGS_CHAIN_MAX_MATRICES];
  float* y[TGS_CHAIN_MAX_MATRICES];
} tgs_chain_step;

/* Bytes of the chain workspace on the current device (0 if no device is usable). */
size_t tgs_chain_workspace_bytes(void);
tgs_status ternary_gemv_chain(const tgs_chain_step* steps, int32_t count, uint32_t* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * ternary_gemv_chain_static (device): ternary_gemv_chain without a workspace argument, for callers
 * that cannot allocate device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation). It allocates and frees nothing. Its workspace is an array owned by the
 * library, one per device (4 * 1025 bytes, held until the process ends); a device whose chain grid
 * needs more than 1025 words (more than 1024 compute units) is refused with TGS_E_SIZE. Each call
 * zero-fills that array on `stream` (a small fill kernel) before the chain, so no call depends on
 * an earlier one. Calls that overlap on one device (on different streams, or from different
 * threads) share the array and race: their results are undefined.
 *   steps, count, stream   as for ternary_gemv_chain (same checks, same statuses)
 *   error   NULL, or a device uint32, 4-byte aligned: after the chain, stream-ordered, it receives
 *           the chain's error word (0: every wait between steps completed; nonzero: a wait gave
 *           up and the outputs are garbage)
 */
tgs_status ternary_gemv_chain_static(const tgs_chain_step* steps, int32_t count, uint32_t* error, void* stream);

/*
 * Measurement helpers (not part of the product; for measuring the rooflines the kernels are
 * compared with).
 *
 * tgs_stream_read (device): read `bytes` of device memory once, as the plainest streaming kernel
 * can (16-byte non-temporal loads over the whole GPU), folding the data into one word per thread,
 * written to sink. Timing it on a buffer far larger than the last-level cache gives the read
 * bandwidth a kernel can actually reach, next to the nominal HBM peak.
 *   buf    device, 16-byte aligned; bytes a positive multiple of 16
 *   sink   device uint32 [tgs_stream_read_sink_words()], 4-byte aligned; its contents are not
 *          meaningful
 */
size_t tgs_stream_read_sink_words(void);
tgs_status tgs_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* tgs_status_string(tgs_status status);

/* Message describing the last failed call on this thread ("" if none). */
const char* tgs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TGS_H */
