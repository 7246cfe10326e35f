// Host side of the C ABI declared in include/tgs.h: packing, unpacking, argument checks and
// kernel dispatch. Everything here runs on the CPU; device work is only queued by the launch
// helpers of the .hip files, after every argument has been checked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "tgs.h"
#include "tgs_internal.h"

namespace {

thread_local std::string g_last_error;

tgs_status fail(tgs_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tgs_status ok() {
  g_last_error.clear();
  return TGS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t row_bytes(int32_t layout, int64_t k) {
  if (k < 128 || k % 128 != 0) return 0;
  if (layout == TGS_LAYOUT_SLOT2) return (size_t)(k / 4);
  if (layout == TGS_LAYOUT_BASE3) return (size_t)(((k + 4) / 5 + 15) / 16 * 16);
  if (layout == TGS_LAYOUT_BINARY) return (size_t)(k / 8);
  return 0;
}

bool valid_layout(int32_t layout) {
  return layout == TGS_LAYOUT_SLOT2 || layout == TGS_LAYOUT_BASE3 || layout == TGS_LAYOUT_BINARY;
}

// Run fn(row_begin, row_end) over [0, n) on up to 16 host threads.
template <class F>
void parallel_rows(int64_t n, int64_t work_per_row, F fn) {
  int64_t threads = (int64_t)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n * work_per_row < (1 << 20)) threads = 1;
  threads = std::min(threads, std::max<int64_t>(n, 1));
  if (threads <= 1) {
    fn((int64_t)0, n);
    return;
  }
  std::vector<std::thread> pool;
  const int64_t per = (n + threads - 1) / threads;
  for (int64_t t = 0; t < threads; ++t) {
    const int64_t b = t * per, e = std::min(n, b + per);
    if (b >= e) break;
    pool.emplace_back([=] { fn(b, e); });
  }
  for (auto& th : pool) th.join();
}

// ---- slot-2: 16 codes per 32-bit word, element j in bits 2j..2j+1, code q = t + 1 --------

bool pack_row_slot2(const int8_t* t, int64_t k, uint8_t* out) {
  for (int64_t c = 0; c < k; c += 16) {
    uint32_t word = 0;
    for (int j = 0; j < 16; ++j) {
      const int v = t[c + j];
      if (v < -1 || v > 1) return false;
      word |= (uint32_t)(v + 1) << (2 * j);
    }
    std::memcpy(out + c / 4, &word, 4);
  }
  return true;
}

bool unpack_row_slot2(const uint8_t* in, int64_t k, int8_t* t) {
  for (int64_t c = 0; c < k; c += 16) {
    uint32_t word;
    std::memcpy(&word, in + c / 4, 4);
    // a slot holding 3 has both bits set
    if (word & (word >> 1) & 0x55555555u) return false;
    for (int j = 0; j < 16; ++j) t[c + j] = (int8_t)((int)((word >> (2 * j)) & 3u) - 1);
  }
  return true;
}

// ---- binary: element j of a row in bit j%8 of byte j/8, set for +1 --------------------------

bool pack_row_binary(const int8_t* t, int64_t k, uint8_t* out) {
  for (int64_t c = 0; c < k; c += 8) {
    uint32_t byte = 0;
    for (int j = 0; j < 8; ++j) {
      const int v = t[c + j];
      if (v != 1 && v != -1) return false;
      byte |= (uint32_t)(v == 1) << j;
    }
    out[c / 8] = (uint8_t)byte;
  }
  return true;
}

void unpack_row_binary(const uint8_t* in, int64_t k, int8_t* t) {
  for (int64_t c = 0; c < k; ++c) t[c] = ((in[c / 8] >> (c % 8)) & 1) ? (int8_t)1 : (int8_t)-1;
}

// ---- base-3: byte b = sum_{j<5} (t[5b+j] + 1) * 3^j, pad bytes 121 -------------------------

bool pack_row_base3(const int8_t* t, int64_t k, size_t rb, uint8_t* out) {
  const int64_t used = (k + 4) / 5;
  for (int64_t b = 0; b < used; ++b) {
    int value = 0;
    for (int j = 4; j >= 0; --j) {
      const int64_t c = 5 * b + j;
      int digit = 1;
      if (c < k) {
        const int v = t[c];
        if (v < -1 || v > 1) return false;
        digit = v + 1;
      }
      value = value * 3 + digit;
    }
    out[b] = (uint8_t)value;
  }
  std::memset(out + used, 121, rb - (size_t)used);
  return true;
}

bool unpack_row_base3(const uint8_t* in, int64_t k, size_t rb, int8_t* t) {
  const int64_t used = (k + 4) / 5;
  for (int64_t b = 0; b < used; ++b) {
    int value = in[b];
    if (value > 242) return false;
    for (int j = 0; j < 5; ++j) {
      const int digit = value % 3;
      value /= 3;
      const int64_t c = 5 * b + j;
      if (c < k)
        t[c] = (int8_t)(digit - 1);
      else if (digit != 1)
        return false;
    }
  }
  for (size_t b = (size_t)used; b < rb; ++b)
    if (in[b] != 121) return false;
  return true;
}

// ---- descriptor checks -------------------------------------------------------------------

tgs_status check_matrix(const tgs_matrix* w, bool device) {
  if (!w) return fail(TGS_E_NULL, "matrix descriptor is NULL");
  if (w->magic != TGS_MAGIC || w->version != TGS_VERSION)
    return fail(TGS_E_LAYOUT, "bad descriptor magic/version (0x%08x, %u); use tgs_matrix_init", w->magic, w->version);
  if (!valid_layout(w->layout)) return fail(TGS_E_LAYOUT, "unknown layout %d", w->layout);
  if (w->rotated != 0 && w->rotated != 1 && w->rotated != 1024)
    return fail(TGS_E_LAYOUT, "rotated must be 0, 1 (128-element blocks) or 1024, got %d", w->rotated);
  if (w->n < 1 || w->k < 128 || w->k % 128 != 0)
    return fail(TGS_E_SHAPE, "need n >= 1 and k a positive multiple of 128 (n=%lld, k=%lld)", (long long)w->n,
                (long long)w->k);
  if (w->rotated == 1024 && w->k % 1024 != 0)
    return fail(TGS_E_SHAPE, "1024-element rotation blocks need k %% 1024 == 0 (k=%lld)", (long long)w->k);
  if (device && (w->n >= (1LL << 24) || w->k >= (1LL << 24) || w->code_row_stride >= (1LL << 24)))
    return fail(TGS_E_SHAPE, "n, k and the row stride must stay below 2^24 for the device kernels (n=%lld, k=%lld)",
                (long long)w->n, (long long)w->k);
  const size_t rb = row_bytes(w->layout, w->k);
  if (w->code_row_stride < (int64_t)rb || w->code_row_stride % 16 != 0)
    return fail(TGS_E_SHAPE, "code_row_stride %lld must be a multiple of 16 and >= %zu", (long long)w->code_row_stride,
                rb);
  if (device && w->n * w->code_row_stride > tgs::kMaxDeviceCodeBytes)
    return fail(TGS_E_SHAPE, "codes of one matrix must stay within 2 GiB - 1 MiB (n * code_row_stride = %lld)",
                (long long)(w->n * w->code_row_stride));
  if (!w->codes || !w->scales) return fail(TGS_E_NULL, "codes or scales pointer is NULL");
  if (!aligned(w->codes, 16)) return fail(TGS_E_ALIGN, "codes must be 16-byte aligned");
  if (!aligned(w->scales, 2)) return fail(TGS_E_ALIGN, "scales must be 2-byte aligned");
  return TGS_OK;
}

tgs_status check_basis(const tgs_matrix* w, const int8_t* signs) {
  if (w->rotated && !signs)
    return fail(TGS_E_BASIS, "weights are in the rotated basis: the sign vector of the rotation is required");
  if (!w->rotated && signs)
    return fail(TGS_E_BASIS, "signs given for weights in the plain basis; refusing to rotate the activations");
  return TGS_OK;
}

tgs_status device_error(hipError_t e, const char* what) {
  return fail(TGS_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t tgs_code_row_bytes(int32_t layout, int64_t k) { return row_bytes(layout, k); }

tgs_status tgs_matrix_init(tgs_matrix* w, int32_t layout, int32_t rotated, int64_t n, int64_t k, const void* codes,
                           const uint16_t* scales) {
  if (!w) return fail(TGS_E_NULL, "matrix descriptor is NULL");
  std::memset(w, 0, sizeof(*w));
  if (!valid_layout(layout)) return fail(TGS_E_LAYOUT, "unknown layout %d", layout);
  if (n < 1 || k < 128 || k % 128 != 0) return fail(TGS_E_SHAPE, "need n >= 1 and k a positive multiple of 128");
  if (rotated != 0 && rotated != 1 && rotated != 128 && rotated != 1024)
    return fail(TGS_E_LAYOUT, "rotated must be 0, 1 (128-element blocks), 128 or 1024, got %d", rotated);
  if (rotated == 1024 && k % 1024 != 0) return fail(TGS_E_SHAPE, "1024-element rotation blocks need k % 1024 == 0");
  // the descriptor is written only once every check has passed: a failed call leaves it zeroed
  w->magic = TGS_MAGIC;
  w->version = TGS_VERSION;
  w->layout = layout;
  w->rotated = rotated == 0 ? 0 : (rotated == 1024 ? 1024 : 1);
  w->n = n;
  w->k = k;
  w->code_row_stride = (int64_t)row_bytes(layout, k);
  w->codes = codes;
  w->scales = scales;
  return ok();
}

tgs_status pack_ternary(int32_t layout, const int8_t* trits, const uint16_t* scales, int64_t n, int64_t k,
                        void* codes_out, size_t codes_bytes, uint16_t* scales_out) {
  if (!valid_layout(layout)) return fail(TGS_E_LAYOUT, "unknown layout %d", layout);
  if (n < 1 || k < 128 || k % 128 != 0) return fail(TGS_E_SHAPE, "need n >= 1 and k a positive multiple of 128");
  if (!trits || !codes_out) return fail(TGS_E_NULL, "trits or codes_out is NULL");
  if ((scales == nullptr) != (scales_out == nullptr))
    return fail(TGS_E_NULL, "scales and scales_out must both be given or both be NULL");
  const size_t rb = row_bytes(layout, k);
  if (codes_bytes < rb * (size_t)n)
    return fail(TGS_E_SIZE, "codes_out holds %zu bytes, %zu needed", codes_bytes, rb * (size_t)n);
  uint8_t* out = static_cast<uint8_t*>(codes_out);
  std::vector<char> bad((size_t)n, 0);
  parallel_rows(n, k, [&](int64_t b, int64_t e) {
    for (int64_t r = b; r < e; ++r) {
      const int8_t* t = trits + r * k;
      uint8_t* o = out + (size_t)r * rb;
      bool good = layout == TGS_LAYOUT_SLOT2   ? pack_row_slot2(t, k, o)
                  : layout == TGS_LAYOUT_BASE3 ? pack_row_base3(t, k, rb, o)
                                               : pack_row_binary(t, k, o);
      if (!good) bad[(size_t)r] = 1;
    }
  });
  for (int64_t r = 0; r < n; ++r)
    if (bad[(size_t)r])
      return fail(TGS_E_CODE, "row %lld holds a value outside %s", (long long)r,
                  layout == TGS_LAYOUT_BINARY ? "{-1, +1}" : "{-1, 0, +1}");
  if (scales) std::memcpy(scales_out, scales, sizeof(uint16_t) * (size_t)n * (size_t)(k / 128));
  return ok();
}

tgs_status unpack_ternary(const tgs_matrix* w, int8_t* trits_out, uint16_t* scales_out) {
  tgs_status st = check_matrix(w, false);
  if (st != TGS_OK) return st;
  if (!trits_out) return fail(TGS_E_NULL, "trits_out is NULL");
  const size_t rb = row_bytes(w->layout, w->k);
  const uint8_t* in = static_cast<const uint8_t*>(w->codes);
  std::vector<char> bad((size_t)w->n, 0);
  parallel_rows(w->n, w->k, [&](int64_t b, int64_t e) {
    for (int64_t r = b; r < e; ++r) {
      const uint8_t* row = in + (size_t)r * (size_t)w->code_row_stride;
      int8_t* t = trits_out + r * w->k;
      bool good = true;
      if (w->layout == TGS_LAYOUT_SLOT2)
        good = unpack_row_slot2(row, w->k, t);
      else if (w->layout == TGS_LAYOUT_BASE3)
        good = unpack_row_base3(row, w->k, rb, t);
      else
        unpack_row_binary(row, w->k, t);  // every byte is valid
      if (!good) bad[(size_t)r] = 1;
    }
  });
  for (int64_t r = 0; r < w->n; ++r)
    if (bad[(size_t)r])
      return fail(TGS_E_CODE, "row %lld holds an invalid code (%s)", (long long)r,
                  w->layout == TGS_LAYOUT_SLOT2 ? "a 2-bit slot of value 3"
                                                : "a byte above 242, a nonzero trit past K or a pad byte other than 121");
  if (scales_out) std::memcpy(scales_out, w->scales, sizeof(uint16_t) * (size_t)w->n * (size_t)(w->k / 128));
  return ok();
}

namespace {

// The batched GEMV, with the RMSNorm prologue when gammas is set (one norm weight vector per matrix).
tgs_status gemv_batched(const tgs_matrix* ws, int32_t count, const void* const* xs, int32_t x_dtype, int64_t m,
                        const uint16_t* const* gammas, float eps, const int8_t* const* signs, float* const* ys,
                        void* stream) {
  if (!ws || !xs || !ys) return fail(TGS_E_NULL, "descriptor, input or output array is NULL");
  if (count < 1 || count > TGS_MAX_BATCH) return fail(TGS_E_SHAPE, "count must be 1..%d, got %d", TGS_MAX_BATCH, count);
  if (x_dtype != TGS_F16) return fail(TGS_E_DTYPE, "ternary_gemv takes fp16 activations (TGS_F16)");
  if (m < 1 || m > TGS_MAX_M_GEMV) return fail(TGS_E_SHAPE, "m must be 1..%d, got %lld", TGS_MAX_M_GEMV, (long long)m);
  for (int32_t i = 0; i < count; ++i) {
    tgs_status st = check_matrix(&ws[i], true);
    if (st != TGS_OK) return st;
    st = check_basis(&ws[i], signs ? signs[i] : nullptr);
    if (st != TGS_OK) return st;
    if (!xs[i] || !ys[i]) return fail(TGS_E_NULL, "input or output %d is NULL", i);
    if (!aligned(xs[i], 16)) return fail(TGS_E_ALIGN, "x must be 16-byte aligned");
    if (!aligned(ys[i], 4)) return fail(TGS_E_ALIGN, "y must be 4-byte aligned");
    if (signs && signs[i] && !aligned(signs[i], 16)) return fail(TGS_E_ALIGN, "signs must be 16-byte aligned");
    if (gammas) {
      if (!gammas[i]) return fail(TGS_E_NULL, "gamma %d is NULL", i);
      if (!aligned(gammas[i], 16)) return fail(TGS_E_ALIGN, "gamma must be 16-byte aligned");
    }
  }
  if (gammas && !(eps > 0.f && eps < INFINITY)) return fail(TGS_E_SHAPE, "eps must be positive and finite");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one launch per distinct plan (layout, lanes per row, basis, kernel, K slices), in call order
  std::vector<char> done((size_t)count, 0);
  for (int32_t i = 0; i < count; ++i) {
    if (done[(size_t)i]) continue;
    tgs::GemvPlan plan = tgs::gemv_plan(ws[i].layout, ws[i].k, m, ws[i].rotated, gammas != nullptr);
    // the jobs of this launch: every remaining matrix with the same plan, in call order
    std::vector<int32_t> members;
    int64_t total_rows = 0;
    for (int32_t j = i; j < count; ++j) {
      if (done[(size_t)j]) continue;
      const tgs::GemvPlan pj = tgs::gemv_plan(ws[j].layout, ws[j].k, m, ws[j].rotated, gammas != nullptr);
      if (pj.layout != plan.layout || pj.lanes != plan.lanes || pj.rotated != plan.rotated ||
          pj.stream != plan.stream || pj.slices != plan.slices || pj.mfma != plan.mfma)
        continue;
      members.push_back(j);
      total_rows += ws[j].n;
      done[(size_t)j] = 1;
    }
    tgs::gemv_plan_set_rows(plan, total_rows);
    tgs::GemvArgs args;
    std::memset(&args, 0, sizeof(args));
    args.m = (int32_t)m;
    args.norm = gammas ? 1 : 0;
    args.eps = eps;
    for (int32_t i = 0; i < tgs::kMaxJobs; ++i) args.start[i] = INT32_MAX;
    int32_t blocks = 0;
    for (int32_t j : members) {
      tgs::GemvJob& job = args.job[args.count++];
      job.codes = static_cast<const uint8_t*>(ws[j].codes);
      job.scales = ws[j].scales;
      job.x = static_cast<const uint16_t*>(xs[j]);
      job.signs = signs ? signs[j] : nullptr;
      job.gamma = gammas ? gammas[j] : nullptr;
      job.y = ys[j];
      job.stride = ws[j].code_row_stride;
      job.n = (int32_t)ws[j].n;
      job.k = (int32_t)ws[j].k;
      job.block0 = blocks;
      args.start[args.count - 1] = blocks;
      job.row_blocks = (int32_t)((ws[j].n + plan.rows_per_block - 1) / plan.rows_per_block);
      blocks += job.row_blocks;
    }
    hipError_t e = tgs::gemv_launch(plan, args, blocks, s);
    if (e != hipSuccess) return device_error(e, "ternary_gemv launch");
  }
  return ok();
}

}  // namespace

tgs_status ternary_gemv_batched(const tgs_matrix* ws, int32_t count, const void* const* xs, int32_t x_dtype,
                                int64_t m, const int8_t* const* signs, float* const* ys, void* stream) {
  return gemv_batched(ws, count, xs, x_dtype, m, nullptr, 0.f, signs, ys, stream);
}

tgs_status ternary_gemv_rmsnorm_batched(const tgs_matrix* ws, int32_t count, const void* const* xs, int32_t x_dtype,
                                        int64_t m, const uint16_t* const* gammas, float eps,
                                        const int8_t* const* signs, float* const* ys, void* stream) {
  if (!gammas) return fail(TGS_E_NULL, "gammas is NULL");
  return gemv_batched(ws, count, xs, x_dtype, m, gammas, eps, signs, ys, stream);
}

tgs_status ternary_gemv_rmsnorm(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m, const uint16_t* gamma,
                                float eps, const int8_t* signs, float* y, void* stream) {
  if (!w) return fail(TGS_E_NULL, "matrix descriptor is NULL");
  const void* xs[1] = {x};
  const uint16_t* gs[1] = {gamma};
  const int8_t* ss[1] = {signs};
  float* ys[1] = {y};
  return ternary_gemv_rmsnorm_batched(w, 1, xs, x_dtype, m, gs, eps, ss, ys, stream);
}

tgs_status ternary_code_flips_batched(const tgs_matrix* as, const tgs_matrix* bs, int32_t count,
                                     uint32_t* const* row_counts, uint64_t* const* totals, void* stream) {
  if (!as || !bs) return fail(TGS_E_NULL, "descriptor array is NULL");
  if (!row_counts && !totals) return fail(TGS_E_NULL, "neither per-row counts nor totals requested");
  if (count < 1 || count > TGS_MAX_BATCH) return fail(TGS_E_SHAPE, "count must be 1..%d, got %d", TGS_MAX_BATCH, count);
  for (int32_t i = 0; i < count; ++i) {
    tgs_status st = check_matrix(&as[i], true);
    if (st != TGS_OK) return st;
    st = check_matrix(&bs[i], true);
    if (st != TGS_OK) return st;
    if (as[i].layout != bs[i].layout || as[i].n != bs[i].n || as[i].k != bs[i].k)
      return fail(TGS_E_SHAPE, "pair %d: the two matrices differ in layout or shape", i);
    if (as[i].rotated != bs[i].rotated)
      return fail(TGS_E_BASIS, "pair %d: one matrix is in the rotated basis and the other is not", i);
    if (as[i].layout != as[0].layout) return fail(TGS_E_LAYOUT, "all pairs of one call must share a layout");
    uint32_t* rc = row_counts ? row_counts[i] : nullptr;
    uint64_t* tot = totals ? totals[i] : nullptr;
    if (!rc && !tot) return fail(TGS_E_NULL, "pair %d: neither a per-row count nor a total requested", i);
    if (rc && !aligned(rc, 4)) return fail(TGS_E_ALIGN, "row counts must be 4-byte aligned");
    if (tot && !aligned(tot, 8)) return fail(TGS_E_ALIGN, "totals must be 8-byte aligned");
  }
  tgs::FlipArgs args;
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  args.layout = as[0].layout;
  const int rows_per_block = tgs::code_flip_rows_per_block();
  int32_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    tgs::FlipJob& job = args.job[i];
    job.a = static_cast<const uint8_t*>(as[i].codes);
    job.b = static_cast<const uint8_t*>(bs[i].codes);
    job.rows = row_counts ? row_counts[i] : nullptr;
    job.total = totals ? totals[i] : nullptr;
    job.stride_a = as[i].code_row_stride;
    job.stride_b = bs[i].code_row_stride;
    job.n = (int32_t)as[i].n;
    job.row_bytes = (int32_t)row_bytes(as[i].layout, as[i].k);
    job.block0 = blocks;
    blocks += (int32_t)((as[i].n + rows_per_block - 1) / rows_per_block);
  }
  hipError_t e = tgs::code_flip_launch(args, blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "ternary_code_flips launch");
  return ok();
}

tgs_status ternary_code_flips(const tgs_matrix* a, const tgs_matrix* b, uint32_t* row_counts, uint64_t* total,
                              void* stream) {
  if (!a || !b) return fail(TGS_E_NULL, "matrix descriptor is NULL");
  uint32_t* rcs[1] = {row_counts};
  uint64_t* tots[1] = {total};
  return ternary_code_flips_batched(a, b, 1, rcs, tots, stream);
}

tgs_status ternary_gemv(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m, const int8_t* signs, float* y,
                        void* stream) {
  const void* xs[1] = {x};
  const int8_t* ss[1] = {signs};
  float* ys[1] = {y};
  if (!w) return fail(TGS_E_NULL, "matrix descriptor is NULL");
  return ternary_gemv_batched(w, 1, xs, x_dtype, m, ss, ys, stream);
}

tgs_status ternary_gemm(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m, const int8_t* signs, float* y,
                        void* stream) {
  return ternary_gemm_ws(w, x, x_dtype, m, signs, y, nullptr, 0, stream);
}

tgs_status ternary_gemm_ws(const tgs_matrix* w, const void* x, int32_t x_dtype, int64_t m, const int8_t* signs,
                           float* y, void* workspace, size_t workspace_bytes, void* stream) {
  tgs_status st = check_matrix(w, true);
  if (st != TGS_OK) return st;
  if (w->rotated)
    return fail(TGS_E_BASIS, "ternary_gemm multiplies plain-basis weights only; these weights are rotated");
  if (signs) return fail(TGS_E_BASIS, "signs given for weights in the plain basis");
  if (x_dtype != TGS_BF16) return fail(TGS_E_DTYPE, "ternary_gemm takes bf16 activations (TGS_BF16)");
  if (m < 1 || m > (1LL << 30)) return fail(TGS_E_SHAPE, "m must be >= 1, got %lld", (long long)m);
  // the kernels address a launch's activation rows (at least 128 of them) with 32-bit offsets
  if (w->k > tgs::kMaxDeviceCodeBytes / (128 * 2))
    return fail(TGS_E_SHAPE, "ternary_gemm needs k <= %lld (got %lld)", (long long)(tgs::kMaxDeviceCodeBytes / 256),
                (long long)w->k);
  if (!x || !y) return fail(TGS_E_NULL, "x or y is NULL");
  if (!aligned(x, 16)) return fail(TGS_E_ALIGN, "x must be 16-byte aligned");
  if (!aligned(y, 4)) return fail(TGS_E_ALIGN, "y must be 4-byte aligned");
  float* ws = static_cast<float*>(workspace);
  if (ws) {
    if (!aligned(ws, 4)) return fail(TGS_E_ALIGN, "workspace must be 4-byte aligned");
    const size_t need = tgs::gemm_workspace_bytes(w->layout, w->n, w->k, m);
    if (workspace_bytes < need)
      return fail(TGS_E_SIZE, "workspace of %zu bytes, this product needs %zu", workspace_bytes, need);
    if (need == 0) ws = nullptr;  // not split
  }
  hipError_t e = tgs::gemm_launch(w->layout, static_cast<const uint8_t*>(w->codes), w->code_row_stride, w->scales,
                                  w->n, w->k, static_cast<const uint16_t*>(x), m, y, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "ternary_gemm launch");
  return ok();
}

size_t ternary_gemm_workspace_size(const tgs_matrix* w, int64_t m) {
  if (check_matrix(w, true) != TGS_OK || w->rotated || m < 1 || m > (1LL << 30) ||
      w->k > tgs::kMaxDeviceCodeBytes / (128 * 2))
    return 0;
  ok();
  return tgs::gemm_workspace_bytes(w->layout, w->n, w->k, m);
}

tgs_status hadamard_rotate(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block, const int8_t* signs,
                           void* y, int32_t y_dtype, void* stream) {
  if (!x || !signs || !y) return fail(TGS_E_NULL, "x, signs or y is NULL");
  if (x_dtype != TGS_F16 && x_dtype != TGS_BF16 && x_dtype != TGS_F32)
    return fail(TGS_E_DTYPE, "x_dtype must be TGS_F16, TGS_BF16 or TGS_F32");
  if (y_dtype != TGS_F16 && y_dtype != TGS_BF16 && y_dtype != TGS_F32)
    return fail(TGS_E_DTYPE, "y_dtype must be TGS_F16, TGS_BF16 or TGS_F32");
  if (block != 128 && block != 1024) return fail(TGS_E_SHAPE, "block must be 128 or 1024, got %lld", (long long)block);
  if (m < 1 || k < block || k % block != 0 || m * (k / block) > (1LL << 40))
    return fail(TGS_E_SHAPE, "need m >= 1 and k a positive multiple of the block (%lld)", (long long)block);
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TGS_E_ALIGN, "x and y must be 16-byte aligned");
  if (!aligned(signs, 16)) return fail(TGS_E_ALIGN, "signs must be 16-byte aligned");
  const size_t xe = x_dtype == TGS_F32 ? 4 : 2, ye = y_dtype == TGS_F32 ? 4 : 2;
  const char *xb = static_cast<const char*>(x), *yb = static_cast<const char*>(y);
  const size_t xn = (size_t)(m * k) * xe, yn = (size_t)(m * k) * ye;
  if (xb < yb + yn && yb < xb + xn) return fail(TGS_E_SHAPE, "x and y overlap");
  hipError_t e = tgs::hadamard_launch(x, x_dtype, m, k, block, signs, y, y_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "hadamard_rotate launch");
  return ok();
}

tgs_status rmsnorm_hadamard_rotate(const void* x, int32_t x_dtype, int64_t m, int64_t k, int64_t block,
                                   const uint16_t* gamma, float eps, const int8_t* signs, void* y, int32_t y_dtype,
                                   void* stream) {
  if (!x || !gamma || !signs || !y) return fail(TGS_E_NULL, "x, gamma, signs or y is NULL");
  if (x_dtype != TGS_F16 && x_dtype != TGS_BF16 && x_dtype != TGS_F32)
    return fail(TGS_E_DTYPE, "x_dtype must be TGS_F16, TGS_BF16 or TGS_F32");
  if (y_dtype != TGS_F16 && y_dtype != TGS_BF16 && y_dtype != TGS_F32)
    return fail(TGS_E_DTYPE, "y_dtype must be TGS_F16, TGS_BF16 or TGS_F32");
  if (block != 128 && block != 1024) return fail(TGS_E_SHAPE, "block must be 128 or 1024, got %lld", (long long)block);
  if (m < 1 || m >= (1LL << 31) || k < block || k % block != 0 || k >= (1LL << 24))
    return fail(TGS_E_SHAPE, "need 1 <= m < 2^31 and k a multiple of the block (%lld) below 2^24", (long long)block);
  if (!(eps > 0.f && eps < INFINITY)) return fail(TGS_E_SHAPE, "eps must be positive and finite");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(TGS_E_ALIGN, "x and y must be 16-byte aligned");
  if (!aligned(signs, 16)) return fail(TGS_E_ALIGN, "signs must be 16-byte aligned");
  if (!aligned(gamma, 16)) return fail(TGS_E_ALIGN, "gamma must be 16-byte aligned");
  const size_t xe = x_dtype == TGS_F32 ? 4 : 2, ye = y_dtype == TGS_F32 ? 4 : 2;
  const char *xb = static_cast<const char*>(x), *yb = static_cast<const char*>(y);
  const size_t xn = (size_t)(m * k) * xe, yn = (size_t)(m * k) * ye;
  if (xb < yb + yn && yb < xb + xn) return fail(TGS_E_SHAPE, "x and y overlap");
  hipError_t e = tgs::rmsnorm_hadamard_launch(x, x_dtype, m, k, block, gamma, eps, signs, y, y_dtype,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "rmsnorm_hadamard_rotate launch");
  return ok();
}

tgs_status hadamard_rotate_g128(const void* x, int32_t x_dtype, int64_t m, int64_t k, const int8_t* signs, void* y,
                                int32_t y_dtype, void* stream) {
  return hadamard_rotate(x, x_dtype, m, k, 128, signs, y, y_dtype, stream);
}

size_t tgs_chain_workspace_bytes(void) {
  const int grid = tgs::chain_grid();
  return grid > 0 ? (size_t)(grid + 1) * sizeof(uint32_t) : 0;
}

// The launch arguments of a chain from the caller's steps (everything but the workspace), or an
// error status.
static tgs_status chain_args(const tgs_chain_step* steps, int32_t count, int grid, tgs::ChainArgs& args) {
  if (!steps) return fail(TGS_E_NULL, "steps is NULL");
  if (count < 1 || count > TGS_CHAIN_MAX_STEPS)
    return fail(TGS_E_SHAPE, "count must be 1..%d, got %d", TGS_CHAIN_MAX_STEPS, count);
  std::memset(&args, 0, sizeof(args));
  args.count = count;
  for (int32_t s = 0; s < count; ++s) {
    const tgs_chain_step& st = steps[s];
    tgs::ChainStep& cs = args.step[s];
    if (st.count < 1 || st.count > TGS_CHAIN_MAX_MATRICES)
      return fail(TGS_E_SHAPE, "step %d: count must be 1..%d", s, TGS_CHAIN_MAX_MATRICES);
    if (st.x_dtype != TGS_F16 && st.x_dtype != TGS_F32)
      return fail(TGS_E_DTYPE, "step %d: x_dtype must be TGS_F16 or TGS_F32", s);
    if (!st.x) return fail(TGS_E_NULL, "step %d: x is NULL", s);
    if (!aligned(st.x, 16)) return fail(TGS_E_ALIGN, "step %d: x must be 16-byte aligned", s);
    if (st.norm != 0 && st.norm != 1) return fail(TGS_E_SHAPE, "step %d: norm must be 0 or 1", s);
    if (st.norm) {
      if (!st.gamma) return fail(TGS_E_NULL, "step %d: gamma is NULL", s);
      if (!aligned(st.gamma, 16)) return fail(TGS_E_ALIGN, "step %d: gamma must be 16-byte aligned", s);
      if (!(st.eps > 0.f && st.eps < INFINITY)) return fail(TGS_E_SHAPE, "step %d: eps must be positive and finite", s);
    }
    int32_t rbs = 0;
    for (int32_t i = 0; i < st.count; ++i) {
      const tgs_matrix* w = &st.w[i];
      tgs_status e = check_matrix(w, true);
      if (e != TGS_OK) return e;
      if (w->layout != TGS_LAYOUT_SLOT2) return fail(TGS_E_LAYOUT, "step %d: the chain takes slot-2 matrices", s);
      if (w->rotated) return fail(TGS_E_BASIS, "step %d: the chain takes plain-basis matrices", s);
      if (w->k != st.w[0].k) return fail(TGS_E_SHAPE, "step %d: the matrices of a step share k", s);
      if (w->k % 512 != 0 || w->k > 16384)
        return fail(TGS_E_SHAPE, "step %d: k must be a multiple of 512 up to 16384 (k=%lld)", s, (long long)w->k);
      if (!st.y[i]) return fail(TGS_E_NULL, "step %d: y[%d] is NULL", s, i);
      if (!aligned(st.y[i], 4)) return fail(TGS_E_ALIGN, "step %d: y must be 4-byte aligned", s);
      tgs::ChainMat& cm = cs.mat[i];
      cm.codes = static_cast<const uint8_t*>(w->codes);
      cm.scales = w->scales;
      cm.y = st.y[i];
      cm.n = (int32_t)w->n;
      cm.stride = (int32_t)w->code_row_stride;
      cm.rb0 = rbs;
      rbs += (int32_t)((w->n + 15) / 16);
    }
    if ((rbs + grid - 1) / grid > tgs::kChainMaxRbsPerWg)
      return fail(TGS_E_SHAPE, "step %d: %d row blocks of 16 exceed %d per compute unit", s, rbs,
                  tgs::kChainMaxRbsPerWg);
    cs.x = st.x;
    cs.gamma = st.norm ? st.gamma : nullptr;
    cs.k = (int32_t)st.w[0].k;
    cs.count = st.count;
    cs.x_f32 = st.x_dtype == TGS_F32 ? 1 : 0;
    cs.norm = st.norm;
    cs.rbs = rbs;
    cs.eps = st.eps;
  }
  return ok();
}

tgs_status ternary_gemv_chain(const tgs_chain_step* steps, int32_t count, uint32_t* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!workspace) return fail(TGS_E_NULL, "workspace is NULL");
  if (!aligned(workspace, 4)) return fail(TGS_E_ALIGN, "workspace must be 4-byte aligned");
  const int grid = tgs::chain_grid();
  if (grid < 1) return fail(TGS_E_DEVICE, "no usable device for the chain launch");
  if (workspace_bytes < (size_t)(grid + 1) * sizeof(uint32_t))
    return fail(TGS_E_SIZE, "workspace holds %zu bytes, needs %zu", workspace_bytes,
                (size_t)(grid + 1) * sizeof(uint32_t));
  tgs::ChainArgs args;
  tgs_status st = chain_args(steps, count, grid, args);
  if (st != TGS_OK) return st;
  args.flags = workspace;
  hipError_t e = tgs::chain_launch(args, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "ternary_gemv_chain launch");
  return ok();
}

tgs_status ternary_gemv_chain_static(const tgs_chain_step* steps, int32_t count, uint32_t* error, void* stream) {
  if (error && !aligned(error, 4)) return fail(TGS_E_ALIGN, "error must be 4-byte aligned");
  const int grid = tgs::chain_grid();
  if (grid < 1) return fail(TGS_E_DEVICE, "no usable device for the chain launch");
  if (grid + 1 > tgs::kChainStaticWords)
    return fail(TGS_E_SIZE, "the library's chain workspace holds %d words; a chain on this device needs %d",
                tgs::kChainStaticWords, grid + 1);
  tgs::ChainArgs args;
  tgs_status st = chain_args(steps, count, grid, args);
  if (st != TGS_OK) return st;
  uint32_t* words = nullptr;
  hipError_t e = tgs::chain_static_workspace(&words);
  if (e != hipSuccess) return device_error(e, "ternary_gemv_chain_static workspace lookup");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the counts start at zero on every call, and so does the error word
  e = tgs::chain_clear(words, grid + 1, s);
  if (e != hipSuccess) return device_error(e, "ternary_gemv_chain_static clear");
  args.flags = words;
  e = tgs::chain_launch(args, grid, s);
  if (e != hipSuccess) return device_error(e, "ternary_gemv_chain_static launch");
  if (error) {
    e = hipMemcpyAsync(error, words + grid, sizeof(uint32_t), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return device_error(e, "ternary_gemv_chain_static error word copy");
  }
  return ok();
}

size_t tgs_stream_read_sink_words(void) { return (size_t)tgs::stream_read_grid() * 256; }

tgs_status tgs_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(TGS_E_NULL, "buf or sink is NULL");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(TGS_E_ALIGN, "buf must be 16-byte and sink 4-byte aligned");
  if (bytes < 16 || bytes % 16 != 0) return fail(TGS_E_SHAPE, "bytes must be a positive multiple of 16");
  hipError_t e = tgs::stream_read_launch(buf, (uint64_t)bytes, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "tgs_stream_read launch");
  return ok();
}

const char* tgs_status_string(tgs_status status) {
  switch (status) {
    case TGS_OK: return "ok";
    case TGS_E_NULL: return "null pointer";
    case TGS_E_SHAPE: return "invalid shape";
    case TGS_E_ALIGN: return "misaligned buffer";
    case TGS_E_CODE: return "invalid code";
    case TGS_E_LAYOUT: return "invalid descriptor or layout";
    case TGS_E_BASIS: return "basis mismatch";
    case TGS_E_SIZE: return "buffer too small";
    case TGS_E_DTYPE: return "unsupported dtype";
    case TGS_E_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* tgs_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
