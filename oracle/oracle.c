/*
 * CPU ORACLE for the ternary group-scaled matmul — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The GPU library never links, includes or calls it, and
 * this file includes nothing from the GPU library: the two share no code.
 *
 * What it computes, in fp64, plainly and slowly:
 *
 *   y[m][n] = sum_k  s[n][k/128] * t[n][k] * xr[m][k]
 *
 * where t[n][k] in {-1, 0, +1} are the ternary codes (in {-1, +1} for the
 * binary sibling format, the two-level variant with the same group scale:
 * "Bonsai 27B and how 1-bit survives" (velog.io), sections "What ternary and
 * binary are" and "What the format is"), s[n][g] is the fp16
 * scale shared by the 128 weights of group g along K, and xr is the
 * activation x, or R x when the weights are stored in the rotated basis.
 *   - The weight definition w = s_g * t with one fp16 scale per 128 weights:
 *     "Ternary Bonsai 2 27B, 5.93GB ... (feat. PrismML)" (discuss.pytorch.kr),
 *     section "Ternary weights and the rotated basis", subsection
 *     "Group-scaled ternary format", the equation for w_i; the same formula in
 *     "Bonsai 27B and how 1-bit survives" (velog.io), section "What the format is".
 *   - The rotation R = (1/sqrt(n)) H_n S with S a fixed +-1 diagonal, and the
 *     layer computing f(x) = W(Rx): same P3 page, subsection "Block-wise
 *     Hadamard rotation". The block size n is 128 (one block per scale group)
 *     or 1024 (the size that subsection names; a block then spans 8 groups),
 *     and H is the natural-order Sylvester matrix H[i][j] =
 *     (-1)^popcount(i & j), the normalised Sylvester transform the WebGPU
 *     loader insists on (P3 page, section "Running in the browser with
 *     WebGPU").
 *
 * Optionally the activation is first normalised with RMSNorm, x^ = gamma * x /
 * sqrt(mean_k x^2 + eps) per row, and x^ takes the place of x above: the
 * BlockHadamard operation of the P3 page's WebGPU runtime has a variant fused
 * with RMSNorm (section "Running in the browser with WebGPU"), and the norm
 * weights gamma stay in bf16, neither rotated nor quantised (section "The
 * 0.0976% kept at high precision"). The pages do not write the norm out; this is
 * the usual root-mean-square normalisation over the row (the mean of the squares
 * over all K entries, eps added inside the square root), gamma applied
 * elementwise after the division.
 *
 * Every step is done the obvious way: each row is unpacked from its packed
 * bytes by a bit-by-bit loop, dequantised to doubles (fp16/bf16 -> double is
 * exact), and multiplied; the rotation is a dense n x n matrix-vector
 * product per block, not a fast transform. Threads split rows only; the
 * arithmetic for each output is a plain sequential sum over k.
 *
 * Packed layouts (the pages fix the cost per weight, not the bit order; these
 * are the readings this oracle fixes):
 *   slot2: code q = t + 1 in {0, 1, 2} (3 is invalid); element k of a row sits
 *          in bits 2*(k%4) .. 2*(k%4)+1 of byte k/4; rows are K/4 bytes apart.
 *          With the fp16 scale per 128 weights this is 34 bytes per 128
 *          weights, the figure the P3 page gives for scale plus 2-bit codes in
 *          "Two packings: PTQ1_0 and PQ2_0".
 *   base3: five trits per byte, byte b of a row = sum_{j<5} (t[5b+j]+1) * 3^j;
 *          trits past K are 0 (digit 1); a row holds ceil(K/5) such bytes,
 *          then pad bytes of value 121 (five zero trits) up to a multiple of 16.
 *   binary: one bit per weight, element k of a row in bit k%8 of byte k/8, a
 *          set bit meaning t = +1 and a clear bit t = -1 (t = 0 cannot be
 *          stored); rows are K/8 bytes apart. With the fp16 scale that is 18
 *          bytes per 128 weights, 1.125 bits per weight, the figure the velog.io
 *          page gives for the binary format with group scales.
 *   scales: a separate fp16 array [n][K/128], row-major.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_CODE -1
#define ORC_BAD_SHAPE -2
#define ORC_BAD_LAYOUT -3

#define ORC_SLOT2 1
#define ORC_BASE3 2
#define ORC_BINARY 3

#define ORC_X_F16 1
#define ORC_X_BF16 2

/* ---- storage dtypes -> double (exact), from the IEEE 754 bit layouts ---- */

double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);       /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

double orc_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1, e = (b >> 7) & 255, m = b & 127;
  double v;
  if (e == 0) v = ldexp((double)m, -133);           /* subnormal: m * 2^-133 */
  else if (e == 255) v = m ? NAN : INFINITY;
  else v = ldexp((double)(128 + m), e - 134);       /* (1 + m/128) * 2^(e-127) */
  return sign ? -v : v;
}

/* ---- layout sizes ---- */

int64_t orc_row_bytes(int32_t layout, int64_t k) {
  if (k <= 0 || k % 128 != 0) return 0;
  if (layout == ORC_SLOT2) return k / 4;
  if (layout == ORC_BINARY) return k / 8;
  if (layout == ORC_BASE3) {
    int64_t used = (k + 4) / 5;
    return (used + 15) / 16 * 16;
  }
  return 0;
}

/* ---- slot2 ---- */

int orc_pack_slot2(const int8_t* t, int64_t n, int64_t k, uint8_t* codes) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = k / 4;
  memset(codes, 0, (size_t)(n * rb));
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      int v = t[r * k + c];
      if (v < -1 || v > 1) return ORC_BAD_CODE;
      int q = v + 1;
      int64_t byte = c / 4;
      int bit = 2 * (int)(c % 4);
      codes[r * rb + byte] |= (uint8_t)(q << bit);
    }
  }
  return ORC_OK;
}

int orc_unpack_slot2(const uint8_t* codes, int64_t n, int64_t k, int8_t* t) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = k / 4;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      int q = (codes[r * rb + c / 4] >> (2 * (c % 4))) & 3;
      if (q == 3) return ORC_BAD_CODE;
      t[r * k + c] = (int8_t)(q - 1);
    }
  }
  return ORC_OK;
}

/* ---- base3 ---- */

int orc_pack_base3(const int8_t* t, int64_t n, int64_t k, uint8_t* codes) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = orc_row_bytes(ORC_BASE3, k);
  int64_t used = (k + 4) / 5;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t b = 0; b < rb; ++b) {
      int value = 0, power = 1;
      for (int j = 0; j < 5; ++j) {
        int64_t c = 5 * b + j;
        int digit = 1; /* trit 0 for positions past K and for pad bytes */
        if (b < used && c < k) {
          int v = t[r * k + c];
          if (v < -1 || v > 1) return ORC_BAD_CODE;
          digit = v + 1;
        }
        value += digit * power;
        power *= 3;
      }
      codes[r * rb + b] = (uint8_t)value;
    }
  }
  return ORC_OK;
}

int orc_unpack_base3(const uint8_t* codes, int64_t n, int64_t k, int8_t* t) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = orc_row_bytes(ORC_BASE3, k);
  int64_t used = (k + 4) / 5;
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t b = 0; b < rb; ++b) {
      int value = codes[r * rb + b];
      if (value > 242) return ORC_BAD_CODE;
      if (b >= used) {
        if (value != 121) return ORC_BAD_CODE;
        continue;
      }
      for (int j = 0; j < 5; ++j) {
        int digit = value % 3;
        value /= 3;
        int64_t c = 5 * b + j;
        if (c < k) t[r * k + c] = (int8_t)(digit - 1);
        else if (digit != 1) return ORC_BAD_CODE; /* positions past K hold trit 0 */
      }
    }
  }
  return ORC_OK;
}

/* ---- binary ---- */

int orc_pack_binary(const int8_t* t, int64_t n, int64_t k, uint8_t* codes) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = k / 8;
  memset(codes, 0, (size_t)(n * rb));
  for (int64_t r = 0; r < n; ++r) {
    for (int64_t c = 0; c < k; ++c) {
      int v = t[r * k + c];
      if (v != -1 && v != 1) return ORC_BAD_CODE;  /* two levels only */
      if (v == 1) codes[r * rb + c / 8] |= (uint8_t)(1u << (c % 8));
    }
  }
  return ORC_OK;
}

int orc_unpack_binary(const uint8_t* codes, int64_t n, int64_t k, int8_t* t) {
  if (k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  int64_t rb = k / 8;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t c = 0; c < k; ++c)
      t[r * k + c] = ((codes[r * rb + c / 8] >> (c % 8)) & 1) ? 1 : -1;
  return ORC_OK;
}

/* ---- one row of codes -> trits (used by the product; same loops as above) ---- */

static int unpack_row(int32_t layout, const uint8_t* row, int64_t k, int8_t* t) {
  if (layout == ORC_SLOT2) return orc_unpack_slot2(row, 1, k, t);
  if (layout == ORC_BASE3) return orc_unpack_base3(row, 1, k, t);
  if (layout == ORC_BINARY) return orc_unpack_binary(row, 1, k, t);
  return ORC_BAD_LAYOUT;
}

/* ---- Sylvester Hadamard and the block rotation ---- */

static int popcount32(uint32_t v) {
  int c = 0;
  while (v) { c += (int)(v & 1u); v >>= 1; }
  return c;
}

/* H[i][j] = (-1)^popcount(i & j), natural (Sylvester) order; n must be a power of 2 */
void orc_hadamard(int32_t n, int8_t* h) {
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < n; ++j)
      h[(int64_t)i * n + j] = (int8_t)((popcount32((uint32_t)(i & j)) & 1) ? -1 : 1);
}

/* xr[m][k] = sum_j H[i][j] * sign[b*n+j] * x[m][b*n+j] / sqrt(n), k = b*n + i, for blocks of
   n = 128 or 1024 (k a multiple of n): a dense n x n product per block */
void orc_rotate_f64(const double* x, const int8_t* sign, int64_t m, int64_t k, int64_t n, double* xr) {
  int8_t* h = (int8_t*)malloc((size_t)(n * n));
  orc_hadamard((int32_t)n, h);
  const double norm = sqrt((double)n);
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t b = 0; b < k / n; ++b) {
      const double* xb = x + r * k + b * n;
      const int8_t* sb = sign + b * n;
      for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += (double)h[i * n + j] * ((double)sb[j] * xb[j]);
        xr[r * k + b * n + i] = acc / norm;
      }
    }
  }
  free(h);
}

/* activation bits -> doubles */
int orc_load_x(const uint16_t* x, int32_t x_dtype, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) {
    if (x_dtype == ORC_X_F16) out[i] = orc_f16_to_f64(x[i]);
    else if (x_dtype == ORC_X_BF16) out[i] = orc_bf16_to_f64(x[i]);
    else return ORC_BAD_LAYOUT;
  }
  return ORC_OK;
}

/* RMSNorm of each row of x [m][k] (doubles): out = gamma * x / sqrt(sum_c x^2 / k + eps), gamma
 * given as bf16 bits [k]. eps must be > 0. */
int orc_rmsnorm_f64(const double* x, const uint16_t* gamma, double eps, int64_t m, int64_t k, double* out) {
  if (m < 1 || k < 1 || !(eps > 0.0)) return ORC_BAD_SHAPE;
  for (int64_t r = 0; r < m; ++r) {
    const double* xr = x + r * k;
    double sq = 0.0;
    for (int64_t c = 0; c < k; ++c) sq += xr[c] * xr[c];
    double rms = sqrt(sq / (double)k + eps);
    for (int64_t c = 0; c < k; ++c) out[r * k + c] = orc_bf16_to_f64(gamma[c]) * xr[c] / rms;
  }
  return ORC_OK;
}

/* The activation the product uses: x, optionally RMS-normalised (gamma != NULL), then
 * optionally rotated (sign != NULL). out: [m][k] doubles. */
static int prepare_x(const uint16_t* x, int32_t x_dtype, const uint16_t* gamma, double eps, const int8_t* sign,
                     int64_t block, int64_t m, int64_t k, double* out) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)(m * k));
  if (!xd) return ORC_BAD_SHAPE;
  int rc = orc_load_x(x, x_dtype, m * k, xd);
  if (rc == ORC_OK && gamma) {
    double* xn = (double*)malloc(sizeof(double) * (size_t)(m * k));
    if (!xn) rc = ORC_BAD_SHAPE;
    else {
      rc = orc_rmsnorm_f64(xd, gamma, eps, m, k, xn);
      free(xd);
      xd = xn;
    }
  }
  if (rc == ORC_OK) {
    if (sign) orc_rotate_f64(xd, sign, m, k, block, out);
    else memcpy(out, xd, sizeof(double) * (size_t)(m * k));
  }
  free(xd);
  return rc;
}

/* The standalone fused operation: out = R (RMSNorm x), or RMSNorm x when sign is NULL. */
int orc_rmsnorm_rotate_f64(const uint16_t* x, int32_t x_dtype, const uint16_t* gamma, double eps,
                           const int8_t* sign, int64_t m, int64_t k, int64_t block, double* out) {
  if (m < 1 || k <= 0 || !gamma) return ORC_BAD_SHAPE;
  if (sign && ((block != 128 && block != 1024) || k % block != 0)) return ORC_BAD_SHAPE;
  return prepare_x(x, x_dtype, gamma, eps, sign, block, m, k, out);
}

/*
 * y[m][j] and bound[m][j] for the selected rows n = rows[j] (all rows if rows == NULL,
 * then n_sel must equal n).
 *   y     = sum_k s * t * xr
 *   bound = 1e-3 * sum_k |s * t * xr| + 1e-6   (per-element tolerance on the result)
 * codes: [n][row_stride] bytes, scales: [n][k/128] fp16 bits, x: [m][k] fp16/bf16 bits,
 * sign: [k] (+-1) or NULL for the unrotated basis.
 */
int orc_matmul_norm_f64(int32_t layout, const uint8_t* codes, int64_t row_stride,
                        const uint16_t* scales, int64_t n, int64_t k,
                        const uint16_t* x, int32_t x_dtype, int64_t m,
                        const uint16_t* gamma, double eps,
                        const int8_t* sign, int64_t block, const int64_t* rows, int64_t n_sel,
                        double* y, double* bound) {
  if (k <= 0 || k % 128 != 0 || m < 1 || n < 0) return ORC_BAD_SHAPE;
  if (sign && (block != 128 && block != 1024)) return ORC_BAD_SHAPE;
  if (sign && k % block != 0) return ORC_BAD_SHAPE;
  if (orc_row_bytes(layout, k) == 0) return ORC_BAD_LAYOUT;
  if (row_stride < orc_row_bytes(layout, k)) return ORC_BAD_SHAPE;
  if (rows == NULL && n_sel != n) return ORC_BAD_SHAPE;

  double* xr = (double*)malloc(sizeof(double) * (size_t)(m * k));
  if (!xr) return ORC_BAD_SHAPE;
  int rc = prepare_x(x, x_dtype, gamma, eps, sign, block, m, k, xr);
  if (rc != ORC_OK) { free(xr); return rc; }

  int status = ORC_OK;
#pragma omp parallel
  {
    int8_t* t = (int8_t*)malloc((size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(dynamic, 16)
    for (int64_t j = 0; j < n_sel; ++j) {
      int64_t r = rows ? rows[j] : j;
      /* several threads may report a failure: each store is atomic, and any one failing status is
         the result */
      if (r < 0 || r >= n) {
#pragma omp atomic write
        status = ORC_BAD_SHAPE;
        continue;
      }
      if (unpack_row(layout, codes + r * row_stride, k, t) != ORC_OK) {
#pragma omp atomic write
        status = ORC_BAD_CODE;
        continue;
      }
      for (int64_t c = 0; c < k; ++c) w[c] = orc_f16_to_f64(scales[r * (k / 128) + c / 128]) * (double)t[c];
      for (int64_t i = 0; i < m; ++i) {
        double acc = 0.0, mag = 0.0;
        for (int64_t c = 0; c < k; ++c) {
          double p = w[c] * xr[i * k + c];
          acc += p;
          mag += fabs(p);
        }
        y[i * n_sel + j] = acc;
        bound[i * n_sel + j] = 1e-3 * mag + 1e-6;
      }
    }
    free(t);
    free(w);
  }
  free(xr);
  return status;
}

/* The product without the norm (gamma == NULL). */
int orc_matmul_f64(int32_t layout, const uint8_t* codes, int64_t row_stride,
                   const uint16_t* scales, int64_t n, int64_t k,
                   const uint16_t* x, int32_t x_dtype, int64_t m,
                   const int8_t* sign, int64_t block, const int64_t* rows, int64_t n_sel,
                   double* y, double* bound) {
  return orc_matmul_norm_f64(layout, codes, row_stride, scales, n, k, x, x_dtype, m, NULL, 0.0, sign, block, rows,
                             n_sel, y, bound);
}

/* ---- code flips between two packed checkpoints ---- */

/*
 * A code flip is a weight whose ternary code changed between two checkpoints, for
 * example 0 -> +1 or +1 -> -1; it is the only way training changes what the model
 * computes, as opposed to nudging the shared scales ("Fine-tuning the ternary
 * Bonsai-8B on Metal" (molayo1419.me), opening section on native-ternary models;
 * the closing advice counts the flips per checkpoint).
 *
 * counts[r] = #{ c < k : t_a[r][c] != t_b[r][c] } for two matrices of the same
 * layout and shape, each row unpacked with the bit-by-bit loops above. Rows are
 * row_stride_a / row_stride_b bytes apart; bytes past the row's codes are not read
 * as codes. Returns the total, or a negative status.
 */
int64_t orc_code_flips(int32_t layout, const uint8_t* a, int64_t row_stride_a, const uint8_t* b,
                       int64_t row_stride_b, int64_t n, int64_t k, int64_t* counts) {
  if (k <= 0 || k % 128 != 0 || n < 0) return ORC_BAD_SHAPE;
  if (orc_row_bytes(layout, k) == 0) return ORC_BAD_LAYOUT;
  if (row_stride_a < orc_row_bytes(layout, k) || row_stride_b < orc_row_bytes(layout, k)) return ORC_BAD_SHAPE;
  int64_t total = 0;
  int status = ORC_OK;
#pragma omp parallel reduction(+ : total)
  {
    int8_t* ta = (int8_t*)malloc((size_t)k);
    int8_t* tb = (int8_t*)malloc((size_t)k);
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < n; ++r) {
      if (unpack_row(layout, a + r * row_stride_a, k, ta) != ORC_OK ||
          unpack_row(layout, b + r * row_stride_b, k, tb) != ORC_OK) {
#pragma omp atomic write
        status = ORC_BAD_CODE;
        continue;
      }
      int64_t c = 0;
      for (int64_t i = 0; i < k; ++i) c += ta[i] != tb[i];
      if (counts) counts[r] = c;
      total += c;
    }
    free(ta);
    free(tb);
  }
  return status == ORC_OK ? total : status;
}
