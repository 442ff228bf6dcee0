/*
 * CPU oracle for silu_dot_fwd_bwd_quant_fuse -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, single-threaded definition that the HIP path
 * is checked against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product library never does,
 * and this file shares no code, header, table or constant with it.
 *
 * What it computes (page "kernelgen-challenge-9-task3-silu-quant" on
 * githubhelp.com, the entry-point listing and the two output bullets that
 * follow it):
 *   x = [gate | up]            bf16 [T, 2H]   (gate = cols [0,H), up = [H,2H))
 *   grad_y                     bf16 [T, H]
 *   y      = silu(gate) * up                       (forward recompute)
 *   d_gate = grad_y * up * s * (1 + gate*(1 - s))  (s = sigmoid(gate))
 *   d_up   = grad_y * silu(gate)
 *   grad_input_q/_s : [d_gate, d_up] quantised to int8, one fp32 scale per
 *                     `group` contiguous channels of each 2H-long row.
 *   y_q_t/_s_t      : y transposed to [H, T], int8, one fp32 scale per
 *                     `group` consecutive tokens of each row of y^T.
 * The same page's list of design constraints fixes two more points used here:
 * every value is rounded through bf16 before it is quantised, and the
 * quantiser multiplies by a precomputed inverse scale.
 *
 * Readings taken where the page is silent (each is listed in the design notes):
 *   - arithmetic is fp32, evaluated strictly left to right in the order
 *     written below, with no fused multiply-add (build with -ffp-contract=off);
 *   - exp(-g) is the correctly rounded fp32 value, obtained from the double
 *     exp and rounded once to float;
 *   - bf16 rounding is round-to-nearest-even on the fp32 bit pattern, with
 *     subnormals kept;
 *   - the group maximum is taken over the bf16-rounded values;
 *   - scale = amax / 127 (1.0 when amax == 0), inv = 1 / scale and the
 *     product p = v * inv are each one fp32 operation, and
 *     q = clamp(rne(p), -127, 127): the page asks for a multiplication by a
 *     precomputed fp32 inverse in place of a division, and in fp32 arithmetic
 *     that multiplication rounds its result to fp32 like every other step
 *     here; rne then rounds that fp32 value to the nearest integer, ties to
 *     even.  q = 0 whenever v == 0 (this avoids 0 * inf when a group's scale
 *     is so small that 1/scale overflows);
 *   - a trailing group shorter than `group` (T or 2H not a multiple of it) is
 *     quantised over the elements it has.
 *
 * The forward quantiser (oracle_silu_fwd_quant) follows the fused launch the
 * page "kquant_mmq.rs" (docs.atlascybernetics.ai) documents for
 * kquant_swiglu_q8_1_rows: h = bf16(swiglu(gate, up) * w[row]), then group
 * quantisation of those bf16 rows.  Readings: w is an optional fp32 weight per
 * row (absent = 1); swiglu is (g * s) * u exactly as in the backward pass, the
 * weight multiplies that fp32 product, and the result is rounded to bf16 once;
 * groups are `group` contiguous channels of each row with the quantiser above.
 * The page's `limit` argument has no stated meaning and is not modelled.
 *
 * The FP8 variant (oracle_silu_dot_fwd_bwd_quant_fuse_fp8) writes the same two
 * products with OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; largest finite value 448; subnormals k * 2^-9):
 * scale = amax / 448 (1.0 when amax == 0), inv = 1 / scale, and the code is
 * the e4m3 value nearest the fp32 product v * inv (ties to even), saturated to
 * +-448; a zero v gives the zero code of its own sign (E4M3 has -0 = 0x80, and
 * this also avoids 0 * inf).  Readings: the product v * inv is one fp32
 * multiplication, exactly as in the int8 quantiser above, and the code is the
 * E4M3 value nearest that fp32 product; saturation only matters for groups
 * whose inverse overflowed, since with a finite inverse |v * inv| stays within
 * 448 * (1 + 2^-22).
 *
 * The group-scaled int8 product (oracle_i8_gemm_group_scaled) is the consumer
 * of the two quantised layouts: the same page's fusion bullet names the
 * K-group and M-group quantisations, i.e. groups of 128 along the contraction
 * axis of the GEMM that reads them.  The page gives no formula for the GEMM;
 * the plain reading is the product of the dequantised operands,
 *   C[m, n] = sum_k (sA[m, k/G] * A[m, k]) * (sB[n/Bb, k/G] * B[n, k])
 *           = sum_g sA[m, g] * sB[n/Bb, g] * (sum_{k in g} A[m, k] * B[n, k]),
 * with A [M, K] and B [N, K] int8 row-major (C = A . B^T), G = group and Bb
 * the number of B rows sharing one scale (1: one scale per row and group, as
 * y_s_t; 128: one per 128 x 128 block, a weight's usual layout).  The integer
 * dot of each group is exact (int64) and the sum over groups is taken in
 * double; the result is reported with the sum of the absolute values of the
 * group terms, which bounds the rounding of any fp32 evaluation order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ---- bf16 <-> fp32 --------------------------------------------------------- */

/* bf16 widens to fp32 exactly: its 16 bits are the top half of the fp32. */
ORACLE_API float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even, on the bit pattern.
 * Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
 * when the dropped half is above the midpoint, or at it with an odd kept half.
 * Subnormals round the same way; NaN is outside the domain. */
ORACLE_API uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static float bf16_round(float f) { return oracle_bf16_to_f32(oracle_f32_to_bf16(f)); }

/* ---- the elementwise part -------------------------------------------------- */

/* Sigmoid as 1 / (1 + exp(-g)).  The intermediate e and den are returned too so
 * that tests can pin each rounding step separately. */
ORACLE_API float oracle_sigmoid_parts(float g, float* e_out, float* den_out) {
  float e = (float)exp(-(double)g); /* one rounding of the (double) exp to fp32 */
  float den = 1.0f + e;
  float s = 1.0f / den;
  if (e_out) *e_out = e;
  if (den_out) *den_out = den;
  return s;
}

ORACLE_API float oracle_sigmoid(float g) { return oracle_sigmoid_parts(g, NULL, NULL); }

/* One (t, h) position before the bf16 round trip: gate g, up u, grad_y d.
 * Order of operations: silu = g*s; y = silu*u;
 * d_gate = ((d*u)*s) * (1 + g*(1 - s)); d_up = d*silu. */
ORACLE_API void oracle_pair_f32(float g, float u, float d, float* y, float* d_gate, float* d_up) {
  float s = oracle_sigmoid(g);
  float silu = g * s;
  *y = silu * u;
  float a = d * u;
  float b = a * s;
  float c = 1.0f - s;
  float k = g * c;
  float m = 1.0f + k;
  *d_gate = b * m;
  *d_up = d * silu;
}

/* ---- the quantiser --------------------------------------------------------- */

/* Largest magnitude of a group of n values spaced stride apart. */
static float oracle_group_amax(const float* v, int64_t n, int64_t stride) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(v[i * stride]);
    if (a > amax) amax = a;
  }
  return amax;
}

/* Quantise n values v[0], v[stride], ... into q[0], q[qstride], ... and return
 * the group's scale.  v holds bf16-representable values. */
ORACLE_API float oracle_quant_group(const float* v, int64_t n, int64_t stride, int8_t* q, int64_t qstride) {
  float amax = oracle_group_amax(v, n, stride);
  float scale = (amax == 0.0f) ? 1.0f : amax / 127.0f;
  float inv = 1.0f / scale;
  for (int64_t i = 0; i < n; ++i) {
    float x = v[i * stride];
    int8_t out = 0;
    if (x != 0.0f) {
      float p = x * inv;       /* one fp32 rounding (no contraction: -ffp-contract=off) */
      float r = nearbyintf(p); /* default rounding mode: to nearest, ties to even */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      out = (int8_t)r;
    }
    q[i * qstride] = out;
  }
  return scale;
}

/* ---- FP8 E4M3 ---------------------------------------------------------------- */

/* Nearest E4M3 code of x (ties to even), saturating at +-448; NaN is outside
 * the domain.  Works in double, where every step below is exact. */
ORACLE_API uint8_t oracle_f32_to_e4m3(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E; /* 448 = 1.75 * 2^8: exponent field 15, mantissa 6 */
  if (a < 0.015625) {                 /* below 2^-6: subnormals k * 2^-9, k = 0..8 */
    double k = nearbyint(a * 512.0);  /* k == 8 is the smallest normal, 2^-6 */
    return sign | (uint8_t)k;         /* k == 8 encodes as exponent field 1, mantissa 0 */
  }
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  double mant = nearbyint(m * 16.0); /* 8 .. 16: the leading one plus 3 fraction bits */
  if (mant == 16.0) {
    mant = 8.0;
    e += 1;
  }
  int efield = e - 1 + 7;
  if (efield > 15 || (efield == 15 && mant > 14.0)) return sign | 0x7E; /* rounds above 448 */
  return sign | (uint8_t)(efield << 3) | (uint8_t)((int)mant - 8);
}

ORACLE_API double oracle_e4m3_to_f64(uint8_t c) {
  double sgn = (c & 0x80) ? -1.0 : 1.0;
  int ef = (c >> 3) & 0xF, mf = c & 7;
  if (ef == 15 && mf == 7) return NAN;
  if (ef == 0) return sgn * mf * ldexp(1.0, -9);
  return sgn * (1.0 + mf / 8.0) * ldexp(1.0, ef - 7);
}

/* Quantise one group to E4M3 codes; returns the scale. */
ORACLE_API float oracle_quant_group_fp8(const float* v, int64_t n, int64_t stride, uint8_t* q, int64_t qstride) {
  float amax = oracle_group_amax(v, n, stride);
  float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  float inv = 1.0f / scale;
  for (int64_t i = 0; i < n; ++i) {
    float x = v[i * stride];
    q[i * qstride] = (x == 0.0f) ? oracle_f32_to_e4m3(x) : oracle_f32_to_e4m3(x * inv);
  }
  return scale;
}

/* ---- the whole pass -------------------------------------------------------- */

enum {
  ORACLE_OK = 0,
  ORACLE_BAD_ARG = 1,
  ORACLE_NO_MEMORY = 2,
};

/* The bf16-rounded intermediates: Y [T, H] (y) and D [T, 2H] ([d_gate, d_up]),
 * stored as float. */
ORACLE_API int oracle_intermediates(const uint16_t* x, const uint16_t* grad_y, float* Y, float* D,
                                    int64_t T, int64_t H) {
  if (T < 0 || H < 0) return ORACLE_BAD_ARG;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      float g = oracle_bf16_to_f32(x[t * 2 * H + h]);
      float u = oracle_bf16_to_f32(x[t * 2 * H + H + h]);
      float d = oracle_bf16_to_f32(grad_y[t * H + h]);
      float y, dg, du;
      oracle_pair_f32(g, u, d, &y, &dg, &du);
      Y[t * H + h] = bf16_round(y);
      D[t * 2 * H + h] = bf16_round(dg);
      D[t * 2 * H + H + h] = bf16_round(du);
    }
  }
  return ORACLE_OK;
}

/* Quantise the intermediates: row groups of D, then column groups of Y. */
ORACLE_API int oracle_quantise(const float* Y, const float* D, int8_t* grad_input_q, float* grad_input_s,
                               int8_t* y_q_t, float* y_s_t, int64_t T, int64_t H, int64_t group) {
  if (T < 0 || H < 0 || group <= 0) return ORACLE_BAD_ARG;
  int64_t row_groups = (2 * H + group - 1) / group;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < row_groups; ++j) {
      int64_t c0 = j * group;
      int64_t n = (2 * H - c0 < group) ? 2 * H - c0 : group;
      grad_input_s[t * row_groups + j] =
          oracle_quant_group(&D[t * 2 * H + c0], n, 1, &grad_input_q[t * 2 * H + c0], 1);
    }
  }
  int64_t col_groups = (T + group - 1) / group;
  for (int64_t h = 0; h < H; ++h) {
    for (int64_t j = 0; j < col_groups; ++j) {
      int64_t t0 = j * group;
      int64_t n = (T - t0 < group) ? T - t0 : group;
      /* column h of Y, tokens t0.., goes to row h of y^T */
      y_s_t[h * col_groups + j] = oracle_quant_group(&Y[t0 * H + h], n, H, &y_q_t[h * T + t0], 1);
    }
  }
  return ORACLE_OK;
}

/* Forward: y = bf16((silu(g) * u) * w[t]) for x = [gate | up] [T, 2H]; writes
 * y_q [T, H] int8 and y_s [T, ceil(H/group)] fp32 (row groups), and, when
 * y_bf16 is not NULL, the bf16 bits of y.  w may be NULL (weight 1). */
ORACLE_API int oracle_silu_fwd_quant(const uint16_t* x, const float* w, int8_t* y_q, float* y_s, uint16_t* y_bf16,
                                     int64_t T, int64_t H, int64_t group) {
  if (T < 0 || H < 0 || group <= 0) return ORACLE_BAD_ARG;
  if (T == 0 || H == 0) return ORACLE_OK;
  float* Y = (float*)malloc((size_t)H * sizeof(float));
  if (!Y) return ORACLE_NO_MEMORY;
  int64_t groups = (H + group - 1) / group;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t h = 0; h < H; ++h) {
      float g = oracle_bf16_to_f32(x[t * 2 * H + h]);
      float u = oracle_bf16_to_f32(x[t * 2 * H + H + h]);
      float s = oracle_sigmoid(g);
      float silu = g * s;
      float v = silu * u;
      if (w) v = v * w[t];
      uint16_t b = oracle_f32_to_bf16(v);
      Y[h] = oracle_bf16_to_f32(b);
      if (y_bf16) y_bf16[t * H + h] = b;
    }
    for (int64_t j = 0; j < groups; ++j) {
      int64_t c0 = j * group;
      int64_t n = (H - c0 < group) ? H - c0 : group;
      y_s[t * groups + j] = oracle_quant_group(&Y[c0], n, 1, &y_q[t * H + c0], 1);
    }
  }
  free(Y);
  return ORACLE_OK;
}

/* The FP8 variant of the whole pass: the same intermediates, E4M3 codes. */
ORACLE_API int oracle_silu_dot_fwd_bwd_quant_fuse_fp8(const uint16_t* x, const uint16_t* grad_y, uint8_t* grad_input_q,
                                                      float* grad_input_s, uint8_t* y_q_t, float* y_s_t, int64_t T,
                                                      int64_t H, int64_t group) {
  if (T < 0 || H < 0 || group <= 0) return ORACLE_BAD_ARG;
  if (T == 0 || H == 0) return ORACLE_OK;
  float* Y = (float*)malloc((size_t)(T * H) * sizeof(float));
  float* D = (float*)malloc((size_t)(T * 2 * H) * sizeof(float));
  if (!Y || !D) {
    free(Y);
    free(D);
    return ORACLE_NO_MEMORY;
  }
  int rc = oracle_intermediates(x, grad_y, Y, D, T, H);
  if (rc == ORACLE_OK) {
    int64_t row_groups = (2 * H + group - 1) / group;
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < row_groups; ++j) {
        int64_t c0 = j * group;
        int64_t n = (2 * H - c0 < group) ? 2 * H - c0 : group;
        grad_input_s[t * row_groups + j] =
            oracle_quant_group_fp8(&D[t * 2 * H + c0], n, 1, &grad_input_q[t * 2 * H + c0], 1);
      }
    int64_t col_groups = (T + group - 1) / group;
    for (int64_t h = 0; h < H; ++h)
      for (int64_t j = 0; j < col_groups; ++j) {
        int64_t t0 = j * group;
        int64_t n = (T - t0 < group) ? T - t0 : group;
        y_s_t[h * col_groups + j] = oracle_quant_group_fp8(&Y[t0 * H + h], n, H, &y_q_t[h * T + t0], 1);
      }
  }
  free(Y);
  free(D);
  return rc;
}

/* ---- IEEE binary16 and the q8_1 block layout -------------------------------- */

/* Nearest binary16 bit pattern of x (ties to even), subnormals (k * 2^-24)
 * kept, infinity from 65520 up (the midpoint between 65504 and 2^16); NaN is
 * outside the domain.  Works in double, where every step below is exact. */
ORACLE_API uint16_t oracle_f32_to_f16(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  double a = fabs((double)x);
  if (isinf(a)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) {                  /* below 2^-14: subnormals k * 2^-24, k = 0..1024 */
    double k = nearbyint(a * ldexp(1.0, 24)); /* k == 1024 is the smallest normal, 2^-14 */
    return sign | (uint16_t)k;                /* and encodes as exponent field 1, mantissa 0 */
  }
  int e;
  double m = frexp(a, &e);             /* a = m * 2^e, m in [0.5, 1) */
  double mant = nearbyint(m * 2048.0); /* 1024 .. 2048: the leading one plus 10 fraction bits */
  if (mant == 2048.0) {
    mant = 1024.0;
    e += 1;
  }
  int efield = e - 1 + 15;
  if (efield >= 31) return sign | 0x7C00; /* past 65504: infinity */
  return sign | (uint16_t)(efield << 10) | (uint16_t)((int)mant - 1024);
}

/* The forward quantiser's output in the block_q8_1 layout of the page
 * "kquant_mmq.rs": per row, H/32 blocks of 32 channels, 36 bytes each.  The
 * page gives a block's content (32 int8 codes and a half2 (d, sum)) and size,
 * not the byte order or what the sum adds up; the readings here: bytes 0-1
 * hold d, the group-32 scale above rounded to binary16; bytes 2-3 the sum,
 * fl32(scale * sum(q)) rounded to binary16, i.e. the block's values as its
 * codes give them; bytes 4-35 the codes, both halves little-endian.  H must be
 * a multiple of 32 (the page's k % 32 == 0). */
/* One 36-byte block from 32 codes and their scale (the layout read above). */
static void oracle_q8_1_block(const int8_t* qb, float scale, uint8_t* blk) {
  int sum = 0;
  for (int i = 0; i < 32; ++i) sum += qb[i];
  float dequant_sum = scale * (float)sum;
  uint16_t d16 = oracle_f32_to_f16(scale), s16 = oracle_f32_to_f16(dequant_sum);
  blk[0] = (uint8_t)(d16 & 0xFF);
  blk[1] = (uint8_t)(d16 >> 8);
  blk[2] = (uint8_t)(s16 & 0xFF);
  blk[3] = (uint8_t)(s16 >> 8);
  memcpy(blk + 4, qb, 32);
}

ORACLE_API int oracle_silu_fwd_quant_q8_1(const uint16_t* x, const float* w, uint8_t* blocks, int64_t T, int64_t H) {
  if (T < 0 || H < 0 || H % 32 != 0) return ORACLE_BAD_ARG;
  if (T == 0 || H == 0) return ORACLE_OK;
  int64_t nb = H / 32;
  int8_t* q = (int8_t*)malloc((size_t)(T * H));
  float* sc = (float*)malloc((size_t)(T * nb) * sizeof(float));
  if (!q || !sc) {
    free(q);
    free(sc);
    return ORACLE_NO_MEMORY;
  }
  int rc = oracle_silu_fwd_quant(x, w, q, sc, NULL, T, H, 32);
  for (int64_t t = 0; rc == ORACLE_OK && t < T; ++t)
    for (int64_t b = 0; b < nb; ++b) oracle_q8_1_block(q + t * H + 32 * b, sc[t * nb + b], blocks + (t * nb + b) * 36);
  free(q);
  free(sc);
  return rc;
}

/* The fused launch of the page "kquant_mmq.rs" in its own argument shape
 * (kquant_swiglu_q8_1_rows): gate and up are separate bf16 [rows, inter]
 * arrays, w an optional fp32 weight per row, and the call writes both
 * h = bf16((silu(gate) * up) * w[row]) [rows, inter] (when h_bf16 is not
 * NULL) and the q8_1 blocks of h [rows, inter/32 * 36].  inter must be a
 * multiple of 32.  Row by row: h as in oracle_silu_fwd_quant, then per 32
 * channels the group quantiser and the block above.  The page's `limit`
 * argument has no stated meaning and is not modelled. */
ORACLE_API int oracle_kquant_swiglu_q8_1_rows(const uint16_t* gate, const uint16_t* up, const float* w,
                                              uint16_t* h_bf16, uint8_t* blocks, int64_t rows, int64_t inter) {
  if (rows < 0 || inter < 0 || inter % 32 != 0) return ORACLE_BAD_ARG;
  if (rows == 0 || inter == 0) return ORACLE_OK;
  int64_t nb = inter / 32;
  float* Y = (float*)malloc((size_t)inter * sizeof(float));
  if (!Y) return ORACLE_NO_MEMORY;
  for (int64_t t = 0; t < rows; ++t) {
    for (int64_t h = 0; h < inter; ++h) {
      float g = oracle_bf16_to_f32(gate[t * inter + h]);
      float u = oracle_bf16_to_f32(up[t * inter + h]);
      float s = oracle_sigmoid(g);
      float silu = g * s;
      float v = silu * u;
      if (w) v = v * w[t];
      uint16_t b = oracle_f32_to_bf16(v);
      Y[h] = oracle_bf16_to_f32(b);
      if (h_bf16) h_bf16[t * inter + h] = b;
    }
    for (int64_t b = 0; b < nb; ++b) {
      int8_t qb[32];
      float scale = oracle_quant_group(&Y[32 * b], 32, 1, qb, 1);
      oracle_q8_1_block(qb, scale, blocks + (t * nb + b) * 36);
    }
  }
  free(Y);
  return ORACLE_OK;
}

/* ---- the group-scaled int8 product ------------------------------------------ */

ORACLE_API int oracle_i8_gemm_group_scaled(const int8_t* A, const float* sA, const int8_t* B, const float* sB,
                                           double* C, double* C_abs, int64_t M, int64_t N, int64_t K,
                                           int64_t group, int64_t b_rows_per_scale) {
  if (M < 0 || N < 0 || K < 0 || group <= 0 || K % group != 0 || b_rows_per_scale <= 0) return ORACLE_BAD_ARG;
  const int64_t groups = K / group;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0, sum_abs = 0.0;
      for (int64_t g = 0; g < groups; ++g) {
        int64_t dot = 0;
        for (int64_t k = g * group; k < (g + 1) * group; ++k) dot += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
        double term = (double)sA[m * groups + g] * (double)sB[(n / b_rows_per_scale) * groups + g] * (double)dot;
        sum += term;
        sum_abs += fabs(term);
      }
      C[m * N + n] = sum;
      if (C_abs) C_abs[m * N + n] = sum_abs;
    }
  }
  return ORACLE_OK;
}

ORACLE_API int oracle_silu_dot_fwd_bwd_quant_fuse(const uint16_t* x, const uint16_t* grad_y, int8_t* grad_input_q,
                                                  float* grad_input_s, int8_t* y_q_t, float* y_s_t, int64_t T,
                                                  int64_t H, int64_t group) {
  if (T < 0 || H < 0 || group <= 0) return ORACLE_BAD_ARG;
  if (T == 0 || H == 0) return ORACLE_OK;
  float* Y = (float*)malloc((size_t)(T * H) * sizeof(float));
  float* D = (float*)malloc((size_t)(T * 2 * H) * sizeof(float));
  if (!Y || !D) {
    free(Y);
    free(D);
    return ORACLE_NO_MEMORY;
  }
  int rc = oracle_intermediates(x, grad_y, Y, D, T, H);
  if (rc == ORACLE_OK) rc = oracle_quantise(Y, D, grad_input_q, grad_input_s, y_q_t, y_s_t, T, H, group);
  free(Y);
  free(D);
  return rc;
}
