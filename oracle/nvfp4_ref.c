/* NVFP4 block quantizer, C twin of oracle/nvfp4.py::quantize_block (oracle).
 *
 * Test infrastructure: only the test suite, the smoke check and the benchmark's CPU
 * baseline load this file's library.  It shares no code with the GPU library.
 *
 * Format: NVFP4 article (aitop.news), section "NVFP4 format: two-level scaling" --
 * E2M1 values, one E4M3 scale per 16-value block, one FP32 global scale.
 * Write path: same article, implementation item 1 (FP8 KV quantized to NVFP4 on write).
 *
 * Per block of 16 fp32 values x[0..15] and global scale g (all arithmetic IEEE fp32,
 * round to nearest even, no contraction -- built with -ffp-contract=off):
 *   1. any NaN in the block  -> scale byte 0x7F, all codes 0
 *   2. a  = max |x_i|
 *   3. sf = (a / 6) / g
 *   4. sb = E4M3 encode of sf (nearest finite e4m3fn value, ties to even, saturating)
 *   5. sd = decode(sb) * g
 *   6. sd == 0 -> all codes 0
 *   7. code_i = E2M1 encode of x_i / sd (nearest, ties to even, saturating, sign kept)
 * A 576-value row is 36 such blocks; packed byte j = code(2j) | code(2j+1) << 4.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define BLOCK 16
#define ROW 576

/* e4m3fn: sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0; 0x7F/0xFF NaN. */
static double e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 0xF, m = code & 7;
  double mag;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0) mag = (m / 8.0) * ldexp(1.0, -6);
  else mag = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -mag : mag;
}

/* E2M1: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0. */
static double e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : (1.0 + m / 2.0) * ldexp(1.0, e - 1);
  return s ? -mag : mag;
}

/* Nearest entry of an increasing non-negative grid to a >= 0, ties to the even index,
 * saturating at the last entry. */
static int nearest_even(double a, const double* grid, int n) {
  if (a >= grid[n - 1]) return n - 1;
  int best = 0;
  double best_d = fabs(a - grid[0]);
  for (int k = 1; k < n; ++k) {
    double d = fabs(a - grid[k]);
    if (d < best_d || (d == best_d && (k % 2) == 0 && (best % 2) == 1)) { best = k; best_d = d; }
  }
  return best;
}

static double E4M3_GRID[127];
static double E2M1_GRID[8];
static int grids_ready = 0;

static void init_grids(void) {
  if (grids_ready) return;
  for (int c = 0; c < 127; ++c) E4M3_GRID[c] = e4m3_value(c);
  for (int c = 0; c < 8; ++c) E2M1_GRID[c] = e2m1_value(c);
  grids_ready = 1;
}

int oracle_e4m3_encode_f32(float x) {
  init_grids();
  if (isnan(x)) return 0x7F;
  int sign = signbit(x) ? 0x80 : 0;
  return sign | nearest_even(fabs((double)x), E4M3_GRID, 127);
}

int oracle_e2m1_encode_f32(float y) {
  init_grids();
  int sign = signbit(y) ? 0x8 : 0;
  return sign | nearest_even(fabs((double)y), E2M1_GRID, 8);
}

static void quantize_block(const float* x, float g, uint8_t* scale_out, int* codes) {
  for (int i = 0; i < BLOCK; ++i)
    if (isnan(x[i])) { *scale_out = 0x7F; memset(codes, 0, sizeof(int) * BLOCK); return; }
  float a = 0.0f;
  for (int i = 0; i < BLOCK; ++i) { float v = fabsf(x[i]); if (v > a) a = v; }
  volatile float t = a / 6.0f;      /* volatile: keep each fp32 rounding step explicit */
  float sf = t / g;
  int sb = oracle_e4m3_encode_f32(sf);
  float sd = (float)e4m3_value(sb) * g;
  *scale_out = (uint8_t)sb;
  if (sd == 0.0f) { memset(codes, 0, sizeof(int) * BLOCK); return; }
  for (int i = 0; i < BLOCK; ++i) {
    float y = x[i] / sd;
    codes[i] = oracle_e2m1_encode_f32(y);
  }
}

/* rows of 576 fp32 values -> packed codes [rows, 288] and scales [rows, 36] */
void oracle_nvfp4_quantize_f32_rows(const float* src, int64_t rows, float g, uint8_t* data, uint8_t* scales) {
  init_grids();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int codes[BLOCK];
    for (int k = 0; k < ROW / BLOCK; ++k) {
      quantize_block(src + r * ROW + k * BLOCK, g, scales + r * (ROW / BLOCK) + k, codes);
      for (int j = 0; j < BLOCK / 2; ++j)
        data[r * (ROW / 2) + k * (BLOCK / 2) + j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
    }
  }
}

/* FP8 source -> fp32 x = fl32(e4m3(c) * src_scale) */
void oracle_fp8_rows_to_f32(const uint8_t* src, int64_t n, float src_scale, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)e4m3_value(src[i]) * src_scale;
}

/* bf16 bits -> fp32 (exact widening) */
void oracle_bf16_rows_to_f32(const uint16_t* src, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b = (uint32_t)src[i] << 16;
    memcpy(&out[i], &b, 4);
  }
}

/* e4m3 encode of an array (nearest, ties to even, saturating; NaN -> 0x7F) */
void oracle_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
  init_grids();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_e4m3_encode_f32(x[i]);
}

/* NVFP4 rows -> fp32 values fl32(fl32(e2m1 * e4m3) * g) */
void oracle_nvfp4_dequant_f32_rows(const uint8_t* data, const uint8_t* scales, int64_t rows, float g, float* out) {
  init_grids();
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int d = 0; d < ROW; ++d) {
      uint8_t byte = data[r * (ROW / 2) + d / 2];
      int code = (d % 2) ? (byte >> 4) : (byte & 0xF);
      float prod = (float)e2m1_value(code) * (float)e4m3_value(scales[r * (ROW / BLOCK) + d / BLOCK]);
      out[r * ROW + d] = prod * g;
    }
}
