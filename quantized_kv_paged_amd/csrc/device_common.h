// Device helpers shared by the mlaq kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlaq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 4-byte-aligned vector for loads from rows whose base is only dword aligned
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kD = 576;       // latent row: kv_lora_rank 512 + rope 64
constexpr int kDV = 512;      // value dims (latent part)
constexpr int kNvData = 288;  // NVFP4 code bytes per row
constexpr int kNvScale = 36;  // NVFP4 scale bytes per row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two e4m3fn bytes (low or high 16 bits of w) -> two fp16, exact (every e4m3fn value is an
// fp16 value).  The scale operand of the gfx950 scaled conversion only applies the
// exponent of its argument, so it is kept at 1.0 here and scales are applied separately.
template <bool HI>
__device__ __forceinline__ f16x2 fp8x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Two E2M1 nibbles (byte SEL of w; low nibble first) -> two fp16, exact.
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two e4m3fn bytes -> two fp32, exact.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer loads (gfx9 buffer descriptor: base, no stride, size in bytes, 32-bit data
// format).  Lanes whose offset lies outside [0, size) read zeros.
typedef __amdgpu_buffer_rsrc_t BufferRsrc;
__device__ __forceinline__ BufferRsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load_b128(BufferRsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ u32x2 buffer_load_b64(BufferRsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
__device__ __forceinline__ uint32_t buffer_load_b32(BufferRsrc r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}

// Transposed 64-bit LDS read of 16-bit elements.  Within each group of 16 lanes, lane j
// receives, as element c, 16-bit component (j % 4) of the 8 bytes addressed by lane
// 4c + j / 4 of the same group (checked on gfx950 with an in-bounds index pattern).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), on the VALU:
// with both operands equal, v_permlane16_swap returns (row pairs' even rows, odd rows) and
// v_permlane32_swap (lower half, upper half), so op(r[0], r[1]) combines the partners
// (lane mapping checked on gfx950 with an in-bounds index pattern).
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  x = fmaxf(u2f(a[0]), u2f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(b[0]), u2f(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  x = u2f(a[0]) + u2f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(b[0]) + u2f(b[1]);
}

// 2^x on the hardware exponential (arguments here are <= 0; results below the fp32 normal
// range flush to zero, which only drops weights under 2^-126 of the running maximum).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even, quiet NaN kept.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> e4m3fn byte: round to nearest even, saturate to +-448, NaN -> 0x7F, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float x) {
  uint32_t u = f2u(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __builtin_fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of step 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  int e = (int)((f2u(a) >> 23) & 0xff) - 127;                 // -6 .. 8
  float q = __builtin_rintf(a * u2f((uint32_t)(127 + 3 - e) << 23));  // 8 .. 16
  return sign | ((uint32_t)(e + 7) << 3) + ((uint32_t)q - 8u);
}

// Two fp32 values -> two e4m3fn bytes (lo in bits 0-7, hi in bits 8-15), the same bytes as
// f32_to_e4m3_rne_sat.  gfx950's fp8 conversion rounds to nearest even like it for every
// magnitude up to 464 but gives NaN above that, and NaN inputs come out as 0xFF; so the inputs
// are clamped to +-448 first (RNE takes (448, 464] to 448 as well) and NaN inputs get 0x7F.
// Checked on the GPU against f32_to_e4m3_rne_sat for every fp32 bit pattern.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float lo, float hi) {
  const float cl = __builtin_amdgcn_fmed3f(lo, -448.0f, 448.0f);
  const float ch = __builtin_amdgcn_fmed3f(hi, -448.0f, 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl, ch, 0, false) & 0xffffu;
  w = lo != lo ? (w & 0xff00u) | 0x7fu : w;
  w = hi != hi ? (w & 0x00ffu) | 0x7f00u : w;
  return w;
}

// Two fp32 values -> two E2M1 nibbles (low nibble = lo) written to byte SEL of w: round to
// nearest even on {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating, sign kept (-0 -> 0x8).  gfx950's
// scaled fp4 conversion at scale 1.0 rounds exactly this way: it gave the same nibble as the
// threshold form (count of the grid midpoints below |y|, a midpoint whose upper neighbour has an
// odd code passed only strictly) for every non-NaN fp32 bit pattern, checked on the GPU; NaN
// inputs never reach it.
template <int SEL>
__device__ __forceinline__ uint32_t f32x2_to_e2m1(uint32_t w, float lo, float hi) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, lo, hi, 1.0f, SEL);
}

// One NVFP4 block of 16 fp32 values x with global scale g (NVFP4 article, format section;
// quantize-on-write, implementation item 1): scale byte sb = e4m3_sat(fl32(fl32(amax / 6) / g)),
// divisor sd = fl32(e4m3(sb) * g), codes e2m1_sat(fl32(x_i / sd)) packed low nibble first
// (0 when sd == 0); a NaN in the block gives sb = 0x7F and zero codes.  IEEE fp32 division
// and no contraction, so the bytes are the same in every kernel that quantizes.
__device__ __forceinline__ void nvfp4_quantize_block(const float (&x)[16], float g, u32x2& packed, uint32_t& sb) {
#pragma clang fp contract(off)
  bool has_nan = false;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    has_nan |= x[i] != x[i];
    amax = fmaxf(amax, __builtin_fabsf(x[i]));
  }
  packed = u32x2{0u, 0u};
  if (has_nan) {
    sb = 0x7Fu;
    return;
  }
  const float sf = (amax / 6.0f) / g;
  sb = f32_to_e4m3_rne_sat(sf);
  const float sd = fp8x2_to_f32<false>(sb)[0] * g;
  if (sd != 0.0f) {
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = x[i] / sd;
    uint32_t w0 = 0u, w1 = 0u;
    w0 = f32x2_to_e2m1<0>(w0, y[0], y[1]);
    w0 = f32x2_to_e2m1<1>(w0, y[2], y[3]);
    w0 = f32x2_to_e2m1<2>(w0, y[4], y[5]);
    w0 = f32x2_to_e2m1<3>(w0, y[6], y[7]);
    w1 = f32x2_to_e2m1<0>(w1, y[8], y[9]);
    w1 = f32x2_to_e2m1<1>(w1, y[10], y[11]);
    w1 = f32x2_to_e2m1<2>(w1, y[12], y[13]);
    w1 = f32x2_to_e2m1<3>(w1, y[14], y[15]);
    packed = u32x2{w0, w1};
  }
}

// The 16 source values of block k of a 576-value row: bf16 bits (exact widening) or e4m3fn
// bytes times src_scale (fl32).
__device__ __forceinline__ void load_src_block(const void* row, bool bf16, float src_scale, int k, float (&x)[16]) {
#pragma clang fp contract(off)
  if (bf16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(row) + 16 * k);
    const u32x4 v0 = p[0], v1 = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = u2f(v0[e] << 16);
      x[2 * e + 1] = u2f(v0[e] & 0xffff0000u);
      x[8 + 2 * e] = u2f(v1[e] << 16);
      x[8 + 2 * e + 1] = u2f(v1[e] & 0xffff0000u);
    }
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(row) + 16 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo = fp8x2_to_f32<false>(v[e]), hi = fp8x2_to_f32<true>(v[e]);
      x[4 * e] = lo[0] * src_scale;
      x[4 * e + 1] = lo[1] * src_scale;
      x[4 * e + 2] = hi[0] * src_scale;
      x[4 * e + 3] = hi[1] * src_scale;
    }
  }
}

}  // namespace mlaq
