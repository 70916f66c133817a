// NVFP4 quantize-on-write and pool dequantization kernels.
//
// Quantize: the NVFP4 article (aitop.news) stores KV as E2M1 values with one E4M3 scale per
// 16 values and one FP32 global scale (format section) and writes the cache by
// quantizing FP8 KV to NVFP4 (implementation item 1).  Per 16-value block, all in IEEE
// fp32 with round-to-nearest-even and no contraction:
//   scale byte sb = e4m3_sat(fl32(fl32(amax / 6) / g));  sd = fl32(e4m3(sb) * g);
//   code_i = e2m1_sat(fl32(x_i / sd))  (0 when sd == 0; NaN block -> sb 0x7F, codes 0).
// One thread owns one block: it loads 16 source values with one 16- or 32-byte load and
// writes 8 code bytes and 1 scale byte; blocks of a row are adjacent threads, so the row's
// 288 code bytes are written as one contiguous span by 36 neighbouring lanes.
//
// Dequantize: fp32 value = fl32(fl32(e2m1 * e4m3) * g) for NVFP4 (fl32(e4m3 * s) for FP8),
// stored as fp32, as bf16 (round to nearest even) or re-encoded as e4m3 (NVFP4 source).
#pragma clang fp contract(off)
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(QuantArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.num_tokens * 36) return;
  const int64_t t = gid / 36;
  const int k = (int)(gid - t * 36);
  // the slot and the source block are loaded together; the slot is checked afterwards
  const int64_t slot = a.slots[t];
  float x[16];
  load_src_block(reinterpret_cast<const uint8_t*>(a.src) + t * kD * (a.src_bf16 ? 2 : 1), a.src_bf16, a.src_scale, k, x);
  if (slot < 0 || slot >= a.pool_tokens) return;
  u32x2 packed;
  uint32_t sb;
  nvfp4_quantize_block(x, a.global_scale, packed, sb);
  *reinterpret_cast<u32x2*>(a.kv_data + slot * kNvData + 8 * k) = packed;
  a.kv_scales[slot * kNvScale + k] = (uint8_t)sb;
}

__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.num_rows * 36) return;
  const int64_t r = gid / 36;
  const int k = (int)(gid - r * 36);
  const int64_t row = a.rows ? a.rows[r] : r;
  const bool ok = row >= 0 && row < a.pool_tokens;
  float v[16];
  if (!ok) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = NAN;
  } else if (a.src_nvfp4) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(a.kv_data + row * kNvData + 8 * k);
    const float s = fp8x2_to_f32<false>((uint32_t)a.kv_scales[row * kNvScale + k])[0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = d[h];
      f32x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      f32x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      f32x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
      f32x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      const float c[8] = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * h + i] = (c[i] * s) * a.scale;
    }
  } else {
    const u32x4 d = *reinterpret_cast<const u32x4*>(a.kv_data + row * kD + 16 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f32x2 lo = fp8x2_to_f32<false>(d[e]), hi = fp8x2_to_f32<true>(d[e]);
      v[4 * e] = lo[0] * a.scale;
      v[4 * e + 1] = lo[1] * a.scale;
      v[4 * e + 2] = hi[0] * a.scale;
      v[4 * e + 3] = hi[1] * a.scale;
    }
  }
  if (a.dst_format == 3) {
    f32x4* o = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dst) + r * kD + 16 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = f32x4{v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]};
  } else if (a.dst_format == 0) {
    u32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = (uint32_t)f32_to_bf16_rne(v[2 * e]) | ((uint32_t)f32_to_bf16_rne(v[2 * e + 1]) << 16);
      o1[e] = (uint32_t)f32_to_bf16_rne(v[8 + 2 * e]) | ((uint32_t)f32_to_bf16_rne(v[8 + 2 * e + 1]) << 16);
    }
    u32x4* o = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.dst) + r * kD + 16 * k);
    o[0] = o0;
    o[1] = o1;
  } else {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = f32x2_to_e4m3(v[4 * e], v[4 * e + 1]) | (f32x2_to_e4m3(v[4 * e + 2], v[4 * e + 3]) << 16);
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(a.dst) + r * kD + 16 * k) = o;
  }
}

hipError_t launch_quantize_nvfp4(const QuantArgs& a, hipStream_t stream) {
  const int64_t n = a.num_tokens * 36;
  hipLaunchKernelGGL(nvfp4_quantize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream) {
  const int64_t n = a.num_rows * 36;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlaq
