// Extend (chunked prefill) over an NVFP4 cache: the workspace the attention reads.
//
// The NVFP4 article (aitop.news), implementation item 2: for a chunk of new tokens, the
// cached prefix of the request is gathered and dequantized into an FP8 workspace, the chunk's
// own KV is appended to it, attention runs over workspace + chunk, and the chunk is then
// quantized into the NVFP4 cache (item 1).  Here:
//   - extend_gather_kernel builds one region of region_rows FP8 rows per request: rows
//     0 .. P-1 are the prefix (pool rows through the page table, value
//     e4m3(fl32(fl32(fl32(e2m1 * e4m3) * g) / chunk_scale))), rows P .. P+C-1 are the chunk's
//     FP8 rows copied as they are, so every workspace byte is in the chunk's scale domain;
//   - extend_index_kernel gives chunk token i of the request its causal length, P + i + 1
//     rows of the region (the token sees the prefix, the chunk tokens before it and itself),
//     and a range of region pages in a per-token numbering that the merge kernel's bounds
//     check reads; tokens of invalid requests get NaN outputs here;
//   - extend_attn_kernel attends the chunk tokens over their rows, and kv_quantize_nvfp4
//     writes the chunk.
// Requests whose lengths or pages are out of range get a length of -1 (NaN outputs) and no
// workspace rows; a prefix page outside the pool gives NaN codes in its rows.
#pragma clang fp contract(off)
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

// bounds of request b: prefix length P, chunk length C, query offset q0; false if invalid
__device__ __forceinline__ bool extend_bounds(const ExtendArgs& a, int b, int& P, int& C, int& q0) {
  P = a.prefix_lens[b];
  q0 = a.qo_indptr[b];
  C = a.qo_indptr[b + 1] - q0;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  return P >= 0 && P <= a.max_prefix_len && C >= 0 && C <= a.max_chunk_len && q0 >= 0 && q0 + C <= a.num_q &&
         p0 >= 0 && p1 >= p0 && p1 <= a.kv_indptr[a.batch] && (int64_t)(p1 - p0) * a.page_size >= (int64_t)P;
}

// one thread per (row of the region, group of 64 dims = 4 blocks): grid
// (ceil(region_rows * 9 / 256), batch); 32 code bytes + 4 scale bytes in, 64 FP8 bytes out
__global__ __launch_bounds__(256) void extend_gather_kernel(ExtendArgs a) {
  const int b = blockIdx.y;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)a.region_rows * 9) return;
  const int r = (int)(gid / 9), k4 = (int)(gid - (int64_t)r * 9);
  int P, C, q0;
  if (!extend_bounds(a, b, P, C, q0) || r >= P + C) return;
  u32x4* dst = reinterpret_cast<u32x4*>(a.ws_rows + ((int64_t)b * a.region_rows + r) * kD + 64 * k4);
  if (r >= P) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.chunk_kv + (int64_t)(q0 + r - P) * kD + 64 * k4);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = src[j];
    return;
  }
  const int page = a.kv_indices[a.kv_indptr[b] + (r >> a.page_shift)];
  const int64_t row = ((int64_t)page << a.page_shift) + (r & (a.page_size - 1));
  if (page < 0 || row >= a.pool_tokens) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = u32x4{0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
    return;
  }
  const u32x4* cp = reinterpret_cast<const u32x4*>(a.kv_data + row * kNvData + 32 * k4);
  const u32x4 d0 = cp[0], d1 = cp[1];
  const uint32_t sw = *reinterpret_cast<const uint32_t*>(a.kv_scales + row * kNvScale + 4 * k4);
  const uint32_t codes[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {          // block 4 k4 + blk: code words 2 blk, 2 blk + 1
    const float s = fp8x2_to_f32<false>((sw >> (8 * blk)) & 0xffu)[0];
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t cw = codes[2 * blk + h];
      const f32x2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
      const f32x2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
      const f32x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
      const f32x2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
      const float c[8] = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (c[i] * s) * a.global_scale;
      if (a.chunk_scale != 1.0f) {   // uniform; x / 1 == x, so the common case skips the divisions
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = v[i] / a.chunk_scale;
      }
      o[2 * h] = f32x2_to_e4m3(v[0], v[1]) | (f32x2_to_e4m3(v[2], v[3]) << 16);
      o[2 * h + 1] = f32x2_to_e4m3(v[4], v[5]) | (f32x2_to_e4m3(v[6], v[7]) << 16);
    }
    dst[blk] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

// one workgroup of 64 threads per query token t (grid num_q): its request (binary search in
// qo_indptr), its length P + i + 1 and its page range (region_rows / 64 pages from t * that)
__global__ __launch_bounds__(64) void extend_index_kernel(ExtendArgs a) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int npp = a.region_rows / kExtendPage;
  if (lane == 0) {
    a.view_indptr[t] = t * npp;
    if (t == a.num_q - 1) a.view_indptr[a.num_q] = a.num_q * npp;
  }
  // request of token t: the largest b with qo_indptr[b] <= t (qo_indptr is read as given;
  // an inconsistent table only yields invalid lengths)
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qo_indptr[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  int P, C, q0;
  const bool ok = extend_bounds(a, b, P, C, q0) && t >= q0 && t < q0 + C;
  if (lane == 0) a.view_lens[t] = ok ? P + (t - q0) + 1 : -1;
  if (!ok && a.nan_out) {   // the attention skips invalid requests: their outputs are NaN
    const int H = a.num_heads;
    float* o = a.nan_out + (int64_t)t * H * kDV;
    for (int k = lane; k < H * kDV; k += 64) o[k] = NAN;
    if (a.nan_lse)
      for (int k = lane; k < H; k += 64) a.nan_lse[(int64_t)t * H + k] = NAN;
  }
}

hipError_t launch_extend_views(const ExtendArgs& a, hipStream_t stream) {
  if (a.region_rows > 0) {
    const int64_t n = (int64_t)a.region_rows * 9;
    hipLaunchKernelGGL(extend_gather_kernel, dim3((unsigned)((n + 255) / 256), (unsigned)a.batch), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(extend_index_kernel, dim3((unsigned)a.num_q), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlaq
