// Internal interface between the host-side C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlaq {

enum KvFormat { FMT_BF16 = 0, FMT_FP8 = 1, FMT_NVFP4 = 2 };

// Decode work decomposition, shared by the kernel and the host split planner.  A workgroup
// runs `streams` online-softmax streams of 32 tokens per tile (2 waves per stream), and
// 160 KB of LDS holds 4 / streams workgroups per CU.  NVFP4 tiles are bound by the
// conversion arithmetic and the per-tile chain of the wave pair, so they take single-stream
// workgroups, whose barrier covers only the pair that swaps scores; FP8 and BF16 tiles carry
// two to four times the bytes per token, so they take two-stream workgroups, which halve the
// split partials.
constexpr int decode_streams(int fmt) { return fmt == FMT_NVFP4 ? 1 : 2; }
constexpr int decode_tile(int streams) { return 32 * streams; }
constexpr int decode_groups_per_cu(int streams) { return 4 / streams; }
constexpr int kComputeUnits = 256;

struct DecodeArgs {
  const uint16_t* q;          // bf16 [B, H, 576]
  const uint8_t* kv;          // FP8 [pool, 576] | NVFP4 codes [pool, 288] | BF16 [pool, 576]
  const uint8_t* kv_scales;   // NVFP4 [pool, 36]
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_lens;
  float* out;                 // [B, H, 512]
  float* lse;                 // [B, H] or null
  float* part_o;              // [B, part_splits, H/16, 16, 512]
  float* part_ml;             // [B, part_splits, H/16, 32]: m (16) then l (16)
  int64_t pool_tokens;
  int32_t batch, num_heads, page_size, max_kv_len, num_splits, chunk_tokens;
  int32_t part_splits;        // partial slots per (request, head group): num_splits (+ 1 with a fused append)
  int32_t page_shift;         // log2(page_size) (page sizes are powers of two)
  // pool pages for the page-tile check: ids in [0, pool_pages) are whole pages of the pool, and
  // page id pool_pages holds pool_tail rows (0: none); with more than 2^31 - 1 pages, every
  // non-negative id is a whole page (pool_pages = 2^31 - 1, pool_tail = page_size)
  int32_t pool_pages, pool_tail;
  float score_scale;          // sm_scale * (kv scale or global scale) * log2(e)
  float out_scale;            // kv scale or global scale
  // fused append (NVFP4 only): the last token of every request is the new row app_src[b],
  // quantized into its pool row and turned into an extra partial by the split kernel
  const void* app_src;        // FP8 bytes or bf16 bits [B, 576], or null (no append)
  uint8_t* app_data;          // the pool's code and scale arrays, written
  uint8_t* app_scales;
  float app_src_scale;        // FP8 source multiplier
  int32_t app_bf16;           // 1: bf16 source
};

struct ProfileEvents {
  hipEvent_t split_start = nullptr, split_end = nullptr, merge_start = nullptr, merge_end = nullptr;
};
hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev);
// device address of the allocation-free decode's scratch on the current device (looked up once
// per device)
hipError_t noalloc_scratch(void** ptr);

struct QuantArgs {
  const void* src;            // FP8 bytes or bf16 bits [n, 576]
  const int64_t* slots;       // [n]
  uint8_t* kv_data;           // [pool, 288]
  uint8_t* kv_scales;         // [pool, 36]
  int64_t num_tokens, pool_tokens;
  float src_scale, global_scale;
  int src_bf16;
};
hipError_t launch_quantize_nvfp4(const QuantArgs& a, hipStream_t stream);

struct DequantArgs {
  const uint8_t* kv_data;
  const uint8_t* kv_scales;   // NVFP4 only
  const int64_t* rows;        // or null
  void* dst;
  int64_t num_rows, pool_tokens;
  float scale;
  int src_nvfp4;              // 0: FP8 source, 1: NVFP4 source
  int dst_format;             // 0 bf16, 1 fp8, 3 fp32 (mlaq_format values)
};
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);

// Extend over an NVFP4 cache: per-request FP8 workspace regions and per-token causal views.
constexpr int kExtendPage = 64;   // rows per page of the workspace views
struct ExtendArgs {
  const int32_t* qo_indptr;   // [B + 1] chunk-token offsets
  const int32_t* prefix_lens; // [B]
  const int32_t* kv_indptr;   // cache page table of the prefixes
  const int32_t* kv_indices;
  const uint8_t* kv_data;     // NVFP4 cache
  const uint8_t* kv_scales;
  const uint8_t* chunk_kv;    // e4m3fn [num_q, 576]
  uint8_t* ws_rows;           // e4m3fn [B, region_rows, 576]
  int32_t* view_indptr;       // [num_q + 1] token t: rows t * region pages (bounds for the merge)
  int32_t* view_lens;         // [num_q] rows token t sees, or -1
  float* nan_out;             // outputs [num_q, num_heads, 512] of invalid tokens set to NaN here
  float* nan_lse;             // (one split; with several the merge writes them)
  int64_t pool_tokens;
  int32_t batch, num_q, num_heads, page_size, page_shift, max_prefix_len, max_chunk_len, region_rows;
  float global_scale, chunk_scale;
};
hipError_t launch_extend_views(const ExtendArgs& a, hipStream_t stream);

// Extend attention with one shared K/V tile per workgroup of kXT chunk tokens and 16 heads.
struct ExtendAttnArgs {
  const uint16_t* q;          // bf16 [num_q, num_heads, 576]
  const uint8_t* ws_rows;     // e4m3fn [batch, region_rows, 576]
  const int32_t* qo_indptr;
  const int32_t* prefix_lens;
  const int32_t* kv_indptr;   // cache page table (bounds check of the prefix only)
  float* out;                 // [num_q, num_heads, 512] (one split)
  float* lse;
  float* part_o;              // [num_q, num_splits, num_heads / 16, 16, 512] (several splits)
  float* part_ml;             // [num_q, num_splits, num_heads / 16, 32]
  int32_t batch, num_q, num_heads, page_size, max_prefix_len, max_chunk_len, region_rows, num_splits,
      tiles_per_split;
  float score_scale, out_scale;
};
hipError_t launch_extend_attn(const ExtendAttnArgs& a, hipStream_t stream);
int extend_attn_tile_rows();
int extend_attn_tokens_per_group();
// the merge pass of the decode kernels on its own (partials already written)
hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream);
// streaming-read probe: `words` 16-byte words of buf, one 16-byte XOR per block to partials
hipError_t launch_read_probe(const void* buf, int64_t words, void* partials, int blocks, hipStream_t stream);

}  // namespace mlaq
