// Host side of the mlaq C ABI: argument validation, split planning, workspace layout and
// kernel launches.  Nothing here touches device memory or synchronises.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "../../include/mlaq.h"
#include "mlaq_kernels.h"

namespace {

thread_local std::string g_err;
thread_local mlaq::ProfileEvents g_events;

mlaq_status fail(mlaq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }


// Fewest splits whose chunks stay within MLAQ_MAX_SPLIT_TOKENS (the fp16 probability range).
int min_splits(int64_t max_kv_len) {
  return (int)std::max<int64_t>(1, (max_kv_len + MLAQ_MAX_SPLIT_TOKENS - 1) / MLAQ_MAX_SPLIT_TOKENS);
}

// Split planning.  Every workgroup processes one (request, chunk, 16-head group) in tiles of
// the format's tile size; with all requests at the host-known bound, workgroups run in
// "rounds" of the resident slots (CUs x workgroups per CU).  Costs are in tile-times, the time
// a workgroup takes for one tile when every slot is busy:
//   rounds * (tiles per chunk + fixed)       each workgroup streams its chunk and pays a
//                                           prologue / epilogue (page ids, first tile, stream
//                                           merge) of about one tile;
//   + crowd * (workgroups on the fullest CU) those fixed latencies grow with the workgroups that
//                                           share a CU (about 3 us each), which is why a small
//                                           batch runs faster on fewer, longer chunks;
//   + rounds * part + part * wgs / slots     with several splits, each workgroup writes a partial
//   + merge                                 and the merge kernel reads them all (its launch
//                                           about one tile-time);
// where part is a partial's bytes (16 heads x 512 fp32 + 32 fp32 = 32,896 B) over a tile's KV
// bytes: 3.2 tiles for NVFP4 (32 tokens x 324 B), 0.89 for FP8 (64 x 576 B), 0.45 for BF16 (64 x
// 1,152 B).  The smallest cost is taken (ties -> fewer splits).  The constants are fitted to
// forced-split sweeps at 12 shapes (32K to 1M tokens per request, 1 to 44 requests, both
// formats); the plan is the fastest measured split count at 11 of them and within 3 % at the
// other.
int plan_splits(int fmt, int batch, int head_groups, int max_kv_len) {
  const int streams = mlaq::decode_streams(fmt);
  const int tile = mlaq::decode_tile(streams);
  const double slots = (double)mlaq::kComputeUnits * mlaq::decode_groups_per_cu(streams);
  const int tiles = (max_kv_len + tile - 1) / tile;
  if (tiles <= 1 || batch <= 0) return 1;
  const double row_bytes = fmt == mlaq::FMT_NVFP4 ? 324.0 : fmt == mlaq::FMT_FP8 ? 576.0 : 1152.0;
  const double part = (16.0 * 512.0 * 4.0 + 32.0 * 4.0) / (tile * row_bytes);
  const double fixed = 1.2, crowd = 1.25, merge = 1.0;
  const int smin = min_splits(max_kv_len);
  int best = smin;
  double best_cost = std::numeric_limits<double>::infinity();
  const int smax = tiles < MLAQ_MAX_SPLITS ? tiles : MLAQ_MAX_SPLITS;
  for (int s = smin; s <= smax; ++s) {
    const double wgs = (double)batch * head_groups * s;
    const double rounds = std::ceil(wgs / slots);
    const double per = std::ceil((double)tiles / s);
    double cost = rounds * (per + fixed) + crowd * std::ceil(std::min(wgs, slots) / mlaq::kComputeUnits);
    if (s > 1) cost += rounds * part + part * wgs / slots + merge;
    if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
  }
  return best;
}

mlaq_status check_params(const mlaq_decode_params* p) {
  if (!p) return fail(MLAQ_ERR_NULL, "params is NULL");
  if (p->batch < 0 || p->batch > 65535) return fail(MLAQ_ERR_SHAPE, "batch %d not in [0, 65535]", p->batch);
  if (p->num_heads < 16 || p->num_heads > 128 || p->num_heads % 16)
    return fail(MLAQ_ERR_SHAPE, "num_heads %d: must be a multiple of 16 in [16, 128]", p->num_heads);
  if (p->page_size < 1 || p->page_size > 1024 || (p->page_size & (p->page_size - 1)))
    return fail(MLAQ_ERR_SHAPE, "page_size %d: must be a power of two in [1, 1024]", p->page_size);
  if (p->max_kv_len < 0 || p->max_kv_len > MLAQ_MAX_KV_LEN)
    return fail(MLAQ_ERR_SHAPE, "max_kv_len %d not in [0, %d]", p->max_kv_len, MLAQ_MAX_KV_LEN);
  if (p->pool_tokens <= 0 || p->pool_tokens > ((int64_t)1 << 40))
    return fail(MLAQ_ERR_SHAPE, "pool_tokens %lld out of range", (long long)p->pool_tokens);
  if (p->num_splits < 0 || p->num_splits > MLAQ_MAX_SPLITS)
    return fail(MLAQ_ERR_SHAPE, "num_splits %d not in [0, %d]", p->num_splits, MLAQ_MAX_SPLITS);
  if (p->num_splits > 0 && p->num_splits < min_splits(p->max_kv_len))
    return fail(MLAQ_ERR_SHAPE,
                "num_splits %d leaves chunks longer than %d tokens (max_kv_len %d needs at least %d splits)",
                p->num_splits, MLAQ_MAX_SPLIT_TOKENS, p->max_kv_len, min_splits(p->max_kv_len));
  if (!std::isfinite(p->sm_scale)) return fail(MLAQ_ERR_VALUE, "sm_scale is not finite");
  return MLAQ_OK;
}

int resolve_splits(int fmt, const mlaq_decode_params* p) {
  return p->num_splits > 0 ? p->num_splits : plan_splits(fmt, p->batch, p->num_heads / 16, p->max_kv_len);
}

// mlaq_format of a decode's KV pool -> kernel format; -1 if it is not a decode format
int kv_format_of(mlaq_format f) {
  return f == MLAQ_FP8_E4M3 ? mlaq::FMT_FP8 : f == MLAQ_NVFP4 ? mlaq::FMT_NVFP4 : f == MLAQ_BF16 ? mlaq::FMT_BF16 : -1;
}

// Fused append (NVFP4): the new rows and where they go.
struct AppendArgs {
  const void* src = nullptr;   // [B, 576] FP8 or bf16, or null: plain decode
  bool bf16 = false;
  float src_scale = 1.0f;
  uint8_t* data = nullptr;
  uint8_t* scales = nullptr;
};

// A single split writes the output directly; a fused append adds one partial slot per
// request (its new token) and always takes the merge pass.
size_t workspace_for(const mlaq_decode_params* p, int splits, bool append = false) {
  if (splits <= 1 && !append) return 0;
  const size_t slots = (size_t)p->batch * (size_t)(splits + (append ? 1 : 0)) * (size_t)(p->num_heads / 16);
  const size_t bytes = slots * (16 * 512 * sizeof(float)) + slots * 32 * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

mlaq_status decode_common(int fmt, const mlaq_decode_params* p, const uint16_t* q, const void* kv,
                          const uint8_t* kv_scales, float scale, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          const AppendArgs& app = AppendArgs()) {
  mlaq_status st = check_params(p);
  if (st != MLAQ_OK) return st;
  if (p->batch == 0) return MLAQ_OK;
  if (!q || !kv || !kv_indptr || !kv_indices || !kv_lens || !out)
    return fail(MLAQ_ERR_NULL, "a required pointer (q, kv, kv_indptr, kv_indices, kv_lens, out) is NULL");
  if (fmt == mlaq::FMT_NVFP4 && !kv_scales) return fail(MLAQ_ERR_NULL, "kv_scales is NULL");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16))
    return fail(MLAQ_ERR_ALIGN, "q, kv and out must be 16-byte aligned");
  if (fmt == mlaq::FMT_NVFP4 && !aligned(kv_scales, 4)) return fail(MLAQ_ERR_ALIGN, "kv_scales must be 4-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(MLAQ_ERR_ALIGN, "lse must be 4-byte aligned");
  if (!aligned(kv_indptr, 4) || !aligned(kv_indices, 4) || !aligned(kv_lens, 4))
    return fail(MLAQ_ERR_ALIGN, "kv_indptr, kv_indices and kv_lens must be 4-byte aligned");
  if (fmt != mlaq::FMT_BF16 && !finite_pos(scale))
    return fail(MLAQ_ERR_VALUE, "the KV scale must be finite and > 0 (got %g)", (double)scale);
  const int splits = resolve_splits(fmt, p);
  const size_t need = workspace_for(p, splits, app.src != nullptr);
  if (need > 0) {
    if (!workspace) return fail(MLAQ_ERR_NULL, "workspace is NULL but %zu bytes are needed", need);
    if (workspace_bytes < need)
      return fail(MLAQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(MLAQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  const int tile = mlaq::decode_tile(mlaq::decode_streams(fmt));
  const int tiles = (p->max_kv_len + tile - 1) / tile;
  const int per = (tiles + splits - 1) / splits;

  mlaq::DecodeArgs a;
  a.q = q;
  a.kv = static_cast<const uint8_t*>(kv);
  a.kv_scales = kv_scales;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.kv_lens = kv_lens;
  a.out = out;
  a.lse = lse;
  const int part_splits = splits + (app.src ? 1 : 0);
  const size_t slots = (size_t)p->batch * part_splits * (p->num_heads / 16);
  a.part_o = need ? static_cast<float*>(workspace) : nullptr;
  a.part_ml = need ? static_cast<float*>(workspace) + slots * 16 * 512 : nullptr;
  a.pool_tokens = p->pool_tokens;
  a.batch = p->batch;
  a.num_heads = p->num_heads;
  a.page_size = p->page_size;
  a.page_shift = __builtin_ctz((unsigned)p->page_size);
  {
    const int64_t pages = p->pool_tokens >> a.page_shift;
    const bool huge = pages > (int64_t)std::numeric_limits<int32_t>::max();   // else id 2^31 - 1 may be the partial page
    a.pool_pages = huge ? std::numeric_limits<int32_t>::max() : (int32_t)pages;
    a.pool_tail = huge ? p->page_size : (int32_t)(p->pool_tokens & (p->page_size - 1));
  }
  a.max_kv_len = p->max_kv_len;
  a.num_splits = splits;
  a.part_splits = part_splits;
  a.chunk_tokens = (per > 0 ? per : 1) * tile;
  const float s = fmt == mlaq::FMT_BF16 ? 1.0f : scale;
  a.score_scale = p->sm_scale * s * 1.4426950408889634f;
  a.out_scale = s;
  a.app_src = app.src;
  a.app_data = app.data;
  a.app_scales = app.scales;
  a.app_src_scale = app.src_scale;
  a.app_bf16 = app.bf16 ? 1 : 0;
  const mlaq::ProfileEvents ev = g_events;
  g_events = mlaq::ProfileEvents();
  hipError_t e = mlaq::launch_decode(fmt, a, stream, ev);
  if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

// Extend: workspace layout (FP8 regions, per-token lengths and page ranges, split partials),
// each part 256-byte aligned, the KV splits of the attention, and the decode parameters the
// merge kernel's bounds check reads (one "request" per chunk token).
struct ExtendLayout {
  int region_rows = 0, npp = 0;
  int tsplits = 1, tiles_per_split = 1;
  size_t rows_off = 0, lens_off = 0, indptr_off = 0, part_off = 0, part_bytes = 0, total = 0;
  mlaq_decode_params dp{};
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

mlaq_status extend_layout(const mlaq_extend_params* p, ExtendLayout& L) {
  if (!p) return fail(MLAQ_ERR_NULL, "params is NULL");
  if (p->batch < 0 || p->batch > 65535) return fail(MLAQ_ERR_SHAPE, "batch %d not in [0, 65535]", p->batch);
  if (p->num_q < 0 || p->num_q > 65535) return fail(MLAQ_ERR_SHAPE, "num_q %d not in [0, 65535]", p->num_q);
  if (p->max_prefix_len < 0 || p->max_chunk_len < 0 ||
      (int64_t)p->max_prefix_len + p->max_chunk_len > MLAQ_MAX_KV_LEN)
    return fail(MLAQ_ERR_SHAPE, "max_prefix_len %d / max_chunk_len %d out of range", p->max_prefix_len,
                p->max_chunk_len);
  if (p->num_q > 0 && p->max_chunk_len < 1) return fail(MLAQ_ERR_SHAPE, "num_q > 0 needs max_chunk_len >= 1");
  const int64_t span = (int64_t)p->max_prefix_len + p->max_chunk_len;
  L.region_rows = (int)((span + mlaq::kExtendPage - 1) / mlaq::kExtendPage * mlaq::kExtendPage);
  L.npp = L.region_rows / mlaq::kExtendPage;
  // the per-token page ranges are int32 offsets t * npp
  if ((int64_t)p->num_q * L.npp >= ((int64_t)1 << 31) || (int64_t)p->batch * L.npp >= ((int64_t)1 << 31))
    return fail(MLAQ_ERR_SHAPE, "extend views too large: num_q %d / batch %d x %d pages per region", p->num_q,
                p->batch, L.npp);
  L.dp.batch = p->num_q;
  L.dp.num_heads = p->num_heads;
  L.dp.page_size = mlaq::kExtendPage;
  L.dp.max_kv_len = (int32_t)span;
  L.dp.pool_tokens = (int64_t)(p->batch > 0 ? p->batch : 1) * (L.region_rows > 0 ? L.region_rows : 1);
  L.dp.num_splits = p->num_splits;
  L.dp.sm_scale = p->sm_scale;
  mlaq_status st = check_params(&L.dp);
  if (st != MLAQ_OK) return st;
  if (p->page_size < 1 || p->page_size > 1024 || (p->page_size & (p->page_size - 1)))
    return fail(MLAQ_ERR_SHAPE, "page_size %d: must be a power of two in [1, 1024]", p->page_size);
  if (p->pool_tokens <= 0 || p->pool_tokens > ((int64_t)1 << 40))
    return fail(MLAQ_ERR_SHAPE, "pool_tokens %lld out of range", (long long)p->pool_tokens);
  L.rows_off = 0;
  L.lens_off = align256((size_t)p->batch * L.region_rows * 576);
  L.indptr_off = L.lens_off + align256((size_t)p->num_q * 4);
  L.part_off = L.indptr_off + align256((size_t)(p->num_q + 1) * 4);
  {
    // KV splits: workgroups (one per kXT chunk tokens of a request and 16-head group, one per CU)
    // run in rounds of the CUs; each split takes whole 32-row tiles.  The automatic count
    // minimizes rounds x tiles per split (in tile-times) plus the partials each extra split
    // writes and the merge reads (measured: about 0.0105 tile-times per query token and 16-head
    // group and split), so the last round is not left mostly idle
    const int tile = mlaq::extend_attn_tile_rows(), per_group = mlaq::extend_attn_tokens_per_group();
    const int max_tiles = (int)((span + tile - 1) / tile);
    const int64_t groups = (int64_t)p->batch * ((p->max_chunk_len + per_group - 1) / per_group) * (p->num_heads / 16);
    // no split may cover more than MLAQ_MAX_SPLIT_TOKENS rows (the fp16 probability range)
    const int smin = min_splits(span);
    if (p->num_splits > 0 && p->num_splits < smin)
      return fail(MLAQ_ERR_SHAPE, "num_splits %d leaves chunks longer than %d rows (%lld rows need at least %d splits)",
                  p->num_splits, MLAQ_MAX_SPLIT_TOKENS, (long long)span, smin);
    int s_ = p->num_splits;
    if (s_ <= 0) {
      s_ = smin;
      double best = std::numeric_limits<double>::infinity();
      const int smax = std::max(smin, std::min(MLAQ_MAX_SPLITS, std::max(1, max_tiles)));
      for (int s = smin; s <= smax; ++s) {
        const double rounds = std::ceil((double)groups * s / mlaq::kComputeUnits);
        const double per = std::ceil((double)max_tiles / s);
        const double cost = rounds * per + (s > 1 ? 0.0105 * p->num_q * (p->num_heads / 16) * s : 0.0);
        if (cost < best - 1e-9) { best = cost; s_ = s; }
      }
    }
    s_ = std::max(smin, std::max(1, std::min(s_, std::max(1, max_tiles))));
    L.tiles_per_split = std::max(1, (max_tiles + s_ - 1) / s_);
    L.tsplits = (max_tiles + L.tiles_per_split - 1) / L.tiles_per_split;
    if (L.tsplits < 1) L.tsplits = 1;
    L.part_bytes = L.tsplits > 1 ? align256((size_t)p->num_q * L.tsplits * (p->num_heads / 16) * (16 * 512 * 4 + 32 * 4))
                                 : 0;
  }
  L.total = L.part_off + L.part_bytes;
  return MLAQ_OK;
}

}  // namespace

extern "C" {

const char* mlaq_last_error(void) { return g_err.c_str(); }

const char* mlaq_version(void) { return "mlaq 0.1 gfx950"; }

mlaq_status mlaq_set_profile_events(hipEvent_t split_start, hipEvent_t split_end, hipEvent_t merge_start,
                                    hipEvent_t merge_end) {
  g_events.split_start = split_start;
  g_events.split_end = split_end;
  g_events.merge_start = merge_start;
  g_events.merge_end = merge_end;
  return MLAQ_OK;
}

int32_t mlaq_decode_num_splits(const mlaq_decode_params* p, mlaq_format kv_format) {
  const int fmt = kv_format_of(kv_format);
  if (fmt < 0) { fail(MLAQ_ERR_UNSUPPORTED, "kv_format %d is not a decode KV format", (int)kv_format); return 0; }
  if (check_params(p) != MLAQ_OK) return 0;
  return resolve_splits(fmt, p);
}

size_t mlaq_decode_format_workspace_bytes(const mlaq_decode_params* p, mlaq_format kv_format) {
  const int fmt = kv_format_of(kv_format);
  if (fmt < 0) { fail(MLAQ_ERR_UNSUPPORTED, "kv_format %d is not a decode KV format", (int)kv_format); return SIZE_MAX; }
  if (check_params(p) != MLAQ_OK) return SIZE_MAX;
  return workspace_for(p, resolve_splits(fmt, p));
}

size_t mlaq_decode_workspace_bytes(const mlaq_decode_params* p) {
  if (check_params(p) != MLAQ_OK) return SIZE_MAX;
  size_t need = 0;
  for (int fmt : {mlaq::FMT_FP8, mlaq::FMT_NVFP4, mlaq::FMT_BF16}) need = std::max(need, workspace_for(p, resolve_splits(fmt, p)));
  return need;
}

mlaq_status mla_decode_fp8(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv, float kv_scale,
                           const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_lens, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(mlaq::FMT_FP8, p, q, kv, nullptr, kv_scale, kv_indptr, kv_indices, kv_lens, out, lse,
                       workspace, workspace_bytes, stream);
}

mlaq_status mla_decode_nvfp4(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv_data,
                             const uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(mlaq::FMT_NVFP4, p, q, kv_data, kv_scales, global_scale, kv_indptr, kv_indices, kv_lens,
                       out, lse, workspace, workspace_bytes, stream);
}

mlaq_status mla_decode_nvfp4_noalloc(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv_data,
                                     const uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                                     const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                                     hipStream_t stream) {
  mlaq_status st = check_params(p);
  if (st != MLAQ_OK) return st;
  if (p->batch == 0) return MLAQ_OK;
  const size_t cap = MLAQ_NOALLOC_SCRATCH_BYTES;
  mlaq_decode_params plan = *p;
  plan.num_splits = resolve_splits(mlaq::FMT_NVFP4, p);
  if (workspace_for(p, plan.num_splits) > cap) {
    // the automatic plan's partials do not fit: the largest split count whose partials do, if the
    // per-split token cap allows it; a forced count is the caller's and is rejected
    const size_t per_split = workspace_for(p, 2) / 2;   // one split's partials for the whole batch
    int fit = (int)std::min<size_t>(cap / per_split, (size_t)MLAQ_MAX_SPLITS);
    if (fit < 2) fit = 1;   // a single split writes the outputs directly and needs no partials
    if (p->num_splits > 0 || fit < min_splits(p->max_kv_len))
      return fail(MLAQ_ERR_WORKSPACE,
                  "noalloc decode: %d splits x batch %d x %d heads need %zu bytes of partials, the scratch holds %zu",
                  plan.num_splits, p->batch, p->num_heads, workspace_for(p, plan.num_splits), cap);
    plan.num_splits = fit;
  }
  const size_t need = workspace_for(&plan, plan.num_splits);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = mlaq::noalloc_scratch(&scratch);
    if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "noalloc decode: scratch lookup failed: %s", hipGetErrorString(e));
  }
  return decode_common(mlaq::FMT_NVFP4, &plan, q, kv_data, kv_scales, global_scale, kv_indptr, kv_indices, kv_lens,
                       out, lse, scratch, scratch ? cap : 0, stream);
}

size_t mlaq_decode_nvfp4_append_workspace_bytes(const mlaq_decode_params* p) {
  if (check_params(p) != MLAQ_OK) return SIZE_MAX;
  return workspace_for(p, resolve_splits(mlaq::FMT_NVFP4, p), true);
}

mlaq_status mla_decode_nvfp4_append(const mlaq_decode_params* p, const uint16_t* q, const void* new_kv,
                                    mlaq_format new_kv_format, float src_scale, uint8_t* kv_data,
                                    uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                                    const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (new_kv_format != MLAQ_FP8_E4M3 && new_kv_format != MLAQ_BF16)
    return fail(MLAQ_ERR_UNSUPPORTED, "mla_decode_nvfp4_append: new_kv format %d is not FP8_E4M3 or BF16",
                (int)new_kv_format);
  if (new_kv_format == MLAQ_FP8_E4M3 && !finite_pos(src_scale))
    return fail(MLAQ_ERR_VALUE, "src_scale must be finite and > 0");
  if (p && p->batch > 0) {
    if (!new_kv) return fail(MLAQ_ERR_NULL, "new_kv is NULL");
    if (!aligned(new_kv, 16)) return fail(MLAQ_ERR_ALIGN, "new_kv must be 16-byte aligned");
  }
  AppendArgs app;
  app.src = new_kv;
  app.bf16 = new_kv_format == MLAQ_BF16;
  app.src_scale = src_scale;
  app.data = kv_data;
  app.scales = kv_scales;
  return decode_common(mlaq::FMT_NVFP4, p, q, kv_data, kv_scales, global_scale, kv_indptr, kv_indices, kv_lens,
                       out, lse, workspace, workspace_bytes, stream, app);
}

size_t mlaq_extend_workspace_bytes(const mlaq_extend_params* p) {
  ExtendLayout L;
  if (extend_layout(p, L) != MLAQ_OK) return SIZE_MAX;
  return L.total;
}

int32_t mlaq_extend_num_splits(const mlaq_extend_params* p) {
  ExtendLayout L;
  if (extend_layout(p, L) != MLAQ_OK) return 0;
  return L.tsplits;
}

mlaq_status mla_extend_nvfp4(const mlaq_extend_params* p, const uint16_t* q, const int32_t* qo_indptr,
                             const uint8_t* chunk_kv, float chunk_scale, uint8_t* kv_data, uint8_t* kv_scales,
                             float global_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* prefix_lens, const int64_t* slot_mapping, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ExtendLayout L;
  mlaq_status st = extend_layout(p, L);
  if (st != MLAQ_OK) return st;
  if (!finite_pos(chunk_scale)) return fail(MLAQ_ERR_VALUE, "chunk_scale must be finite and > 0");
  if (!finite_pos(global_scale)) return fail(MLAQ_ERR_VALUE, "global_scale must be finite and > 0");
  if (p->batch == 0 || p->num_q == 0) return MLAQ_OK;
  if (!q || !qo_indptr || !chunk_kv || !kv_data || !kv_scales || !kv_indptr || !kv_indices || !prefix_lens ||
      !slot_mapping || !out)
    return fail(MLAQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(chunk_kv, 16) || !aligned(kv_data, 16) || !aligned(out, 16))
    return fail(MLAQ_ERR_ALIGN, "q, chunk_kv, kv_data and out must be 16-byte aligned");
  if (!aligned(kv_scales, 4) || !aligned(qo_indptr, 4) || !aligned(kv_indptr, 4) || !aligned(kv_indices, 4) ||
      !aligned(prefix_lens, 4) || (lse && !aligned(lse, 4)) || !aligned(slot_mapping, 8))
    return fail(MLAQ_ERR_ALIGN, "kv_scales, index and length arrays need 4-byte alignment, slot_mapping 8-byte");
  if (!workspace) return fail(MLAQ_ERR_NULL, "workspace is NULL but %zu bytes are needed", L.total);
  if (workspace_bytes < L.total)
    return fail(MLAQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
  if (!aligned(workspace, 256)) return fail(MLAQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  mlaq::ExtendArgs a;
  a.qo_indptr = qo_indptr;
  a.prefix_lens = prefix_lens;
  a.kv_indptr = kv_indptr;
  a.kv_indices = kv_indices;
  a.kv_data = kv_data;
  a.kv_scales = kv_scales;
  a.chunk_kv = chunk_kv;
  a.ws_rows = ws + L.rows_off;
  a.view_lens = reinterpret_cast<int32_t*>(ws + L.lens_off);
  a.view_indptr = reinterpret_cast<int32_t*>(ws + L.indptr_off);
  a.pool_tokens = p->pool_tokens;
  a.batch = p->batch;
  a.num_q = p->num_q;
  a.page_size = p->page_size;
  a.page_shift = __builtin_ctz((unsigned)p->page_size);
  a.max_prefix_len = p->max_prefix_len;
  a.max_chunk_len = p->max_chunk_len;
  a.region_rows = L.region_rows;
  a.global_scale = global_scale;
  a.chunk_scale = chunk_scale;
  a.num_heads = p->num_heads;
  a.nan_out = L.tsplits == 1 ? out : nullptr;
  a.nan_lse = L.tsplits == 1 ? lse : nullptr;
  hipError_t e = mlaq::launch_extend_views(a, stream);
  if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "extend view launch failed: %s", hipGetErrorString(e));
  {
    mlaq::ExtendAttnArgs x;
    x.q = q;
    x.ws_rows = a.ws_rows;
    x.qo_indptr = qo_indptr;
    x.prefix_lens = prefix_lens;
    x.kv_indptr = kv_indptr;
    x.out = out;
    x.lse = lse;
    x.part_o = L.part_bytes ? reinterpret_cast<float*>(ws + L.part_off) : nullptr;
    x.part_ml = L.part_bytes ? x.part_o + (size_t)p->num_q * L.tsplits * (p->num_heads / 16) * 16 * 512 : nullptr;
    x.batch = p->batch;
    x.num_q = p->num_q;
    x.num_heads = p->num_heads;
    x.page_size = p->page_size;
    x.max_prefix_len = p->max_prefix_len;
    x.max_chunk_len = p->max_chunk_len;
    x.region_rows = L.region_rows;
    x.num_splits = L.tsplits;
    x.tiles_per_split = L.tiles_per_split;
    x.score_scale = p->sm_scale * chunk_scale * 1.4426950408889634f;
    x.out_scale = chunk_scale;
    const mlaq::ProfileEvents ev = g_events;
    g_events = mlaq::ProfileEvents();
    if (ev.split_start) (void)hipEventRecord(ev.split_start, stream);
    e = mlaq::launch_extend_attn(x, stream);
    if (ev.split_end) (void)hipEventRecord(ev.split_end, stream);
    if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "extend attention launch failed: %s", hipGetErrorString(e));
    if (L.tsplits > 1) {
      mlaq::DecodeArgs m{};
      m.kv_indptr = a.view_indptr;
      m.kv_lens = a.view_lens;
      m.out = out;
      m.lse = lse;
      m.part_o = x.part_o;
      m.part_ml = x.part_ml;
      m.batch = p->num_q;
      m.num_heads = p->num_heads;
      m.page_size = mlaq::kExtendPage;
      m.max_kv_len = L.dp.max_kv_len;
      m.num_splits = L.tsplits;
      m.part_splits = L.tsplits;
      m.out_scale = chunk_scale;
      if (ev.merge_start) (void)hipEventRecord(ev.merge_start, stream);
      e = mlaq::launch_merge(m, stream);
      if (ev.merge_end) (void)hipEventRecord(ev.merge_end, stream);
      if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "extend merge launch failed: %s", hipGetErrorString(e));
    }
  }
  return kv_quantize_nvfp4(chunk_kv, MLAQ_FP8_E4M3, chunk_scale, p->num_q, slot_mapping, kv_data, kv_scales,
                           p->pool_tokens, global_scale, stream);
}

mlaq_status mla_decode_bf16(const mlaq_decode_params* p, const uint16_t* q, const uint16_t* kv,
                            const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_lens, float* out,
                            float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_common(mlaq::FMT_BF16, p, q, kv, nullptr, 1.0f, kv_indptr, kv_indices, kv_lens, out, lse,
                       workspace, workspace_bytes, stream);
}

mlaq_status kv_quantize_nvfp4(const void* src, mlaq_format src_format, float src_scale, int64_t num_tokens,
                              const int64_t* slot_mapping, uint8_t* kv_data, uint8_t* kv_scales, int64_t pool_tokens,
                              float global_scale, hipStream_t stream) {
  if (src_format != MLAQ_FP8_E4M3 && src_format != MLAQ_BF16)
    return fail(MLAQ_ERR_UNSUPPORTED, "kv_quantize_nvfp4: source format %d is not FP8_E4M3 or BF16", (int)src_format);
  if (num_tokens < 0 || num_tokens > ((int64_t)1 << 32))
    return fail(MLAQ_ERR_SHAPE, "num_tokens %lld out of range", (long long)num_tokens);
  if (pool_tokens <= 0 || pool_tokens > ((int64_t)1 << 40))
    return fail(MLAQ_ERR_SHAPE, "pool_tokens %lld out of range", (long long)pool_tokens);
  if (!finite_pos(global_scale)) return fail(MLAQ_ERR_VALUE, "global_scale must be finite and > 0");
  if (src_format == MLAQ_FP8_E4M3 && !finite_pos(src_scale)) return fail(MLAQ_ERR_VALUE, "src_scale must be finite and > 0");
  if (num_tokens == 0) return MLAQ_OK;
  if (!src || !slot_mapping || !kv_data || !kv_scales) return fail(MLAQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(src, 16) || !aligned(kv_data, 16) || !aligned(kv_scales, 4) || !aligned(slot_mapping, 8))
    return fail(MLAQ_ERR_ALIGN, "src and kv_data need 16-byte, kv_scales 4-byte, slot_mapping 8-byte alignment");
  mlaq::QuantArgs a;
  a.src = src;
  a.slots = slot_mapping;
  a.kv_data = kv_data;
  a.kv_scales = kv_scales;
  a.num_tokens = num_tokens;
  a.pool_tokens = pool_tokens;
  a.src_scale = src_scale;
  a.global_scale = global_scale;
  a.src_bf16 = src_format == MLAQ_BF16;
  hipError_t e = mlaq::launch_quantize_nvfp4(a, stream);
  if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "quantize launch failed: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

mlaq_status kv_dequantize(mlaq_format src_format, const uint8_t* kv_data, const uint8_t* kv_scales, float scale,
                          const int64_t* rows, int64_t num_rows, int64_t pool_tokens, mlaq_format dst_format, void* dst,
                          hipStream_t stream) {
  if (src_format != MLAQ_FP8_E4M3 && src_format != MLAQ_NVFP4)
    return fail(MLAQ_ERR_UNSUPPORTED, "kv_dequantize: source format %d is not FP8_E4M3 or NVFP4", (int)src_format);
  if (dst_format != MLAQ_BF16 && dst_format != MLAQ_FP32 && dst_format != MLAQ_FP8_E4M3)
    return fail(MLAQ_ERR_UNSUPPORTED, "kv_dequantize: destination format %d not supported", (int)dst_format);
  if (dst_format == MLAQ_FP8_E4M3 && src_format != MLAQ_NVFP4)
    return fail(MLAQ_ERR_UNSUPPORTED, "kv_dequantize: FP8 destination needs an NVFP4 source");
  if (src_format == MLAQ_FP8_E4M3 && kv_scales)
    return fail(MLAQ_ERR_UNSUPPORTED, "kv_dequantize: kv_scales must be NULL for an FP8 source");
  if (num_rows < 0 || num_rows > ((int64_t)1 << 36)) return fail(MLAQ_ERR_SHAPE, "num_rows out of range");
  if (pool_tokens <= 0 || pool_tokens > ((int64_t)1 << 40)) return fail(MLAQ_ERR_SHAPE, "pool_tokens out of range");
  if (!rows && num_rows > pool_tokens) return fail(MLAQ_ERR_SHAPE, "num_rows > pool_tokens with rows == NULL");
  if (!finite_pos(scale)) return fail(MLAQ_ERR_VALUE, "scale must be finite and > 0");
  if (num_rows == 0) return MLAQ_OK;
  if (!kv_data || !dst || (src_format == MLAQ_NVFP4 && !kv_scales)) return fail(MLAQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(kv_data, 16) || !aligned(dst, 16) || (rows && !aligned(rows, 8)))
    return fail(MLAQ_ERR_ALIGN, "kv_data and dst need 16-byte alignment, rows 8-byte");
  mlaq::DequantArgs a;
  a.kv_data = kv_data;
  a.kv_scales = kv_scales;
  a.rows = rows;
  a.dst = dst;
  a.num_rows = num_rows;
  a.pool_tokens = pool_tokens;
  a.scale = scale;
  a.src_nvfp4 = src_format == MLAQ_NVFP4;
  a.dst_format = (int)dst_format;
  hipError_t e = mlaq::launch_dequantize(a, stream);
  if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "dequantize launch failed: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

mlaq_status mlaq_read_probe(const void* buf, int64_t bytes, void* partials, int32_t num_blocks, hipStream_t stream) {
  if (bytes < 0 || bytes % 16) return fail(MLAQ_ERR_SHAPE, "read probe: bytes %lld must be a multiple of 16", (long long)bytes);
  if (num_blocks < 1 || num_blocks > (1 << 20))
    return fail(MLAQ_ERR_SHAPE, "read probe: num_blocks %d not in [1, 2^20]", num_blocks);
  if (!partials || (bytes > 0 && !buf)) return fail(MLAQ_ERR_NULL, "read probe: a required pointer is NULL");
  if (!aligned(buf, 16) || !aligned(partials, 16)) return fail(MLAQ_ERR_ALIGN, "read probe: buf and partials need 16-byte alignment");
  hipError_t e = mlaq::launch_read_probe(buf, bytes / 16, partials, num_blocks, stream);
  if (e != hipSuccess) return fail(MLAQ_ERR_LAUNCH, "read probe launch failed: %s", hipGetErrorString(e));
  return MLAQ_OK;
}

}  // extern "C"
