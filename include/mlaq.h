/* mlaq.h -- paged MLA decode over an FP8 / NVFP4 latent KV pool on MI355X (gfx950).
 *
 * A small C ABI.  Pointers are DEVICE pointers unless marked (host).  The caller owns
 * all memory: queries, pools, page table, lengths, outputs and the workspace.  Calls
 * are asynchronous on `stream`; they never allocate, never synchronise the device and
 * never read device memory on the host, so a call can be captured in a HIP graph and
 * replayed (its launches use no memset or copy nodes).  Every argument that can be checked on the
 * host is checked before any launch; a non-OK status means nothing was launched and
 * mlaq_last_error() (thread-local) says why.
 *
 * What the calls compute, and where the pages say so:
 *   - single-token decode attention of `num_heads` absorbed MLA queries over the latent
 *     KV rows of each request, reached through a CSR page table (kv_indptr / kv_indices
 *     / kv_lens), no causal mask, softmax scale sm_scale: the FlashInfer MLA decode
 *     plan of "The Smoking Gun: Tracing the FP8-to-BF16 KV Cache Cast" (section
 *     "Message Overview": plan(qo_indptr, kv_indptr, kv_indices, kv_len_arr,
 *     num_local_heads, kv_lora_rank, qk_rope_head_dim, 1, False, sm_scale, q dtype,
 *     kv dtype));
 *   - the latent row is 576 = kv_lora_rank 512 + qk_rope_head_dim 64 with one shared KV
 *     head, pool [tokens, 1, 576] (same page, section "The Investigation Leading to This
 *     Message"); the value is the first 512 dims of the same row;
 *   - the KV may stay in FP8 e4m3fn or NVFP4 and is dequantized inside the kernel
 *     instead of casting the pool to BF16 (the cast is the bottleneck found on that
 *     page; NVFP4 decode reads the packed format directly: NVFP4 article on aitop.news,
 *     implementation item 3);
 *   - NVFP4 = E2M1 values, one E4M3 scale per 16 values, one FP32 global scale (same
 *     article, format section); the cache is filled by quantize-on-write (item 1).
 *
 * Layouts (row-major, contiguous):
 *   q            bf16 bits  [batch, num_heads, 576]; dims 0-511 latent, 512-575 rope
 *   FP8 pool     e4m3fn     [pool_tokens, 576]
 *   BF16 pool    bf16 bits  [pool_tokens, 576]
 *   NVFP4 pool   data       [pool_tokens, 288]  byte j = code(dim 2j) | code(dim 2j+1) << 4
 *                scales     [pool_tokens, 36]   e4m3fn; scale k covers dims 16k .. 16k+15
 *   kv_indptr    int32 [batch + 1]  page offsets of each request into kv_indices
 *   kv_indices   int32 [kv_indptr[batch]]  physical page ids; token j of request b lives in
 *                pool row kv_indices[kv_indptr[b] + j / page_size] * page_size + j % page_size
 *   kv_lens      int32 [batch]  tokens per request
 *   out          fp32 [batch, num_heads, 512]
 *   lse          fp32 [batch, num_heads] natural-log sum of exp of the scaled scores; may be NULL
 *
 * Device-resident contents are checked in the kernels without faulting: a request whose
 * length is negative, above max_kv_len or beyond its pages, or that names a page outside
 * the pool, gets NaN in out and lse.  A request with kv_len 0 gets out = 0, lse = -inf.
 */
#ifndef MLAQ_H
#define MLAQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLAQ_HEAD_DIM 576
#define MLAQ_LATENT_DIM 512
#define MLAQ_ROPE_DIM 64
#define MLAQ_NVFP4_DATA_BYTES 288
#define MLAQ_NVFP4_SCALE_BYTES 36
#define MLAQ_MAX_SPLITS 1024
#define MLAQ_MAX_KV_LEN (1 << 24)
/* Longest KV chunk one split may cover.  Probabilities enter the PV products as fp16 relative to
 * the chunk's running maximum, so a token far below that maximum rounds on the fp16 subnormal grid
 * (absolute error at most 2^-25 of the largest weight); capping the chunk bounds the sum of those
 * errors by 2^14 * 2^-25 = 2^-11 of the largest weight, the size of ordinary fp16 rounding.  A
 * forced num_splits must therefore satisfy max_kv_len <= num_splits * MLAQ_MAX_SPLIT_TOKENS, and
 * the automatic plan always does. */
#define MLAQ_MAX_SPLIT_TOKENS (1 << 14)

typedef enum {
  MLAQ_OK = 0,
  MLAQ_ERR_NULL = 1,        /* a required pointer is NULL */
  MLAQ_ERR_SHAPE = 2,       /* a size is out of the supported range */
  MLAQ_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  MLAQ_ERR_UNSUPPORTED = 4, /* format combination not implemented */
  MLAQ_ERR_WORKSPACE = 5,   /* workspace smaller than the size the call needs */
  MLAQ_ERR_LAUNCH = 6,      /* the HIP launch itself failed */
  MLAQ_ERR_VALUE = 7        /* a scalar argument is not finite / not positive (a scale of 0 or NaN
                               would make every output NaN without an error) */
} mlaq_status;

typedef enum { MLAQ_BF16 = 0, MLAQ_FP8_E4M3 = 1, MLAQ_NVFP4 = 2, MLAQ_FP32 = 3 } mlaq_format;

/* The host-side inputs of the decode plan ("The Smoking Gun: Tracing the FP8-to-BF16 KV Cache
 * Cast", section "Message Overview": plan() receives the head count, kv_lora_rank 512 + rope 64,
 * page size, sm_scale and host copies of the lengths). */
typedef struct {            /* (host) */
  int32_t batch;            /* >= 0; 0 is a no-op */
  int32_t num_heads;        /* multiple of 16, 16 .. 128 */
  int32_t page_size;        /* tokens per page: a power of two, 1 .. 1024 */
  int64_t pool_tokens;      /* rows in the pool (> 0) */
  int32_t max_kv_len;       /* host upper bound of kv_lens[] (split planning), 0 .. MLAQ_MAX_KV_LEN */
  int32_t num_splits;       /* KV chunks per request; 0 = choose automatically; a forced count
                               must satisfy max_kv_len <= num_splits * MLAQ_MAX_SPLIT_TOKENS */
  float sm_scale;           /* multiplies q . k before the softmax; finite */
} mlaq_decode_params;

/* (host) Workspace bytes that serve a decode of any KV format (FP8, NVFP4, BF16) with these
 * parameters: the largest of mlaq_decode_format_workspace_bytes over the three formats.  0 when
 * no format needs one (one split each), SIZE_MAX if the parameters are invalid.  The workspace
 * holds one fp32 partial output plus running max and sum per (request, split, 16-head group)
 * (the split-KV partials of the decode plan, same passage as mlaq_decode_params); it must be
 * 256-byte aligned. */
size_t mlaq_decode_workspace_bytes(const mlaq_decode_params* p);

/* (host) The exact workspace bytes a decode of one KV format (MLAQ_FP8_E4M3, MLAQ_NVFP4 or
 * MLAQ_BF16) needs; the formats run different workgroup shapes and so plan different split
 * counts.  SIZE_MAX if the parameters or the format are invalid. */
size_t mlaq_decode_format_workspace_bytes(const mlaq_decode_params* p, mlaq_format kv_format);

/* (host) Splits a decode of the given KV format will use for these parameters (resolves
 * num_splits = 0), or 0 if the parameters or the format are invalid.  Host arguments only. */
int32_t mlaq_decode_num_splits(const mlaq_decode_params* p, mlaq_format kv_format);

/* Decode over an FP8 e4m3fn pool, dequantized inside the kernel: the pool the pages' server
 * kept in float8_e4m3fn and cast whole to BF16 before every decode ("The Smoking Gun: Tracing the
 * FP8-to-BF16 KV Cache Cast", section "The Investigation Leading to This Message"; "The FP8 KV
 * Cache Wall", section "Context and Motivation"), here read as stored.  kv_scale (> 0, finite) is
 * the per-tensor dequant multiplier: k = e4m3(code) * kv_scale.  Workspace: at least
 * mlaq_decode_format_workspace_bytes(p, MLAQ_FP8_E4M3) (mlaq_decode_workspace_bytes(p) always
 * suffices).  Alignment: q, kv, out 16 B; lse 4 B. */
mlaq_status mla_decode_fp8(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv, float kv_scale,
                           const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_lens,
                           float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode over an NVFP4 pool read as stored (NVFP4 article on aitop.news, implementation item 3:
 * packed tiles and E4M3 block scales converted in the kernel, the global scale applied as a scalar
 * factor; format section: k = e2m1(code) * e4m3(block scale) * global_scale).  Workspace: at least
 * mlaq_decode_format_workspace_bytes(p, MLAQ_NVFP4).  Alignment: q, kv_data, out 16 B; kv_scales
 * 4 B; lse 4 B. */
mlaq_status mla_decode_nvfp4(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv_data,
                             const uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                             const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free NVFP4 decode, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same computation, kernels
 * and arguments as mla_decode_nvfp4, without the workspace: the split partials go to a scratch
 * array of MLAQ_NOALLOC_SCRATCH_BYTES (48 MiB) that the library holds on each device it runs on
 * until the process ends.  The call allocates and frees nothing; its first call on a device looks
 * the array's address up once.  The split plan is mla_decode_nvfp4's whenever its partials fit the
 * scratch (the outputs are then bit for bit those of mla_decode_nvfp4; the pages' workloads, up to
 * 128 requests at 32K context, 56 at 160K and 16 at 1M, all fit), else the largest split count whose
 * partials fit (the outputs then equal mla_decode_nvfp4's with that num_splits).  A forced
 * num_splits whose partials do not fit, or a batch whose partials do not fit even at the fewest
 * splits the per-split token cap allows, returns MLAQ_ERR_WORKSPACE before any launch.  Every call
 * on one device shares that device's scratch, which keeps the last call's contents (nothing in it
 * has to start at zero): calls that overlap on one device, on different streams or from different
 * threads, race and give wrong outputs; serialize them. */
#define MLAQ_NOALLOC_SCRATCH_BYTES (48u << 20)
mlaq_status mla_decode_nvfp4_noalloc(const mlaq_decode_params* p, const uint16_t* q, const uint8_t* kv_data,
                                     const uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                                     const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                                     hipStream_t stream);

/* Fused append-then-attend over an NVFP4 pool (one decode call per layer and step): token
 * kv_lens[b] - 1 of every request is the new token.  Its pool row (found through the page
 * table like any other token) is overwritten with the NVFP4 encoding of new_kv[b], exactly as
 * kv_quantize_nvfp4 would write it (NVFP4 article on aitop.news, implementation item 1:
 * quantize-on-write), and the decode then attends all kv_lens[b] tokens, the new one included
 * (implementation item 3: decode reads the packed format).  The split kernel writes the row
 * and attends tokens 0 .. kv_lens[b] - 2; the merge pass adds the new token from the row it
 * wrote, so one call replaces a quantize launch plus a decode.
 * new_kv: [batch, 576] e4m3fn bytes (x = e4m3 * src_scale) or bf16 bits (new_kv_format
 * MLAQ_FP8_E4M3 or MLAQ_BF16), 16-B aligned; the other arguments are those of
 * mla_decode_nvfp4, with kv_data / kv_scales written.  kv_lens[b] must be >= 1 (0 gives NaN);
 * a request whose new row lies outside the pool gets NaN and writes nothing.  The new rows
 * must not be read by another request of the same call.  The workspace size is
 * mlaq_decode_nvfp4_append_workspace_bytes(p): the merge pass always runs. */
size_t mlaq_decode_nvfp4_append_workspace_bytes(const mlaq_decode_params* p);    /* (host) SIZE_MAX if p is invalid */
mlaq_status mla_decode_nvfp4_append(const mlaq_decode_params* p, const uint16_t* q, const void* new_kv,
                                    mlaq_format new_kv_format, float src_scale, uint8_t* kv_data,
                                    uint8_t* kv_scales, float global_scale, const int32_t* kv_indptr,
                                    const int32_t* kv_indices, const int32_t* kv_lens, float* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Extend (chunked prefill) over an NVFP4 cache (NVFP4 article on aitop.news, implementation
 * item 2): for each request b, the chunk's query tokens q[qo_indptr[b] .. qo_indptr[b+1]) attend
 * the request's cached prefix (prefix_lens[b] tokens through the cache page table) followed by
 * the chunk's own rows, causally: chunk token i sees the prefix, chunk tokens 0 .. i-1 and
 * itself.  As on the page, the prefix is first dequantized into an FP8 workspace
 * (e4m3 of fl32(e2m1 * e4m3 * global_scale) / chunk_scale: lossy, up to 6 significant bits
 * round to 4), the chunk's FP8 rows are appended, attention runs over that workspace, and
 * the chunk is then quantized into the cache at slot_mapping[t] (kv_quantize_nvfp4 with
 * src_scale = chunk_scale; rows < 0 skipped).  The attention reads each workspace row once
 * per eight chunk tokens and 16-head group, on MFMA; KV splits of long prefixes are merged
 * like the decode splits.
 *   q          bf16 [num_q, num_heads, 576]      chunk_kv  e4m3fn [num_q, 576], x = e4m3 * chunk_scale
 *   qo_indptr  int32 [batch + 1]                  prefix_lens int32 [batch]
 *   out        fp32 [num_q, num_heads, 512]       lse fp32 [num_q, num_heads] or NULL
 * Device-resident lengths and pages are checked: a request whose prefix or chunk length is
 * outside [0, max_*_len], whose pages do not cover its prefix or whose query range leaves
 * [0, num_q) gets NaN; a prefix page outside the pool gives NaN for the tokens that see it.
 * The workspace (mlaq_extend_workspace_bytes(p), 256-B aligned) holds batch regions of
 * round_up(max_prefix_len + max_chunk_len, 64) FP8 rows, per-token lengths and the split
 * partials; it is reused across layers. */
typedef struct {              /* (host) */
  int32_t batch;              /* requests, 0 .. 65535 */
  int32_t num_heads;          /* multiple of 16, 16 .. 128 */
  int32_t page_size;          /* cache page size: a power of two, 1 .. 1024 */
  int64_t pool_tokens;        /* cache rows */
  int32_t num_q;              /* chunk tokens over all requests (rows of q, chunk_kv, out), 0 .. 65535 */
  int32_t max_prefix_len;     /* host bounds of prefix_lens[] and of the chunk lengths */
  int32_t max_chunk_len;
  int32_t num_splits;         /* KV chunks per query token in the attention; 0 = automatic */
  float sm_scale;
} mlaq_extend_params;
size_t mlaq_extend_workspace_bytes(const mlaq_extend_params* p);   /* (host) SIZE_MAX if p is invalid */
int32_t mlaq_extend_num_splits(const mlaq_extend_params* p);       /* (host) 0 if p is invalid */
mlaq_status mla_extend_nvfp4(const mlaq_extend_params* p, const uint16_t* q, const int32_t* qo_indptr,
                             const uint8_t* chunk_kv, float chunk_scale, uint8_t* kv_data, uint8_t* kv_scales,
                             float global_scale, const int32_t* kv_indptr, const int32_t* kv_indices,
                             const int32_t* prefix_lens, const int64_t* slot_mapping, float* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode over a BF16 pool: the second half of the path the pages' server ran, which cast the
 * FP8 pool to BF16 and then decoded in BF16 ("The Smoking Gun: Tracing the FP8-to-BF16 KV Cache
 * Cast", section "The Investigation Leading to This Message"), kept as the comparison baseline and
 * as a cross-check of the quantized paths.  Workspace: at least
 * mlaq_decode_format_workspace_bytes(p, MLAQ_BF16).  Alignment: q, kv, out 16 B; lse 4 B. */
mlaq_status mla_decode_bf16(const mlaq_decode_params* p, const uint16_t* q, const uint16_t* kv,
                            const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_lens,
                            float* out, float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* NVFP4 quantize-on-write (NVFP4 article, implementation item 1): each source row of 576
 * values becomes 36 blocks of 16, written to pool row slot_mapping[t] (rows with a
 * negative slot are skipped; a slot >= pool_tokens is skipped too and not written).
 * Per block, in IEEE fp32 with round-to-nearest-even: scale byte = e4m3(sat) of
 * (amax / 6) / global_scale; codes = e2m1(sat) of x / (e4m3(scale) * global_scale);
 * a NaN in the block gives scale 0x7F and zero codes; a zero divisor gives zero codes.
 * src: MLAQ_FP8_E4M3 bytes (x = e4m3 * src_scale) or MLAQ_BF16 bits, [num_tokens, 576],
 * 16-B aligned.  kv_data 16-B aligned, kv_scales 4-B aligned. */
mlaq_status kv_quantize_nvfp4(const void* src, mlaq_format src_format, float src_scale, int64_t num_tokens,
                              const int64_t* slot_mapping, uint8_t* kv_data, uint8_t* kv_scales,
                              int64_t pool_tokens, float global_scale, hipStream_t stream);

/* Dequantize pool rows into a dense buffer dst [num_rows, 576]: the whole-pool FP8 -> BF16 cast of
 * the pages' server ("The Smoking Gun: Tracing the FP8-to-BF16 KV Cache Cast", section "The
 * Investigation Leading to This Message"), the cast of only the active rows that was its first fix
 * ("The FP8 KV Cache Wall", sections "The Message" and "Aftermath"), and the NVFP4 -> FP8 prefix
 * workspace of extend (NVFP4 article on aitop.news, implementation item 2).
 * src_format MLAQ_FP8_E4M3: value = e4m3(code) * scale (kv_scales must be NULL);
 * src_format MLAQ_NVFP4:    value = e2m1 * e4m3(block scale) * scale.
 * The fp32 value is fl32(fl32(e2m1 * e4m3) * scale) (fl32(e4m3 * scale) for FP8);
 * dst_format MLAQ_FP32 stores it, MLAQ_BF16 rounds it to nearest even, MLAQ_FP8_E4M3
 * re-encodes it (nearest even, saturating at 448; NVFP4 source only).
 * rows: int64 [num_rows] pool rows to read (each in [0, pool_tokens), else the output row is
 * NaN), or NULL for rows 0 .. num_rows-1.  pool_tokens (the rows of kv_data) is what lets a
 * device-resident row list be range-checked without a fault.  kv_data and dst 16-B aligned. */
mlaq_status kv_dequantize(mlaq_format src_format, const uint8_t* kv_data, const uint8_t* kv_scales, float scale,
                          const int64_t* rows, int64_t num_rows, int64_t pool_tokens, mlaq_format dst_format,
                          void* dst, hipStream_t stream);

/* ---- Measurement aids (not steps of the path) ---- */

/* (host) Profiling hook for callers that time the kernels themselves, and the one piece of
 * thread-local state besides the error message.  Registers up to four
 * HIP events (hipEvent_t, or NULL) for the NEXT decode call made on this thread: the split-KV
 * kernel is launched with `split_start` / `split_end` recorded at its own start and end
 * (hipExtLaunchKernelGGL), and the merge kernel, if the call runs one, with `merge_start` /
 * `merge_end`; then the registration is cleared.  A call without a merge kernel leaves the
 * merge events untouched.  The events are owned by the caller. */
mlaq_status mlaq_set_profile_events(hipEvent_t split_start, hipEvent_t split_end, hipEvent_t merge_start,
                                    hipEvent_t merge_end);

/* Measurement aid, not part of the attention path: a streaming read of `bytes` bytes of buf
 * (a multiple of 16; buf and partials 16-byte aligned) with nontemporal 16-byte loads by
 * `num_blocks` workgroups of 256 threads, grid-stride.  Block k writes the XOR of the 16-byte
 * words it read to partials[16k .. 16k+15], so the XOR of all partials is the XOR of all
 * words of the buffer.  Timed over a buffer far larger than the 256 MB Infinity Cache, it gives
 * the HBM read bandwidth this device actually reaches, the measured ceiling reported beside
 * the nominal 8 TB/s.  Errors: bad size or block count (MLAQ_ERR_SHAPE), NULL pointers,
 * misalignment, launch failure. */
mlaq_status mlaq_read_probe(const void* buf, int64_t bytes, void* partials, int32_t num_blocks, hipStream_t stream);

/* (host) Message for the last non-OK status returned on this thread ("" if none). */
const char* mlaq_last_error(void);

/* (host) Library version string. */
const char* mlaq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLAQ_H */
