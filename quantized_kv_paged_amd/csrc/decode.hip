// Split-KV paged MLA decode with in-kernel dequantization (FP8 e4m3fn, NVFP4, BF16 pools),
// and the merge pass over splits.
//
// What is computed (per request b, query head h): softmax over all kv_len tokens of
// sm_scale * q[b,h,:] . k_j (576 dims) and the weighted sum of v_j = k_j[0:512]; the pool is
// read through the page table; no causal mask.  This is the FlashInfer MLA decode plan
// shown on "The Smoking Gun: Tracing the FP8-to-BF16 KV Cache Cast" (section "Message
// Overview"), run directly on the stored FP8 / NVFP4 rows, as the NVFP4 article
// (aitop.news, implementation item 3) describes for decode: packed tiles and E4M3 block
// scales read as stored, converted in registers, global scale applied as a scalar factor.
//
// gfx950 design: one workgroup = one request x one KV chunk x 16 heads, running NS
// online-softmax streams (token groups) with two waves each.  FP8 and BF16: NS = 2, 4 waves,
// 80 KB of LDS, two workgroups per CU; NVFP4: NS = 1, 2 waves, 40 KB, four per CU.  Either
// way every SIMD runs two waves (at most 256 VGPRs each) of independent workgroups.
//   * every head shares the single latent KV row, so each KV byte is read from HBM once and
//     both products are dense 16-head contractions on MFMA;
//   * tile = 32 NS tokens.  Wave w = (token group tg = w % NS, dim half dh = w / NS) owns
//     tokens 32tg .. 32tg+31 of each tile as two 16-token MFMA blocks.  S^T = K Q^T
//     (v_mfma_f32_16x16x32) is split over the pair (tg, 0) / (tg, 1): half dh is value dims
//     256dh .. 256dh+255 plus rope dims 512+32dh .. +31; each wave holds that half of the query
//     operand and converts that half of its 32 rows, and the pair swaps 2 KB of partial scores
//     through LDS (double-buffered, one barrier per tile);
//   * each token group is its own online-softmax stream over the chunk; its 32 probabilities
//     per head are already in the A-operand layout of a 32-token v_mfma_f32_16x16x32 (lane =
//     head, 8 tokens), so O += P V needs no score traffic: wave (tg, dh) accumulates the 256
//     value dims of half dh over its 32 tokens, the V operand coming from LDS with two gfx950
//     transposed reads (ds_read_b64_tr_b16) per 16 dims.  At the end of the chunk the streams
//     are merged through the waves' own value tiles (one barrier);
//   * K rows go global -> VGPR: with pages of at least a tile, a tile is contiguous pool rows,
//     read with buffer loads through a per-tile descriptor whose size admits only the
//     tile's valid rows (other lanes read zeros); the registers of a tile are refilled with
//     the next tile's loads as soon as they are converted, so the loads are in flight during
//     the softmax and PV of the tile.  Rows are converted to fp16 in registers (FP8: exact;
//     NVFP4: E2M1 -> fp16 times the fp16 E4M3 block scale, exact since every E2M1 x E4M3
//     product is an fp16 value); the converted operand feeds the QK MFMA directly and its value
//     dims are written once to an XOR-swizzled LDS tile;
//   * a wave reads back only the value dims it wrote itself, so each wave has a private
//     single-buffered LDS value tile (LDS operations of one wave complete in order);
//   * the per-tensor FP8 scale or NVFP4 global scale and a power-of-two query prescale
//     (bf16 queries are converted to fp16 exactly) fold into the score and output scales.
#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>

#include "device_common.h"
#include "mlaq.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kBlocks = 2;                 // 16-token MFMA blocks per wave per tile
constexpr int kVRow = 512;                 // bytes per LDS value row of a wave (its 256 fp16 dims)
constexpr int kWaveV = 16 * kBlocks * kVRow;       // a wave's value tile (16 KB)
constexpr int kSwapW = kBlocks * 64 * 16;          // bytes of a wave's partial scores (2 KB)

// Workgroup geometry for NS online-softmax streams (token groups): 2 NS waves (one per
// (stream, dim half)), tiles of 32 NS tokens, LDS = value tiles + double-buffered score swap.
template <int NS> struct Geo {
  static constexpr int kStreams = NS;
  static constexpr int kTile = 16 * kBlocks * NS;
  static constexpr int kWaves = 2 * NS;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kSwap = kWaves * kWaveV;                 // byte offset of the swap buffers
  static constexpr int kSmem = kSwap + 2 * kWaves * kSwapW;     // 40 KB (NS = 1) or 80 KB (NS = 2)
  static_assert(kTile == decode_tile(NS), "tile size shared with the host planner");
  static_assert(decode_groups_per_cu(NS) * kSmem <= 160 * 1024, "resident workgroups per CU");
};
constexpr float kMinusBig = -3.0e38f;   // initial running max: finite, so an empty stream stays finite
constexpr float kSlack = 8.0f;          // lazy-rescale threshold of the running max (log2 units)

// The lane's share of one token row for its dim half dh and lane group g, as 9 k-blocks of 8
// dims (any order of the 576 dims gives the same dot product; the query operand uses the same
// map).  The map is chosen per format so that a lane's k-blocks are 16 contiguous bytes of
// the row:
//   FP8, BF16: kb < 8 (m = kb/2, h = kb%2): value dims 256dh + 64m + 16g + 8h .. +8 (the
//              four lane groups of a token read 64 contiguous bytes per load)
//   NVFP4:     kb < 8 (c = kb/4, s = kb%4): value dims 256dh + 64g + 32c + 8s .. +8 (a lane
//              reads 32 contiguous bytes = 64 dims = four whole 16-value scale blocks, so its
//              block scales are one aligned 4-byte word of the scale row)
//   kb = 8: rope dims 512 + 32dh + 8g .. +8.
template <int FMT> struct RawTile;
template <> struct RawTile<FMT_FP8> { u32x4 d[4]; u32x2 e; };                  // 4 x 16 B + 8 B
// codes (2 x 16 B + 4 B rope), the scales of blocks 16dh + 4g .. +3 (s) and rope blocks 32..35 (sr)
template <> struct RawTile<FMT_NVFP4> { u32x4 d[2]; uint32_t e; uint32_t s; uint32_t sr; };
template <> struct RawTile<FMT_BF16> { u32x4 d[9]; };                           // 9 x 16 B

template <int FMT> struct OpType { typedef f16x8 type; typedef _Float16 elem; };
template <> struct OpType<FMT_BF16> { typedef bf16x8 type; typedef __bf16 elem; };

// A wave's LDS value tile: row r (its token 16tg + r) of 512 B holds its 256 value dims; the
// 16-byte chunk c is stored at chunk c ^ vswz(r), vswz(r) = x ^ 2x (mod 16) for x = r mod 16.
// The 16-byte row writes of the QK phase (16 rows x 4 chunks per instruction) and the
// transposed 8-byte reads of the PV phase (16 rows x 2 chunks) then spread over all banks for
// any grouping of the wave's lanes into 256-byte (64 banks) or 128-byte (32 banks) cycles
// (checked by enumeration).  Since the XOR only touches chunk bits 0-3, every address is one
// per-lane base XOR a per-instruction constant in bits 4-7, plus a constant offset.
__device__ __forceinline__ int vswz(int r) { const int x = r & 15; return (x ^ (x << 1)) & 15; }

template <int FMT>
__device__ __forceinline__ int kb_dim(int dh, int kb, int g) {
  if (kb == 8) return 512 + 32 * dh + 8 * g;
  return FMT == FMT_NVFP4 ? 256 * dh + 64 * g + 32 * (kb >> 2) + 8 * (kb & 3)
                          : 256 * dh + 64 * (kb >> 1) + 16 * g + 8 * (kb & 1);
}

// The chunk's page-table entries, 64 at a time: lane l of `cur` holds entry
// first + 64 * batch + l of the request's page list (clamped to its last entry, so every load
// is in bounds; validity is decided separately by tile_row), and `next` the following batch,
// loaded one batch ahead.  A tile's entries never straddle two batches (tiles are 64-token
// aligned and pages are powers of two), so the batch switch is uniform, and the id of a
// tile's page is a lane read of a register that arrived long before: no page-table load
// sits between a tile's row loads and their use.
struct PageWindow {
  const int* list;   // kv_indices + p0
  int first, last, batch, cur, next;
  __device__ __forceinline__ void init(const DecodeArgs& a, int p0, int npages, int t_begin, int lane) {
    list = a.kv_indices + p0;
    first = t_begin >> a.page_shift;
    last = npages - 1;
    batch = 0;
    cur = list[min(first + lane, last)];
    next = list[min(first + 64 + lane, last)];
  }
  // page id of the lane's token tok; TILEPAGE: the tile's page (tok = its first token)
  template <bool TILEPAGE>
  __device__ __forceinline__ int page(const DecodeArgs& a, int tok, int lane) {
    const int e = (tok >> a.page_shift) - first;
    if ((e >> 6) != batch) {   // uniform
      ++batch;
      cur = next;
      next = list[min(first + 64 * (batch + 1) + lane, last)];
    }
    if constexpr (TILEPAGE) return __builtin_amdgcn_readlane(cur, e & 63);
    else return __builtin_amdgcn_ds_bpermute(4 * (e & 63), cur);
  }
};

// Pool row of the lane's token and its state: 0 = valid, 1 = beyond the chunk (contributes
// zeros, masked out of the softmax), 2 = bad page (contributes NaN).  Invalid lanes read row 0.
__device__ __forceinline__ int64_t tile_row(const DecodeArgs& a, int npages, int tok, int end, int page,
                                            int& state) {
  const int pi = tok >> a.page_shift;
  const int64_t row = ((int64_t)page << a.page_shift) + (tok & (a.page_size - 1));
  state = tok >= end ? 1 : (pi >= npages || page < 0 || row >= a.pool_tokens) ? 2 : 0;
  return state == 0 ? row : 0;
}

template <int FMT>
__device__ __forceinline__ void load_raw(RawTile<FMT>& r, const DecodeArgs& a, int64_t row, int dh, int g) {
  if constexpr (FMT == FMT_FP8) {
    const uint8_t* base = a.kv + row * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) r.d[m] = *reinterpret_cast<const u32x4*>(base + 256 * dh + 64 * m + 16 * g);
    r.e = *reinterpret_cast<const u32x2*>(base + 512 + 32 * dh + 8 * g);
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint8_t* base = a.kv + row * kNvData;
#pragma unroll
    for (int c = 0; c < 2; ++c) r.d[c] = *reinterpret_cast<const u32x4*>(base + 128 * dh + 32 * g + 16 * c);
    r.e = *reinterpret_cast<const uint32_t*>(base + 256 + 16 * dh + 4 * g);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.kv_scales + row * kNvScale);
    r.s = sp[4 * dh + g];   // blocks 16dh + 4g .. +3
    r.sr = sp[8];           // rope blocks 32 .. 35
  } else {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.kv) + row * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      r.d[2 * m] = *reinterpret_cast<const u32x4*>(base + 256 * dh + 64 * m + 16 * g);
      r.d[2 * m + 1] = *reinterpret_cast<const u32x4*>(base + 256 * dh + 64 * m + 16 * g + 8);
    }
    r.d[8] = *reinterpret_cast<const u32x4*>(base + 512 + 32 * dh + 8 * g);
  }
}

// Same loads for a tile whose rows are contiguous in the pool: buffer loads through
// descriptors whose base is the tile's first row (kv, and the NVFP4 scales in sc) and whose
// size covers only the tile's valid rows, so the lanes of other rows read zeros; the lane's
// constant byte offsets are o.v (value part), o.e (rope part), o.s (NVFP4 scale row).
struct LaneOffsets { uint32_t v, e, s; };
template <int FMT>
__device__ __forceinline__ LaneOffsets lane_offsets(int tok_in_tile, int dh, int g) {
  LaneOffsets o;
  if constexpr (FMT == FMT_FP8) {
    o.v = tok_in_tile * kD + 256 * dh + 16 * g;
    o.e = tok_in_tile * kD + 512 + 32 * dh + 8 * g;
    o.s = 0;
  } else if constexpr (FMT == FMT_NVFP4) {
    o.v = tok_in_tile * kNvData + 128 * dh + 32 * g;
    o.e = tok_in_tile * kNvData + 256 + 16 * dh + 4 * g;
    o.s = tok_in_tile * kNvScale;
  } else {
    o.v = 2 * (tok_in_tile * kD + 256 * dh + 16 * g);
    o.e = 2 * (tok_in_tile * kD + 512 + 32 * dh + 8 * g);
    o.s = 0;
  }
  return o;
}

template <int FMT>
__device__ __forceinline__ void load_raw_tile(RawTile<FMT>& r, BufferRsrc kv, BufferRsrc sc, const LaneOffsets& o,
                                              int dh, int g, int tok0) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t so = tok0 * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) r.d[m] = buffer_load_b128(kv, o.v + 64 * m, so);
    r.e = buffer_load_b64(kv, o.e, so);
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint32_t so = tok0 * kNvData, ss = tok0 * kNvScale;
#pragma unroll
    for (int c = 0; c < 2; ++c) r.d[c] = buffer_load_b128(kv, o.v + 16 * c, so);
    r.e = buffer_load_b32(kv, o.e, so);
    r.s = buffer_load_b32(sc, o.s + 16 * dh + 4 * g, ss);    // blocks 16dh + 4g .. +3
    r.sr = buffer_load_b32(sc, o.s + 32, ss);                // rope blocks 32 .. 35
  } else {
    const uint32_t so = tok0 * 2 * kD;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      r.d[2 * m] = buffer_load_b128(kv, o.v + 128 * m, so);
      r.d[2 * m + 1] = buffer_load_b128(kv, o.v + 128 * m + 16, so);
    }
    r.d[8] = buffer_load_b128(kv, o.e, so);
  }
}

// Replace the data of masked lanes by zeros and of bad-page lanes by NaN codes.
template <int FMT>
__device__ __forceinline__ void fix_raw(RawTile<FMT>& r, int state) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t f = state == 2 ? 0x7f7f7f7fu : 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[m][e] = state ? f : r.d[m][e];
    r.e[0] = state ? f : r.e[0];
    r.e[1] = state ? f : r.e[1];
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint32_t f = state == 2 ? 0x7f7f7f7fu : 0u;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[c][e] = state ? 0u : r.d[c][e];
    r.e = state ? 0u : r.e;
    r.s = state ? f : r.s;
    r.sr = state ? f : r.sr;
  } else {
    const uint32_t f = state == 2 ? 0x7fc07fc0u : 0u;
#pragma unroll
    for (int k = 0; k < 9; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[k][e] = state ? f : r.d[k][e];
  }
}

// MFMA operand of k-block KB of the lane's row half.  NVFP4: the 16-dim block of k-block
// 4c + s is byte 2c + s/2 of s; bytes 2c and 2c + 1 convert together to an fp16 pair, and the
// products take the block's half of it in both lanes of the pair (an operand select of the packed
// multiply, no extra instruction); the block of k-block 8 is byte 2dh + g/2 of sr (selector ssel).
template <int FMT, int KB>
__device__ __forceinline__ typename OpType<FMT>::type dequant(const RawTile<FMT>& r, uint32_t ssel) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t w0 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1)] : r.e[0];
    const uint32_t w1 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1) + 1] : r.e[1];
    const f16x2 a = fp8x2_to_f16<false>(w0), b = fp8x2_to_f16<true>(w0);
    const f16x2 c = fp8x2_to_f16<false>(w1), d = fp8x2_to_f16<true>(w1);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else if constexpr (FMT == FMT_NVFP4) {
    f16x2 s2;
    if constexpr (KB < 8) {
      const f16x2 sp = fp8x2_to_f16<((KB >> 2) != 0)>(r.s);
      s2 = __builtin_shufflevector(sp, sp, (KB & 3) >> 1, (KB & 3) >> 1);
    } else {
      s2 = fp8x2_to_f16<false>(__builtin_amdgcn_perm(0u, r.sr, ssel));
    }
    const uint32_t w = KB < 8 ? r.d[KB >> 2][KB & 3] : r.e;
    const f16x2 a = fp4x2_to_f16<0>(w) * s2, b = fp4x2_to_f16<1>(w) * s2;
    const f16x2 c = fp4x2_to_f16<2>(w) * s2, d = fp4x2_to_f16<3>(w) * s2;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    return __builtin_bit_cast(bf16x8, r.d[KB]);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// The new token of a fused append (NVFP4 pools): thread k < 36 quantizes block k of the
// request's source row exactly as the quantize-on-write kernel does, the first head group
// writes the codes and scales to the token's pool row, and every head group stores the row as
// the request's extra partial (slot num_splits): m = the head's log2-domain score, l = 1,
// O = the row's value dims.  Values are dequantized without the global scale, like the pool
// rows the tiles convert (it is folded into the score and output scales).  A row outside the
// pool gives an (m, l) of NaN, so the request's output is NaN.  Uses 3.3 KB of the LDS after
// the workgroup's other LDS users are done.
template <int NT>
__device__ __forceinline__ void append_partial(const DecodeArgs& a, int b, int hg, int L, int p0, char* smem) {
  const int tid = threadIdx.x, H = a.num_heads;
  const int64_t slot = ((int64_t)b * a.part_splits + a.num_splits) * (H / 16) + hg;
  const int j = L - 1;
  const int page = a.kv_indices[p0 + (j >> a.page_shift)];
  const int64_t row = ((int64_t)page << a.page_shift) + (j & (a.page_size - 1));
  if (page < 0 || row >= a.pool_tokens) {   // uniform
    if (tid < 32) a.part_ml[slot * 32 + tid] = NAN;
    return;
  }
  float* xs = reinterpret_cast<float*>(smem);   // [576] the dequantized row
  float* red = xs + kD;                         // [NT / 16][16] partial dot products
  __syncthreads();
  if (tid < 36) {
    float x[16];
    load_src_block(static_cast<const uint8_t*>(a.app_src) + (int64_t)b * kD * (a.app_bf16 ? 2 : 1),
                   a.app_bf16 != 0, a.app_src_scale, tid, x);
    u32x2 packed;
    uint32_t sb;
    nvfp4_quantize_block(x, a.out_scale, packed, sb);
    if (hg == 0) {
      *reinterpret_cast<u32x2*>(a.app_data + row * kNvData + 8 * tid) = packed;
      a.app_scales[row * kNvScale + tid] = (uint8_t)sb;
    }
    const float sc = fp8x2_to_f32<false>(sb)[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 lo = fp4x2_to_f16<0>(packed[i >> 1] >> (16 * (i & 1)));
      const f16x2 hi = fp4x2_to_f16<1>(packed[i >> 1] >> (16 * (i & 1)));
      xs[16 * tid + 4 * i] = (float)lo[0] * sc;
      xs[16 * tid + 4 * i + 1] = (float)lo[1] * sc;
      xs[16 * tid + 4 * i + 2] = (float)hi[0] * sc;
      xs[16 * tid + 4 * i + 3] = (float)hi[1] * sc;
    }
  }
  __syncthreads();
  // q . row per head: thread -> head tid % 16, dims [part * kPer, (part + 1) * kPer)
  constexpr int kParts = NT / 16, kPer = kD / kParts;
  static_assert(kD % kParts == 0, "dims split evenly");
  const int h = tid & 15, part = tid >> 4;
  const uint16_t* qr = a.q + ((int64_t)b * H + 16 * hg + h) * kD + part * kPer;
  float dot = 0.0f;
  for (int i = 0; i < kPer; ++i) dot += u2f((uint32_t)qr[i] << 16) * xs[part * kPer + i];
  red[part * 16 + h] = dot;
  __syncthreads();
  if (tid < 16) {
    float sdot = 0.0f;
#pragma unroll
    for (int k = 0; k < kParts; ++k) sdot += red[k * 16 + tid];
    a.part_ml[slot * 32 + tid] = sdot * a.score_scale;
    a.part_ml[slot * 32 + 16 + tid] = 1.0f;
  }
  float* po = a.part_o + slot * (16 * kDV);
  for (int k = tid; k < 16 * kDV / 4; k += NT) {
    const int hh = k / (kDV / 4), d4 = k % (kDV / 4);
    *reinterpret_cast<f32x4*>(po + hh * kDV + 4 * d4) = *reinterpret_cast<const f32x4*>(xs + 4 * d4);
  }
}

template <int FMT, bool DIRECT, bool TILEPAGE, int NS>
__global__ __launch_bounds__(Geo<NS>::kThreads, 2) void mla_decode_kernel(DecodeArgs a) {
  constexpr int kStreams = Geo<NS>::kStreams, kTile = Geo<NS>::kTile, kWaves = Geo<NS>::kWaves;
  constexpr int kThreads = Geo<NS>::kThreads, kSwap = Geo<NS>::kSwap, kSmem = Geo<NS>::kSmem;
  typedef typename OpType<FMT>::type Op;
  // the waves' value tiles (kWaves x 16 KB) and the partial-score swap buffers (2 x kWaves x
  // 2 KB); at the end of the chunk, the waves' accumulators and the streams' (m, l)
  __shared__ __attribute__((aligned(16))) char smem[kSmem];

  const int split = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int tg = w % kStreams, dh = w / kStreams;   // the pair partner is w ^ kStreams
  const int H = a.num_heads;

  // ---- request bounds (device data, checked without faulting).  With a fused append the
  //      last of the L tokens is the new row: the tiles cover L - 1 tokens, and the workgroup
  //      whose chunk holds token L - 1 adds the new row as one more partial (append_partial).
  const bool app = FMT == FMT_NVFP4 && a.app_src != nullptr;
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npages = p1 - p0;
  const bool bad = L < (app ? 1 : 0) || L > a.max_kv_len || p0 < 0 || npages < 0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)npages * a.page_size < (int64_t)L;
  const int t_begin = split * a.chunk_tokens;
  const int t_end = bad ? t_begin : min(app ? L - 1 : L, t_begin + a.chunk_tokens);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  const int hbase = hg * 16;
  const bool app_here = app && !bad && t_begin <= L - 1 && L - 1 < t_begin + a.chunk_tokens;   // uniform
  if (ntiles == 0) {   // bad request or empty chunk
    if constexpr (DIRECT) {
      float* outb = a.out + ((int64_t)b * H + hbase) * kDV;
      for (int k = tid; k < 16 * kDV; k += kThreads) outb[k] = bad ? NAN : 0.0f;
      if (a.lse && tid < 16) a.lse[(int64_t)b * H + hbase + tid] = bad ? NAN : -INFINITY;
    } else {
      const int64_t slot = ((int64_t)b * a.part_splits + split) * (H / 16) + hg;
      if (tid < 16) {
        a.part_ml[slot * 32 + tid] = -INFINITY;
        a.part_ml[slot * 32 + 16 + tid] = 0.0f;
      }
    }
    if constexpr (FMT == FMT_NVFP4) {
      if (app_here) append_partial<kThreads>(a, b, hg, L, p0, smem);
    }
    return;
  }

  // ---- running state of this wave's stream: m for head l16, l_run the sum of the lane's own
  //      probabilities of head l16 (the lane groups' sums are added at the end of the chunk);
  //      O for heads 4grp+i, dims 256dh + 16nt + l16
  float m_run = kMinusBig, l_run = 0.0f;
  f32x4 o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the lane's token of block tb of a tile: 32tg + 16tb + l16
  const int my_tok = 16 * kBlocks * tg + l16;
  char* const vt = smem + w * kWaveV;
  float* const sX = reinterpret_cast<float*>(smem + kSwap);
  // one raw tile per wave: refilled with the next tile's rows as soon as it is converted (two
  // in flight do not fit the registers next to the output accumulator)
  RawTile<FMT> rawA[kBlocks];
  int stA[kBlocks];
  // prologue, ordered for the in-order load counter: the first two page-table batches, this
  // wave's half of the query rows, then the first tiles' rows; the query is converted while
  // those are in flight
  PageWindow pw;
  pw.init(a, p0, npages, t_begin, lane);
  const LaneOffsets lofs = lane_offsets<FMT>(my_tok, dh, grp);
  constexpr int kRowBytes = FMT == FMT_FP8 ? kD : FMT == FMT_NVFP4 ? kNvData : 2 * kD;
  // loads of the lane's share of tile t0 (both blocks) into r, validity states into s
  // (0 valid, 1 past the chunk, 2 no valid row; see tile_row).  With pages of at least a tile,
  // all lanes share the page: the tile's valid rows (tokens before t_end, rows inside the pool)
  // are rows row0 .. row0 + nvalid - 1, and lanes of other rows read zeros through the
  // descriptors' size limit, which fix_raw keeps (past the chunk) or replaces by NaN codes (a
  // whole page of the pool holds the tile, which never straddles pages; the pool's partial last
  // page holds pool_tail rows; any other id holds none).  The descriptors are formed apart from
  // the loads, so that their scalar chain can run beside the previous tile's conversion.
  struct TileDesc { BufferRsrc kv, sc; int nvalid; };
  auto tile_desc = [&](int t0) __attribute__((always_inline)) {
    const int page = pw.page<true>(a, t0, lane);
    const int off = t0 & (a.page_size - 1);
    const int want = max(0, min(kTile, t_end - t0));
    const int nvalid = (unsigned)page < (unsigned)a.pool_pages ? want
                       : page == a.pool_pages ? max(0, min(want, a.pool_tail - off)) : 0;
    const int64_t rbase = nvalid > 0 ? ((int64_t)page << a.page_shift) + off : 0;
    TileDesc d;
    d.kv = make_rsrc(a.kv + rbase * kRowBytes, nvalid * kRowBytes);
    d.sc = make_rsrc(FMT == FMT_NVFP4 ? a.kv_scales + rbase * kNvScale : a.kv, FMT == FMT_NVFP4 ? nvalid * kNvScale : 0);
    d.nvalid = nvalid;
    return d;
  };
  // (page tiles: the states of the lanes' rows are formed only for a tile with invalid rows, see
  // compute; s[0] keeps the tile's count of valid rows)
  auto issue = [&](RawTile<FMT>(&r)[kBlocks], int(&s)[kBlocks], const TileDesc& d) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb) load_raw_tile<FMT>(r[tb], d.kv, d.sc, lofs, dh, grp, 16 * tb);
    s[0] = d.nvalid;
  };
  auto fetch = [&](RawTile<FMT>(&r)[kBlocks], int(&s)[kBlocks], int t0) __attribute__((always_inline)) {
    if constexpr (TILEPAGE) {
      issue(r, s, tile_desc(t0));
    } else {
#pragma unroll
      for (int tb = 0; tb < kBlocks; ++tb) {
        const int tok = t0 + my_tok + 16 * tb;
        const int page = pw.page<false>(a, tok, lane);
        load_raw<FMT>(r[tb], a, tile_row(a, npages, tok, t_end, page, s[tb]), dh, grp);
      }
    }
  };
  u32x4 qraw[9];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * H + hbase + l16) * kD;
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) qraw[kb] = *reinterpret_cast<const u32x4*>(qrow + kb_dim<FMT>(dh, kb, grp));
  }
  fetch(rawA, stA, t_begin);

  Op qop[9];
  float score_scale = a.score_scale;
  if constexpr (FMT == FMT_BF16) {
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) qop[kb] = __builtin_bit_cast(bf16x8, qraw[kb]);
  } else {
    // exact bf16 -> fp16 with a power-of-two prescale 2^s per head chosen so that max|q| < 2^16
    // over both dim halves (the 4 lane groups of a head are the 4 rows of the wave; the pair
    // partners exchange their halves' maxima through the swap buffer that tile 1 uses first);
    // 2^-s goes into the score scale, which is then the same for both halves' partial scores
    uint32_t mx = 0;
#pragma unroll
    for (int kb = 0; kb < 9; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = qraw[kb][e];
        mx = max(mx, max((v & 0x7fffu) << 16, v & 0x7fff0000u));
      }
    float qmax = rows_max(u2f(mx));
    {
      float* const sX0 = reinterpret_cast<float*>(smem + kSwap);
      if (lane < 16) sX0[(kWaves + w) * (kSwapW / 4) + lane] = qmax;
      __syncthreads();
      qmax = fmaxf(qmax, sX0[(kWaves + (w ^ kStreams)) * (kSwapW / 4) + l16]);
    }
    const int ex = (int)((f2u(qmax) >> 23) & 0xff) - 127;       // floor(log2 max|q|)
    const int sh = (qmax == 0.0f || ex >= 128) ? 0 : min(15 - ex, 64);   // in [-112, 64]
    const float up = u2f((uint32_t)(127 + sh) << 23);
    score_scale = a.score_scale * u2f((uint32_t)(127 - sh) << 23);
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) {
      f16x8 qv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = qraw[kb][e];
        qv[2 * e] = (_Float16)(u2f(v << 16) * up);
        qv[2 * e + 1] = (_Float16)(u2f(v & 0xffff0000u) * up);
      }
      qop[kb] = qv;
    }
  }

  // NVFP4 rope block-scale byte selector (see dequant)
  uint32_t ssel;
  {
    const uint32_t b1 = (uint32_t)(2 * dh + (grp >> 1));
    ssel = b1 | (b1 << 8) | 0x0c0c0000u;
  }
  // Byte addresses in the wave's value tile (rows = its 32 tokens 16tb + r, dims relative to
  // 256dh).  Writes of k-block kb of block tb: row 16tb + l16, chunk kb_dim / 8 stored at its
  // bits 0-3 XOR vswz(l16): FP8 / BF16 chunk 16(m >> 1) + (8(m & 1) | 2g | h) for kb = 2m + h,
  // i.e. vwb ^ 16(8(m & 1) | h), plus 256(m >> 1); NVFP4 chunk 16(g >> 1) + (8(g & 1) | kb),
  // i.e. vwb ^ 16kb; plus 16 kVRow tb.  (Both write patterns and the reads below are
  // conflict-free, checked by enumeration.)  Transposed reads of dims 16nt + 4q .. +3 of block tb by lane
  // (g, 4i + q): row 16tb + 4g + i, chunk 16(nt >> 3) + ((2(nt & 7) | (q >> 1)) ^ vswz(row)),
  // i.e. vrb ^ 32(nt & 7), plus 256(nt >> 3) + 16 kVRow tb.
  const int vwb = FMT == FMT_NVFP4 ? l16 * kVRow + 256 * (grp >> 1) + 16 * ((8 * (grp & 1)) ^ vswz(l16))
                                   : l16 * kVRow + 16 * ((2 * grp) ^ vswz(l16));
  const int q4 = l16 & 3, vrow = 4 * grp + (l16 >> 2);
  const int vrb = vrow * kVRow + 16 * ((q4 >> 1) ^ vswz(vrow)) + 8 * (q4 & 1);

  // One tile: partial S^T of this wave's dim half for its two token blocks (value dims to
  // LDS), refill of the raw buffer with the next tile, swap of partial scores with the
  // pair partner, online softmax of the stream, O += P V over the wave's dim half.
  auto compute = [&](RawTile<FMT>(&cur)[kBlocks], int(&st)[kBlocks], int t0, int buf, bool more)
                     __attribute__((always_inline)) {
    // the next tile's descriptors, formed here (pinned by an empty use) so that their scalar
    // chain runs while the wave waits for this tile's rows rather than after the conversion
    TileDesc nd;
    if constexpr (TILEPAGE) {
      nd = tile_desc(t0 + kTile);
      asm volatile("" ::"s"(nd.kv), "s"(nd.sc));
    }
    if constexpr (TILEPAGE) {
      const int nvalid = __builtin_amdgcn_readfirstlane(st[0]);
      if (t0 + kTile > t_end || nvalid < kTile) {   // uniform: rows past the chunk or outside the pool
#pragma unroll
        for (int tb = 0; tb < kBlocks; ++tb) {
          const int tt = my_tok + 16 * tb;
          const int state = t0 + tt >= t_end ? 1 : (tt >= nvalid ? 2 : 0);
          if (__any(state != 0)) fix_raw<FMT>(cur[tb], state);
        }
      }
    } else {
#pragma unroll
      for (int tb = 0; tb < kBlocks; ++tb)
        if (__any(st[tb] != 0)) fix_raw<FMT>(cur[tb], st[tb]);
    }
    f32x4 sacc[kBlocks];
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb) sacc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#define MLAQ_QK_STEP(KB)                                                                          \
    _Pragma("unroll") for (int tb = 0; tb < kBlocks; ++tb) {                                      \
      const Op kop = dequant<FMT, KB>(cur[tb], ssel);                                             \
      sacc[tb] = mfma16x16x32(kop, qop[KB], sacc[tb]);                                            \
      if (KB < 8)                                                                                 \
        *reinterpret_cast<Op*>(vt + (FMT == FMT_NVFP4 ? (vwb ^ (16 * KB))                         \
                                     : (vwb ^ (16 * ((KB & 2) * 4 + (KB & 1)))) + 256 * (KB >> 2)) + \
                                     16 * kVRow * tb) = kop;                                     \
    }
    MLAQ_QK_STEP(0) MLAQ_QK_STEP(1) MLAQ_QK_STEP(2) MLAQ_QK_STEP(3) MLAQ_QK_STEP(4)
    MLAQ_QK_STEP(5) MLAQ_QK_STEP(6) MLAQ_QK_STEP(7) MLAQ_QK_STEP(8)
#undef MLAQ_QK_STEP
    // issue order of the 18 (k-block, token block) steps: about one step's conversion (10 VALU),
    // then one product and one value-tile write, so every product overlaps the next step's
    // conversion (measured: split kernel 1-2 % faster from HBM, 6 % with the KV in L2, than the
    // compiler's own order)
#pragma unroll
    for (int i = 0; i < 9 * kBlocks; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);   // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // LDS write
    }
    // the raw tile is converted: its registers take the loads of the next tile, which
    // are in flight during this tile's softmax and PV and the next tiles
    // wave priority: the conversion and QK stretch runs at the highest priority, so that
    // the other wave of the SIMD (of another workgroup) fills its gaps only while this one
    // waits; the score swap runs at 1, the softmax and PV (latency-bound) at 0
    __builtin_amdgcn_s_setprio(1);
    if (more) {
      if constexpr (TILEPAGE) issue(cur, st, nd);
      else fetch(cur, st, t0 + kTile);
    }
    // lane: head l16, tokens 32tg + 16tb + 4grp + i (partial sums of this dim half, unscaled:
    // both halves share the head's score scale, applied once to their sum)
    f32x4 sp[kBlocks];
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb) sp[tb] = sacc[tb];
    if (t0 + kTile > t_end) {   // partial tile (uniform)
#pragma unroll
      for (int tb = 0; tb < kBlocks; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + my_tok - l16 + 16 * tb + 4 * grp + i >= t_end) sp[tb][i] = -INFINITY;
    }
    // swap partial scores with the other half of the pair (buffer buf alternates with the
    // tiles: a wave reaches this barrier again only after its partner has read the previous
    // contents of the other buffer)
    float* const xw = sX + (buf * kWaves + w) * (kSwapW / 4);
    float* const xp = sX + (buf * kWaves + (w ^ kStreams)) * (kSwapW / 4);
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb) *reinterpret_cast<f32x4*>(xw + 256 * tb + 4 * lane) = sp[tb];
    // value operands of the first kVAhead dim blocks: they depend only on this wave's own
    // value tile, so they are read before the swap barrier and their latency overlaps the
    // wait for the partner.  Dim block nt of token block tb is at vrb ^ 32(nt & 7), plus
    // 256(nt >> 3) + 16 kVRow tb; the operand of the 32-token product is the pair of reads.
    // The base is made opaque per tile so that the 8 XORed addresses are recomputed (8 VALU)
    // instead of being held in registers across the loop.
    constexpr int kVAhead = 6;
    int vrb_t = vrb;
    asm volatile("" : "+v"(vrb_t));
    auto vread = [&](int nt) __attribute__((always_inline)) {
      const char* p = vt + (vrb_t ^ (32 * (nt & 7))) + 256 * (nt >> 3);
      const i16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 16 * kVRow);
      return i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    i16x8 vop[16];
#pragma unroll
    for (int nt = 0; nt < kVAhead; ++nt) vop[nt] = vread(nt);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    f32x4 sq[kBlocks];
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb) sq[tb] = *reinterpret_cast<const f32x4*>(xp + 256 * tb + 4 * lane);

    // online softmax of this stream (both waves of the pair compute the same values:
    // sp + sq and sq + sp round identically)
    float sc[4 * kBlocks];
#pragma unroll
    for (int tb = 0; tb < kBlocks; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * tb + i] = sp[tb][i] + sq[tb][i];
    // The reference point m_run of the exponentials moves only when a score exceeds it by more
    // than kSlack (log2 units), so probabilities stay below 2^kSlack (exact in fp16 / bf16 and
    // far from overflow in the fp32 sums) and the accumulators are rescaled only then.  Whether
    // any head must move is one vote over the lanes' own maxima; the heads' maxima over their
    // lane groups are formed only then.
    float lmax = sc[0];
#pragma unroll
    for (int j = 1; j < 4 * kBlocks; ++j) lmax = fmaxf(lmax, sc[j]);
    if (__any(lmax * score_scale > m_run + kSlack)) {
      const float tmax = rows_max(lmax) * score_scale;
      const bool grow = tmax > m_run + kSlack;
      const float m_new = grow ? tmax : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int nt = 0; nt < 16; ++nt) o[nt][i] *= ai;
      }
    }
    // P in the A-operand layout of the 32-token product: lane (g, head l16) holds k-indices
    // 8g .. 8g+7 = tokens 4g .. 4g+3 of block 0, then 4g .. 4g+3 of block 1
    Op pop;
#pragma unroll
    for (int j = 0; j < 4 * kBlocks; ++j) {
      // the sum takes the rounded probabilities the products use, so that the output is a
      // convex combination of value rows (rows with equal values reproduce them exactly)
      const float pe = fast_exp2(__builtin_fmaf(sc[j], score_scale, -m_run));
      if constexpr (FMT == FMT_BF16) pop[j] = (__bf16)pe;
      else pop[j] = (_Float16)pe;
    }
#pragma unroll
    for (int j = 0; j < 4 * kBlocks; j += 2) {    // the rounded pairs added to the sum, one dot2 per pair
      if constexpr (FMT == FMT_BF16)
        l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pop[j], pop[j + 1]}, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, l_run, false);
      else
        l_run = __builtin_amdgcn_fdot2(f16x2{pop[j], pop[j + 1]}, f16x2{(_Float16)1.0f, (_Float16)1.0f}, l_run, false);
    }
    // O += P V: 16 dims per product, K = this group's 32 tokens.  The operands are read in
    // batches of kVAhead dim blocks, each batch issued before the products of the previous
    // one (scheduling barriers keep the compiler from shortening that distance, so a product
    // does not wait on a read issued just before it)
#pragma unroll
    for (int nb = kVAhead; nb < 16 + kVAhead; nb += kVAhead) {
#pragma unroll
      for (int nt = nb; nt < nb + kVAhead && nt < 16; ++nt) vop[nt] = vread(nt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = nb - kVAhead; nt < nb && nt < 16; ++nt)
        o[nt] = mfma16x16x32(pop, __builtin_bit_cast(Op, vop[nt]), o[nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(3);   // the next tile's conversion and QK
  };

  __builtin_amdgcn_s_setprio(3);
  // ---- tile loop; the score swap buffers alternate with the tiles
  for (int k = 0; k < ntiles; ++k) compute(rawA, stA, t_begin + k * kTile, k & 1, k + 1 < ntiles);

  l_run = rows_sum(l_run);   // head l16's sum over the stream's tokens, in every lane group
  // ---- end of the chunk: merge of the token-group streams.  Stream tg: running max m_tg, sum
  //      l_tg; weights w_tg = 2^(m_tg - M), M = max_tg m_tg; L = sum_tg w_tg l_tg.
  //      Each wave leaves its accumulator in its own value tile, which no other wave reads and
  //      whose last reads (the products of the last tile) are done, as fp32 rows [head][256]
  //      with the 16-byte chunks of row h XORed by 4((h >> 2) & 3) (the lane groups of a write
  //      hit different banks, the 64 lanes of a row read hit 64 chunks); its (m, l) go to its
  //      slot of the swap buffer the last tile did not use (every wave read that buffer for the
  //      last time before the last tile's barrier).  With one stream a wave then reads back
  //      its own rows (in order within the wave); with two, one barrier, then wave (tg, dh)
  //      writes heads 8tg .. 8tg + 7 of dim half dh from both streams' rows.
  {
    float* const dump = reinterpret_cast<float*>(vt);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) dump[(4 * grp + i) * 256 + 16 * (nt ^ grp) + l16] = o[nt][i];
    if constexpr (kStreams > 1) {
      float* const tab = sX + ((ntiles & 1) * kWaves + w) * (kSwapW / 4);
      if (grp == 0) { tab[l16] = m_run; tab[16 + l16] = l_run; }
      __syncthreads();
    } else {
      __builtin_amdgcn_wave_barrier();
    }
  }
  constexpr int kHeadsPerWave = 16 / kStreams;
#pragma unroll
  for (int j = 0; j < kHeadsPerWave; ++j) {
    const int h = kHeadsPerWave * tg + j;
    float mg[kStreams], lg[kStreams];
#pragma unroll
    for (int g = 0; g < kStreams; ++g) {
      if constexpr (kStreams == 1) {
        mg[g] = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(m_run), h));   // lane h holds head h
        lg[g] = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(l_run), h));
      } else {
        const float* tab = sX + ((ntiles & 1) * kWaves + g) * (kSwapW / 4);
        mg[g] = tab[h];
        lg[g] = tab[16 + h];
      }
    }
    float M = kMinusBig;
#pragma unroll
    for (int g = 0; g < kStreams; ++g) M = fmaxf(M, mg[g]);
    float Lsum = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kStreams; ++g) {
      const float wg = fast_exp2(mg[g] - M);
      Lsum += wg * lg[g];
      const float* rows = reinterpret_cast<const float*>(smem + (g + kStreams * dh) * kWaveV);
      acc += *reinterpret_cast<const f32x4*>(rows + h * 256 + 4 * (lane ^ (4 * ((h >> 2) & 3)))) * wg;
    }
    const int d = 256 * dh + 4 * lane;
    if constexpr (DIRECT) {
      float f = Lsum > 0.0f ? a.out_scale / Lsum : 0.0f;
      if (Lsum != Lsum) f = Lsum;   // NaN stays NaN
      *reinterpret_cast<f32x4*>(a.out + ((int64_t)b * H + hbase + h) * kDV + d) = acc * f;
      if (a.lse && dh == 0 && lane == 0)
        a.lse[(int64_t)b * H + hbase + h] = Lsum > 0.0f ? (M + __log2f(Lsum)) * kLn2 : (Lsum != Lsum ? Lsum : -INFINITY);
    } else {
      const int64_t slot = ((int64_t)b * a.part_splits + split) * (H / 16) + hg;
      *reinterpret_cast<f32x4*>(a.part_o + slot * (16 * kDV) + h * kDV + d) = acc;
      if (dh == 0 && lane == 0) {
        a.part_ml[slot * 32 + h] = M;
        a.part_ml[slot * 32 + 16 + h] = Lsum;
      }
    }
  }
  if constexpr (FMT == FMT_NVFP4) {
    if (app_here) append_partial<kThreads>(a, b, hg, L, p0, smem);
  }
}

// Merge of the split partials of one (request, head, DIMS-dim chunk): weights
// w_s = 2^(m_s - M) over the splits (M = max_s m_s), output = sum_s w_s O_s / sum_s w_s l_s,
// natural-log lse.  The 256 threads are 1024 / DIMS groups of DIMS / 4 lanes; group k sums the
// splits s = k (mod groups), each lane 4 dims, so every load of a group is DIMS x 4 contiguous
// bytes.  Narrow chunks (DIMS = 32, 64 or 128) spread small batches over many workgroups;
// wide ones (DIMS = 256) keep large batches from repeating the weight computation.  Every load that
// does not depend on another one (the first batch of partials, all (m, l) pairs, the request's
// bounds) is issued up front, so the kernel pays one memory latency before its reductions;
// later batches of partials are loaded one batch ahead of their use.
constexpr int kMergeThreads = 256;
constexpr int kMergeUnroll = 4;                                  // splits per group per batch of loads
// partial slots per (request, head group): up to MLAQ_MAX_SPLITS splits, plus the new token's slot
// of a fused append
constexpr int kMergeMaxSlots = MLAQ_MAX_SPLITS + 1;
constexpr int kMergeMLPer = (kMergeMaxSlots + kMergeThreads - 1) / kMergeThreads;   // (m, l) per thread
template <int DIMS>
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(DecodeArgs a) {
  constexpr int kMergeDims = DIMS;                                 // dims per workgroup
  constexpr int kMergeGroups = kMergeThreads / (kMergeDims / 4);   // split-strided lane groups
  constexpr int kBatch = kMergeGroups * kMergeUnroll;              // splits per batch of loads
  __shared__ float sw[kMergeMaxSlots];
  __shared__ __attribute__((aligned(16))) float sred[kMergeGroups][kMergeDims];
  __shared__ float sx[2][4];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int grp = tid / (kMergeDims / 4), li = tid % (kMergeDims / 4);
  const int H = a.num_heads, hg = h >> 4, hh = h & 15, S = a.part_splits, HG = H / 16;
  const int64_t slot0 = (int64_t)b * S * HG + hg;
  const int64_t sstride = (int64_t)HG * 16 * kDV;
  const float* po = a.part_o + slot0 * (16 * kDV) + hh * kDV + kMergeDims * chunk + 4 * li;
  // first batch of partials (a split whose weight turns out 0 may hold stale data: it is
  // selected away below, never multiplied), then every (m, l) of the request's splits
  f32x4 v[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int s = grp + kMergeGroups * u;
    v[u] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mv[kMergeMLPer], lv[kMergeMLPer];
#pragma unroll
  for (int j = 0; j < kMergeMLPer; ++j) {
    const int s = tid + kMergeThreads * j;
    const float* ml = a.part_ml + (slot0 + (int64_t)s * HG) * 32;
    mv[j] = s < S ? ml[hh] : -INFINITY;
    lv[j] = s < S ? ml[16 + hh] : 0.0f;
  }
  // (a fused append's new token is the last partial slot; a request without it is invalid)
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const bool bad = L < (a.app_src ? 1 : 0) || L > a.max_kv_len || p0 < 0 || p1 < p0 ||
                   p1 > a.kv_indptr[a.batch] || (int64_t)(p1 - p0) * a.page_size < (int64_t)L;
  float* outp = a.out + ((int64_t)b * H + h) * kDV + kMergeDims * chunk;
  if (bad) {
    if (tid < kMergeDims) outp[tid] = NAN;
    if (a.lse && chunk == 0 && tid == 0) a.lse[(int64_t)b * H + h] = NAN;
    return;
  }
  // M = max_s m_s
  float mx = mv[0];
#pragma unroll
  for (int j = 1; j < kMergeMLPer; ++j) mx = fmaxf(mx, mv[j]);
  mx = wave_max(mx);
  if (lane == 0) sx[0][w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(sx[0][0], sx[0][1]), fmaxf(sx[0][2], sx[0][3]));
  float tot = 0.0f;
#pragma unroll
  for (int j = 0; j < kMergeMLPer; ++j) {
    const int s = tid + kMergeThreads * j;
    const float ws = mv[j] == -INFINITY ? 0.0f : exp2f(mv[j] - M);
    if (s < S) sw[s] = ws;
    tot += ws * lv[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  if (lane == 0) sx[1][w] = tot;
  __syncthreads();
  tot = (sx[1][0] + sx[1][1]) + (sx[1][2] + sx[1][3]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    f32x4 vn[kMergeUnroll];
    if (s0 + kBatch < S) {
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int s = s0 + kBatch + grp + kMergeGroups * u;
        vn[u] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + grp + kMergeGroups * u;
      const float ws = s < S ? sw[s] : 0.0f;
      if (ws != 0.0f) acc += ws * v[u];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) v[u] = vn[u];
  }
  *reinterpret_cast<f32x4*>(&sred[grp][4 * li]) = acc;
  __syncthreads();
  if (tid < kMergeDims) {
    float o = 0.0f;
#pragma unroll
    for (int g = 0; g < kMergeGroups; ++g) o += sred[g][tid];
    const float f = tot > 0.0f ? a.out_scale / tot : (tot != tot ? tot : 0.0f);
    outp[tid] = o * f;
  }
  if (a.lse && chunk == 0 && tid == 0)
    a.lse[(int64_t)b * H + h] = tot > 0.0f ? (M + __log2f(tot)) * kLn2 : (tot != tot ? tot : -INFINITY);
}

// The same merge for a few splits (at most kRowMergeMax partial slots): one wave per (request,
// head) row and 8 value dims per lane.  Every lane loads all of the row's (m, l) pairs and its
// dims of every partial at once, so the row costs one memory latency and no cross-lane step or
// barrier; the extend call's partials (one row per chunk token and head, two or three splits)
// take this path, where the chunked kernel above would run tens of thousands of workgroups with
// most of their lane groups idle.  The sums run over the splits as a pairwise tree.
constexpr int kRowMergeMax = 8;
constexpr int kRowMergeRows = 4;   // rows (waves) per workgroup

template <int LO, int N, typename T, int A>
__device__ __forceinline__ T tree_sum(const T (&x)[A]) {
  if constexpr (N == 1) return x[LO];
  else return tree_sum<LO, N / 2>(x) + tree_sum<LO + N / 2, N - N / 2>(x);
}

__global__ __launch_bounds__(64 * kRowMergeRows) void mla_merge_rows_kernel(DecodeArgs a) {
  const int H = a.num_heads, HG = H / 16, S = a.part_splits;
  const int row = blockIdx.x * kRowMergeRows + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.batch * H) return;                // wave-uniform
  const int b = row / H, h = row - b * H, hg = h >> 4, hh = h & 15;
  const int64_t slot0 = (int64_t)b * S * HG + hg;
  const int64_t sstride = (int64_t)HG * 16 * kDV;
  const float* po = a.part_o + slot0 * (16 * kDV) + hh * kDV + 8 * lane;
  f32x4 v[kRowMergeMax][2];
  float mv[kRowMergeMax], lv[kRowMergeMax];
#pragma unroll
  for (int s = 0; s < kRowMergeMax; ++s) {
    const float* ml = a.part_ml + (slot0 + (int64_t)s * HG) * 32;
    v[s][0] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
    v[s][1] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    mv[s] = s < S ? ml[hh] : -INFINITY;
    lv[s] = s < S ? ml[16 + hh] : 0.0f;
  }
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const bool bad = L < (a.app_src ? 1 : 0) || L > a.max_kv_len || p0 < 0 || p1 < p0 ||
                   p1 > a.kv_indptr[a.batch] || (int64_t)(p1 - p0) * a.page_size < (int64_t)L;
  float* outp = a.out + ((int64_t)b * H + h) * kDV + 8 * lane;
  if (bad) {
    *reinterpret_cast<f32x4*>(outp) = f32x4{NAN, NAN, NAN, NAN};
    *reinterpret_cast<f32x4*>(outp + 4) = f32x4{NAN, NAN, NAN, NAN};
    if (a.lse && lane == 0) a.lse[(int64_t)b * H + h] = NAN;
    return;
  }
  float M = mv[0];
#pragma unroll
  for (int s = 1; s < kRowMergeMax; ++s) M = fmaxf(M, mv[s]);
#pragma unroll
  for (int s = 0; s < kRowMergeMax; ++s) {
    // a split whose weight is 0 (no rows, or an unused slot) may hold stale data: selected away
    const float ws = mv[s] == -INFINITY ? 0.0f : exp2f(mv[s] - M);
    lv[s] *= ws;
    v[s][0] = ws != 0.0f ? ws * v[s][0] : f32x4{0.f, 0.f, 0.f, 0.f};
    v[s][1] = ws != 0.0f ? ws * v[s][1] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 v0[kRowMergeMax], v1[kRowMergeMax];
#pragma unroll
  for (int s = 0; s < kRowMergeMax; ++s) v0[s] = v[s][0], v1[s] = v[s][1];
  const float tot = tree_sum<0, kRowMergeMax>(lv);
  const f32x4 o0 = tree_sum<0, kRowMergeMax>(v0), o1 = tree_sum<0, kRowMergeMax>(v1);
  const float f = tot > 0.0f ? a.out_scale / tot : (tot != tot ? tot : 0.0f);
  *reinterpret_cast<f32x4*>(outp) = o0 * f;
  *reinterpret_cast<f32x4*>(outp + 4) = o1 * f;
  if (a.lse && lane == 0)
    a.lse[(int64_t)b * H + h] = tot > 0.0f ? (M + __log2f(tot)) * kLn2 : (tot != tot ? tot : -INFINITY);
}

// Launches; with profile events the kernel is launched through hipExtLaunchKernelGGL, which
// records them at the kernel's own start and end.
template <typename K>
static hipError_t launch(K kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t t0, hipEvent_t t1,
                         const DecodeArgs& a) {
  if (t0 || t1) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t0, t1, 0, a);
  else hipLaunchKernelGGL(kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

// Merge shape: small batches spread over more workgroups (narrow dim chunks); with at most
// 64 splits, 128-dim chunks (two batches of loads, half the workgroups) measured faster than
// 64-dim ones (5.2 vs 5.5 us at 8 requests x 16 heads x 64 splits), with more splits slower;
// with hundreds of splits, 32-dim chunks (twice the lane groups, half the batches per
// workgroup) were faster again (7.7 vs 8.2 us at 2 requests x 512 splits)
static hipError_t launch_fmt_merge(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (a.part_splits <= kRowMergeMax) {
    const int64_t rows = (int64_t)a.batch * a.num_heads;
    return launch(mla_merge_rows_kernel, dim3((unsigned)((rows + kRowMergeRows - 1) / kRowMergeRows)),
                  dim3(64 * kRowMergeRows), stream, t0, t1, a);
  }
  if (a.batch * a.num_heads <= 256) {
    if (a.part_splits <= 64)
      return launch(mla_merge_kernel<128>, dim3(kDV / 128, a.num_heads, a.batch), dim3(kMergeThreads), stream, t0,
                    t1, a);
    if (a.part_splits > 256)
      return launch(mla_merge_kernel<32>, dim3(kDV / 32, a.num_heads, a.batch), dim3(kMergeThreads), stream, t0, t1, a);
    return launch(mla_merge_kernel<64>, dim3(kDV / 64, a.num_heads, a.batch), dim3(kMergeThreads), stream, t0, t1, a);
  }
  return launch(mla_merge_kernel<256>, dim3(kDV / 256, a.num_heads, a.batch), dim3(kMergeThreads), stream, t0, t1,
                a);
}

template <int FMT, bool TILEPAGE, int NS>
static hipError_t launch_fmt(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  const dim3 grid(a.num_splits, a.batch, a.num_heads / 16), block(Geo<NS>::kThreads);
  if (a.num_splits == 1 && !a.app_src)
    return launch(mla_decode_kernel<FMT, true, TILEPAGE, NS>, grid, block, stream, ev.split_start, ev.split_end, a);
  hipError_t e = launch(mla_decode_kernel<FMT, false, TILEPAGE, NS>, grid, block, stream, ev.split_start,
                        ev.split_end, a);
  if (e != hipSuccess) return e;
  return launch_fmt_merge(a, stream, ev.merge_start, ev.merge_end);
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t stream) {
  return launch_fmt_merge(a, stream, nullptr, nullptr);
}

// Pages of at least a tile hold whole tiles (one descriptor per tile); shorter pages are
// read row by row.
template <int FMT>
static hipError_t launch_pages(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  constexpr int NS = decode_streams(FMT);
  return a.page_size >= Geo<NS>::kTile ? launch_fmt<FMT, true, NS>(a, stream, ev)
                                       : launch_fmt<FMT, false, NS>(a, stream, ev);
}

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  switch (fmt) {
    case FMT_FP8: return launch_pages<FMT_FP8>(a, stream, ev);
    case FMT_NVFP4: return launch_pages<FMT_NVFP4>(a, stream, ev);
    default: return launch_pages<FMT_BF16>(a, stream, ev);
  }
}

// ---- Scratch of the allocation-free decode (mla_decode_nvfp4_noalloc): the split partials of
//      one call, in a file-scope device array that the code object brings with it, so the call
//      needs no allocation.  Host code never passes the array's name to a kernel (in host code
//      it is only a stand-in for the symbol): its device address is looked up once per device,
//      with that device current, and kept.  Every call on a device shares that device's array.
static __device__ __align__(256) char scratch[MLAQ_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace mlaq
