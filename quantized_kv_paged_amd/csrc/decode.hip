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
// gfx950 design: one workgroup of 8 waves = one request x one KV chunk x 16 heads, one
// workgroup per CU.
//   * every head shares the single latent KV row, so each KV byte is read from HBM once and
//     both products are dense 16-head contractions on MFMA;
//   * tile = 64 tokens.  Wave w = (token group tg = w % 4, dim half dh = w / 4).  S^T = K Q^T
//     (v_mfma_f32_16x16x32) is split over the pair (tg, 0) / (tg, 1): half dh is value dims
//     256dh .. 256dh+255 plus rope dims 512+32dh .. +31; each wave holds that half of the query
//     operand and converts that half of each of its group's 16 rows, and the pair swaps 1 KB
//     of partial scores through LDS;
//   * each token group is its own online-softmax stream over the chunk; its probabilities are
//     already in the layout of the A operand of v_mfma_f32_16x16x16 (lane = head, 4 tokens),
//     so O += P V needs no score traffic: wave (tg, dh) accumulates the 256 value dims of half
//     dh over its 16 tokens, the V operand coming from LDS with one gfx950 transposed read
//     (ds_read_b64_tr_b16) per 16 dims.  The four streams are merged in LDS at the end;
//   * K rows go global -> VGPR with 8/16-byte loads issued one tile ahead (two register
//     buffers), and are converted to fp16 in registers (FP8: exact; NVFP4: E2M1 -> fp16 times
//     the fp16 E4M3 block scale, exact since every E2M1 x E4M3 product is an fp16 value); the
//     converted operand feeds the QK MFMA directly and its value dims are written once to an
//     XOR-swizzled LDS tile;
//   * LDS tiles are double-buffered, so one barrier per tile suffices;
//   * the per-tensor FP8 scale or NVFP4 global scale and a power-of-two query prescale
//     (bf16 queries are converted to fp16 exactly) fold into the score and output scales.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "mlaq.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kTile = 64;       // tokens per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kVRow = 1024;     // bytes per LDS value row (512 16-bit dims); 16-B chunks XOR-swizzled
constexpr float kMinusBig = -3.0e38f;   // initial running max: finite, so an empty stream stays finite
constexpr float kSlack = 8.0f;          // lazy-rescale threshold of the running max (log2 units)

// The lane's share of one token row for its dim half dh and lane group g:
//   k-block kb < 8 (m = kb/2, h = kb%2): value dims 256dh + 64m + 16g + 8h .. +8;  kb = 8:
//   rope dims 512 + 32dh + 8g .. +8.  (Any order of the 576 dims gives the same dot product;
//   the query operand uses the same map.)
template <int FMT> struct RawTile;
template <> struct RawTile<FMT_FP8> { u32x4 d[4]; u32x2 e; };                  // 4 x 16 B + 8 B
template <> struct RawTile<FMT_NVFP4> { u32x2 d[4]; uint32_t e; uint32_t s[5]; };  // codes + scales
template <> struct RawTile<FMT_BF16> { u32x4 d[9]; };                           // 9 x 16 B

template <int FMT> struct OpType { typedef f16x8 type; typedef _Float16 elem; };
template <> struct OpType<FMT_BF16> { typedef bf16x8 type; typedef __bf16 elem; };

// LDS value tile: row r (token) of 1024 B holds dims 0..511; its 16-byte chunk c is stored at
// chunk c ^ vswz(r), vswz(r) = x ^ 2x (mod 16) for x = r mod 16.  The 16-byte row writes of the
// QK phase (16 rows x 4 chunks per instruction) and the transposed 8-byte reads of the PV phase
// (16 rows x 2 chunks) then spread over all banks for any grouping of the wave's lanes into
// 256-byte (64 banks) or 128-byte (32 banks) cycles (checked by enumeration).  Since the XOR
// only touches chunk bits 0-3, every address is one per-lane base XOR a per-instruction
// constant in bits 4-7, plus a constant offset.
__device__ __forceinline__ int vswz(int r) { const int x = r & 15; return (x ^ (x << 1)) & 15; }

__device__ __forceinline__ int kb_dim(int dh, int kb, int g) {
  return kb < 8 ? 256 * dh + 64 * (kb >> 1) + 16 * g + 8 * (kb & 1) : 512 + 32 * dh + 8 * g;
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
    for (int m = 0; m < 4; ++m) r.d[m] = *reinterpret_cast<const u32x2*>(base + 128 * dh + 32 * m + 8 * g);
    r.e = *reinterpret_cast<const uint32_t*>(base + 256 + 16 * dh + 4 * g);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.kv_scales + row * kNvScale);
    const u32x4 s4 = *reinterpret_cast<const u32x4_a4*>(sp + 4 * dh);   // blocks 16dh .. 16dh+15
    r.s[0] = s4[0]; r.s[1] = s4[1]; r.s[2] = s4[2]; r.s[3] = s4[3];
    r.s[4] = sp[8];                                                      // rope blocks 32 .. 35
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
    for (int m = 0; m < 4; ++m) { r.d[m][0] = state ? 0u : r.d[m][0]; r.d[m][1] = state ? 0u : r.d[m][1]; }
    r.e = state ? 0u : r.e;
#pragma unroll
    for (int k = 0; k < 5; ++k) r.s[k] = state ? f : r.s[k];
  } else {
    const uint32_t f = state == 2 ? 0x7fc07fc0u : 0u;
#pragma unroll
    for (int k = 0; k < 9; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[k][e] = state ? f : r.d[k][e];
  }
}

// MFMA operand of k-block KB of the lane's row half.  NVFP4: the 16-dim block of k-block
// 2m + h is byte g of s[m] (selector ssel[0]), that of k-block 8 byte 2dh + g/2 of s[4]
// (ssel[1]); each selector also replicates the byte into both halves of the fp16 pair.
template <int FMT, int KB>
__device__ __forceinline__ typename OpType<FMT>::type dequant(const RawTile<FMT>& r, const uint32_t* ssel) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t w0 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1)] : r.e[0];
    const uint32_t w1 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1) + 1] : r.e[1];
    const f16x2 a = fp8x2_to_f16<false>(w0), b = fp8x2_to_f16<true>(w0);
    const f16x2 c = fp8x2_to_f16<false>(w1), d = fp8x2_to_f16<true>(w1);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint32_t sb = KB < 8 ? __builtin_amdgcn_perm(0u, r.s[KB >> 1], ssel[0])
                               : __builtin_amdgcn_perm(0u, r.s[4], ssel[1]);
    const f16x2 s2 = fp8x2_to_f16<false>(sb);
    const uint32_t w = KB < 8 ? r.d[KB >> 1][KB & 1] : r.e;
    const f16x2 a = fp4x2_to_f16<0>(w) * s2, b = fp4x2_to_f16<1>(w) * s2;
    const f16x2 c = fp4x2_to_f16<2>(w) * s2, d = fp4x2_to_f16<3>(w) * s2;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    return __builtin_bit_cast(bf16x8, r.d[KB]);
  }
}

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16x16x16(f16x4_t a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(i16x4 a, i16x4 b, f32x4 c) {   // bf16 bits
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int FMT, bool DIRECT, bool TILEPAGE>
__global__ __launch_bounds__(kThreads, 2) void mla_decode_kernel(DecodeArgs a) {
  typedef typename OpType<FMT>::type Op;
  typedef typename OpType<FMT>::elem Elem;
  typedef typename std::conditional<FMT == FMT_BF16, i16x4, f16x4_t>::type Pop;
  // value tiles (2 x 64 KB), reused as the 4-stream output buffer at the end; partial scores
  // of every wave (2 x 8 x 1 KB); per-stream running max / sum
  __shared__ __attribute__((aligned(16))) char sV[2][kTile * kVRow];
  __shared__ __attribute__((aligned(16))) float sX[2][kWaves][256];
  __shared__ float sML[4][2][16];

  const int split = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int tg = w & 3, dh = w >> 2;
  const int H = a.num_heads;

  // ---- request bounds (device data, checked without faulting)
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npages = p1 - p0;
  const bool bad = L < 0 || L > a.max_kv_len || p0 < 0 || npages < 0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)npages * a.page_size < (int64_t)L;
  const int t_begin = split * a.chunk_tokens;
  const int t_end = bad ? t_begin : min(L, t_begin + a.chunk_tokens);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;

  const int hbase = hg * 16;
  if (ntiles == 0) {   // bad request or empty chunk
    if constexpr (DIRECT) {
      float* outb = a.out + ((int64_t)b * H + hbase) * kDV;
      for (int k = tid; k < 16 * kDV; k += kThreads) outb[k] = bad ? NAN : 0.0f;
      if (a.lse && tid < 16) a.lse[(int64_t)b * H + hbase + tid] = bad ? NAN : -INFINITY;
    } else {
      const int64_t slot = ((int64_t)b * a.num_splits + split) * (H / 16) + hg;
      if (tid < 16) {
        a.part_ml[slot * 32 + tid] = -INFINITY;
        a.part_ml[slot * 32 + 16 + tid] = 0.0f;
      }
    }
    return;
  }

  // ---- running state of this wave's stream: m, l for head l16; O for heads 4grp+i,
  //      dims 256dh + 16nt + l16
  float m_run = kMinusBig, l_run = 0.0f;
  f32x4 o[16];
#pragma unroll
  for (int nt = 0; nt < 16; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int my_tok = 16 * tg + l16;
  RawTile<FMT> bufA, bufB;
  int stA, stB = 0;
  // prologue, ordered for the in-order load counter: the first two page-table batches, this
  // wave's half of the query rows, then tile 0's rows; the query is converted while those are
  // in flight
  PageWindow pw;
  pw.init(a, p0, npages, t_begin, lane);
  auto row_of = [&](int t0, int& st) __attribute__((always_inline)) {   // row of the lane's token of tile t0
    const int page = pw.page<TILEPAGE>(a, TILEPAGE ? t0 : t0 + my_tok, lane);
    return tile_row(a, npages, t0 + my_tok, t_end, page, st);
  };
  u32x4 qraw[9];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * H + hbase + l16) * kD;
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) qraw[kb] = *reinterpret_cast<const u32x4*>(qrow + kb_dim(dh, kb, grp));
  }
  load_raw<FMT>(bufA, a, row_of(t_begin, stA), dh, grp);

  Op qop[9];
  float score_scale = a.score_scale;
  if constexpr (FMT == FMT_BF16) {
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) qop[kb] = __builtin_bit_cast(bf16x8, qraw[kb]);
  } else {
    // exact bf16 -> fp16 with a power-of-two prescale 2^s per (head, dim half) chosen so that
    // max|q| < 2^16 (the 4 lane groups of a head are the 4 rows of the wave); 2^-s goes into
    // the score scale of this half's partial scores
    uint32_t mx = 0;
#pragma unroll
    for (int kb = 0; kb < 9; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t v = qraw[kb][e];
        mx = max(mx, max((v & 0x7fffu) << 16, v & 0x7fff0000u));
      }
    const float qmax = rows_max(u2f(mx));
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

  // NVFP4 block-scale byte selectors (see dequant)
  uint32_t ssel[2];
  {
    const uint32_t b0 = (uint32_t)grp, b1 = (uint32_t)(2 * dh + (grp >> 1));
    ssel[0] = b0 | (b0 << 8) | 0x0c0c0000u;
    ssel[1] = b1 | (b1 << 8) | 0x0c0c0000u;
  }
  // LDS byte addresses.  Value writes of k-block 2m + h: row my_tok, chunk
  // 32dh + 16(m >> 1) + ((8(m & 1) | 2g | h) ^ vswz(my_tok)), i.e. vwb ^ 16(8(m & 1) | h), plus
  // 256(m >> 1).  Transposed reads of dims 256dh + 16nt + 4q .. +3 by lane (g, 4i + q): row
  // 16tg + 4g + i, chunk 32dh + 16(nt >> 3) + ((2(nt & 7) | (q >> 1)) ^ vswz(row)), i.e.
  // vrb ^ 32(nt & 7), plus 256(nt >> 3).
  const int vwb = my_tok * kVRow + 512 * dh + 16 * ((2 * grp) ^ vswz(my_tok));
  const int q4 = l16 & 3, vrow = 16 * tg + 4 * grp + (l16 >> 2);
  const int vrb = vrow * kVRow + 512 * dh + 16 * ((q4 >> 1) ^ vswz(vrow)) + 8 * (q4 & 1);

  auto compute = [&](RawTile<FMT>& cur, int st, int t0, int buf) __attribute__((always_inline)) {
    if (__any(st != 0)) fix_raw<FMT>(cur, st);
    char* v = sV[buf];
    // partial S^T over this wave's dim half for its 16 tokens; value dims to LDS
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // two MFMA chains
#define MLAQ_QK_STEP(KB)                                                          \
    {                                                                             \
      const Op kop = dequant<FMT, KB>(cur, ssel);                                 \
      sacc[KB & 1] = mfma16x16x32(kop, qop[KB], sacc[KB & 1]);                    \
      if (KB < 8)                                                                 \
        *reinterpret_cast<Op*>(v + ((vwb ^ (16 * ((KB & 2) * 4 + (KB & 1)))) + 256 * (KB >> 2))) = kop; \
    }
    MLAQ_QK_STEP(0) MLAQ_QK_STEP(1) MLAQ_QK_STEP(2) MLAQ_QK_STEP(3) MLAQ_QK_STEP(4)
    MLAQ_QK_STEP(5) MLAQ_QK_STEP(6) MLAQ_QK_STEP(7) MLAQ_QK_STEP(8)
#undef MLAQ_QK_STEP
    // lane: head l16, tokens 16tg + 4grp + i
    f32x4 sp;
    {
      const f32x4 s = sacc[0] + sacc[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * tg + 4 * grp + i;
        sp[i] = tok < t_end ? s[i] * score_scale : -INFINITY;
      }
      *reinterpret_cast<f32x4*>(&sX[buf][w][4 * lane]) = sp;
    }
    __syncthreads();
    const f32x4 sq = *reinterpret_cast<const f32x4*>(&sX[buf][w ^ 4][4 * lane]);
    // value operands of the first 8 dim blocks (issued before the softmax arithmetic so their
    // latency overlaps it)
    i16x4 vop[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) vop[nt] = lds_read_tr16(v + (vrb ^ (32 * nt)));

    // online softmax of this stream (both waves of the pair compute the same values:
    // sp + sq and sq + sp round identically)
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sp[i] + sq[i];
    // The reference point m_run of the exponentials moves only when a score exceeds it by more
    // than kSlack (log2 units), so probabilities stay below 2^kSlack (exact in fp16 / bf16 and
    // far from overflow in the fp32 sums) and the accumulators are rescaled only then.
    const float tmax = rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const bool grow = tmax > m_run + kSlack;
    if (__any(grow)) {
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
    Pop pop;
    float rsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = fast_exp2(sc[i] - m_run);
      rsum += pe;
      if constexpr (FMT == FMT_BF16) pop[i] = (short)f32_to_bf16_rne(pe);
      else pop[i] = (_Float16)pe;
    }
    l_run += rows_sum(rsum);
    // O += P V: 16 dims per MFMA, K = this group's 16 tokens; the operands of dim blocks 8-15
    // are read while the first 8 products run
    i16x4 vop2[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) vop2[nt] = lds_read_tr16(v + (vrb ^ (32 * nt)) + 256);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[nt] = mfma16x16x16(pop, vop[nt], o[nt]);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) o[8 + nt] = mfma16x16x16(pop, vop2[nt], o[8 + nt]);
  };

  // ---- tile pipeline: two register buffers alternate (A holds even tiles, B odd ones);
  //      while one tile is computed, the other's loads are in flight.
  //      Loads are issued unconditionally (lanes without a valid row read row 0), so the code
  //      between issue and use is straight-line.  LDS tiles alternate with the tiles.
  if constexpr (FMT == FMT_BF16) {
    // 16-bit pool (comparison path): one register buffer
    for (int k = 0; k < ntiles; ++k) {
      const int t0 = t_begin + k * kTile;
      compute(bufA, stA, t0, k & 1);
      if (k + 1 >= ntiles) break;
      load_raw<FMT>(bufA, a, row_of(t0 + kTile, stA), dh, grp);
    }
  } else {
    for (int k = 0; k < ntiles; k += 2) {
      const int t0 = t_begin + k * kTile;
      load_raw<FMT>(bufB, a, row_of(t0 + kTile, stB), dh, grp);
      compute(bufA, stA, t0, 0);
      if (k + 1 >= ntiles) break;
      load_raw<FMT>(bufA, a, row_of(t0 + 2 * kTile, stA), dh, grp);
      compute(bufB, stB, t0 + kTile, 1);
    }
  }

  // ---- merge the four token-group streams in LDS.  Stream tg: running max m_tg, sum l_tg;
  //      weights w_tg = 2^(m_tg - M), M = max_tg m_tg; L = sum_tg w_tg l_tg.
  __syncthreads();                                   // all value-tile reads are done
  if (dh == 0 && grp == 0) { sML[tg][0][l16] = m_run; sML[tg][1][l16] = l_run; }
  __syncthreads();
  float* sO = reinterpret_cast<float*>(&sV[0][0]);   // [tg][head][512] fp32 = 128 KB
  {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      const float M = fmaxf(fmaxf(sML[0][0][h], sML[1][0][h]), fmaxf(sML[2][0][h], sML[3][0][h]));
      const float wi = fast_exp2(sML[tg][0][h] - M);
      float* dst = sO + (tg * 16 + h) * kDV + 256 * dh + l16;
#pragma unroll
      for (int nt = 0; nt < 16; ++nt) dst[16 * nt] = o[nt][i] * wi;
    }
  }
  __syncthreads();
  // thread -> heads 4(tid/128) .. +3, dims 4(tid % 128) .. +3
  const int dq = 4 * (tid & 127);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (tid >> 7) + i;
    float M = kMinusBig;
#pragma unroll
    for (int g = 0; g < 4; ++g) M = fmaxf(M, sML[g][0][h]);
    float Lsum = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) Lsum += fast_exp2(sML[g][0][h] - M) * sML[g][1][h];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) acc += *reinterpret_cast<const f32x4*>(sO + (g * 16 + h) * kDV + dq);
    if constexpr (DIRECT) {
      float f = Lsum > 0.0f ? a.out_scale / Lsum : 0.0f;
      if (Lsum != Lsum) f = Lsum;   // NaN stays NaN
      *reinterpret_cast<f32x4*>(a.out + ((int64_t)b * H + hbase + h) * kDV + dq) = acc * f;
      if (a.lse && (tid & 127) == 0)
        a.lse[(int64_t)b * H + hbase + h] = Lsum > 0.0f ? (M + __log2f(Lsum)) * kLn2 : (Lsum != Lsum ? Lsum : -INFINITY);
    } else {
      const int64_t slot = ((int64_t)b * a.num_splits + split) * (H / 16) + hg;
      *reinterpret_cast<f32x4*>(a.part_o + slot * (16 * kDV) + h * kDV + dq) = acc;
      if ((tid & 127) == 0) {
        a.part_ml[slot * 32 + h] = M;
        a.part_ml[slot * 32 + 16 + h] = Lsum;
      }
    }
  }
}

// Merge of the split partials of one (request, head, 256-dim half) by 4 waves: weights
// w_s = 2^(m_s - M) over the splits (M = max_s m_s), output = sum_s w_s O_s / sum_s w_s l_s,
// natural-log lse.  Wave w sums splits s = w (mod 4); each lane holds 4 dims.  The partial
// loads of the first 32 splits are issued before the weights are computed, so their latency
// overlaps that of the (m, l) loads and the reductions.
constexpr int kMergeThreads = 256;
constexpr int kMergeUnroll = 8;   // splits per wave per batch of loads
__global__ __launch_bounds__(kMergeThreads) void mla_merge_kernel(DecodeArgs a) {
  __shared__ float sw[MLAQ_MAX_SPLITS];
  __shared__ __attribute__((aligned(16))) float sred[4][256];
  __shared__ float sx[2][4];
  const int half = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int H = a.num_heads, hg = h >> 4, hh = h & 15, S = a.num_splits, HG = H / 16;
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const bool bad = L < 0 || L > a.max_kv_len || p0 < 0 || p1 < p0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)(p1 - p0) * a.page_size < (int64_t)L;
  float* outp = a.out + ((int64_t)b * H + h) * kDV + 256 * half;
  if (bad) {
    outp[tid] = NAN;
    if (a.lse && half == 0 && tid == 0) a.lse[(int64_t)b * H + h] = NAN;
    return;
  }
  const int64_t slot0 = (int64_t)b * S * HG + hg;
  const int64_t sstride = (int64_t)HG * 16 * kDV;
  const float* po = a.part_o + slot0 * (16 * kDV) + hh * kDV + 256 * half + 4 * lane;
  // first batch of partials (a split whose weight turns out 0 may hold stale data: it is
  // selected away below, never multiplied)
  f32x4 v[kMergeUnroll];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int s = w + 4 * u;
    v[u] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // M = max_s m_s
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kMergeThreads) mx = fmaxf(mx, a.part_ml[(slot0 + (int64_t)s * HG) * 32 + hh]);
  mx = wave_max(mx);
  if (lane == 0) sx[0][w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(sx[0][0], sx[0][1]), fmaxf(sx[0][2], sx[0][3]));
  float tot = 0.0f;
  for (int s = tid; s < S; s += kMergeThreads) {
    const float* ml = a.part_ml + (slot0 + (int64_t)s * HG) * 32;
    const float ms = ml[hh];
    const float ws = ms == -INFINITY ? 0.0f : exp2f(ms - M);
    sw[s] = ws;
    tot += ws * ml[16 + hh];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  if (lane == 0) sx[1][w] = tot;
  __syncthreads();
  tot = (sx[1][0] + sx[1][1]) + (sx[1][2] + sx[1][3]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 4 * kMergeUnroll) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int s = s0 + w + 4 * u;
        v[u] = s < S ? *reinterpret_cast<const f32x4*>(po + s * sstride) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + w + 4 * u;
      const float ws = s < S ? sw[s] : 0.0f;
      if (ws != 0.0f) acc += ws * v[u];
    }
  }
  *reinterpret_cast<f32x4*>(&sred[w][4 * lane]) = acc;
  __syncthreads();
  const float o = (sred[0][tid] + sred[1][tid]) + (sred[2][tid] + sred[3][tid]);
  const float f = tot > 0.0f ? a.out_scale / tot : (tot != tot ? tot : 0.0f);
  outp[tid] = o * f;
  if (a.lse && half == 0 && tid == 0)
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

template <int FMT, bool TILEPAGE>
static hipError_t launch_fmt(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  const dim3 grid(a.num_splits, a.batch, a.num_heads / 16);
  if (a.num_splits == 1)
    return launch(mla_decode_kernel<FMT, true, TILEPAGE>, grid, dim3(kThreads), stream, ev.split_start,
                  ev.split_end, a);
  hipError_t e = launch(mla_decode_kernel<FMT, false, TILEPAGE>, grid, dim3(kThreads), stream, ev.split_start,
                        ev.split_end, a);
  if (e != hipSuccess) return e;
  return launch(mla_merge_kernel, dim3(2, a.num_heads, a.batch), dim3(kMergeThreads), stream, ev.merge_start,
                ev.merge_end, a);
}

template <int FMT>
static hipError_t launch_pages(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  return a.page_size >= kTile ? launch_fmt<FMT, true>(a, stream, ev) : launch_fmt<FMT, false>(a, stream, ev);
}

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  switch (fmt) {
    case FMT_FP8: return launch_pages<FMT_FP8>(a, stream, ev);
    case FMT_NVFP4: return launch_pages<FMT_NVFP4>(a, stream, ev);
    default: return launch_pages<FMT_BF16>(a, stream, ev);
  }
}

}  // namespace mlaq
