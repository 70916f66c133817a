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
// gfx950 design (one workgroup = 4 waves = one request x one KV chunk x 16 heads):
//   * every head shares the single latent KV row, so each KV byte is read from HBM once and
//     both products are dense 16-head contractions on MFMA v_mfma_f32_16x16x32_{f16,bf16};
//   * tile = 64 tokens; wave w owns tokens 16w..16w+15 of the tile for S^T = K Q^T and
//     dims 128w..128w+127 of the output for O += P V;
//   * K rows go global -> VGPR with 16-byte loads issued one tile ahead, are converted to
//     fp16 in registers (FP8: exact; NVFP4: E2M1 -> fp16, times the fp16 E4M3 block
//     scale, exact since every E2M1 x E4M3 product is an fp16 value) and feed the QK MFMA
//     directly; the 512 value dims are also written once to LDS, from where the PV MFMA
//     operand is read with the gfx950 transposed LDS read (ds_read_b64_tr_b16);
//   * the per-tensor FP8 scale or NVFP4 global scale and a power-of-two query prescale
//     (bf16 queries are converted to fp16 exactly) are folded into the score scale and the
//     output scale;
//   * online softmax in fp32 (exp2 domain) per tile, kept identically in all 4 waves;
//   * the dimension a lane reads for the QK contraction is permuted (any order of the 576
//     dims gives the same dot product): lane group g of a wave takes dims
//     [64j + 16g, 64j + 16g + 16) for j = 0..8, so each lane loads 16 contiguous FP8
//     bytes (or 8 NVFP4 bytes = exactly one scale block) per j.
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kVStride = 528;   // fp16 elements per LDS value row: 1056 B, rows 8 banks apart
constexpr int kSStride = 68;    // floats per LDS score row (per head)

template <int FMT> struct RawTile;
template <> struct RawTile<FMT_FP8> { u32x4 d[9]; };
template <> struct RawTile<FMT_NVFP4> { u32x2 d[9]; uint32_t s[9]; };
template <> struct RawTile<FMT_BF16> { u32x4 d[18]; };

template <int FMT> struct OpType { typedef f16x8 type; };
template <> struct OpType<FMT_BF16> { typedef bf16x8 type; };

// Page id of the lane's token (clamped into the request's page list, so the load is always
// in bounds; validity is decided separately by tile_row).
__device__ __forceinline__ int load_page(const DecodeArgs& a, int p0, int npages, int tok) {
  const int pi = min(tok / a.page_size, max(npages - 1, 0));
  return a.kv_indices[p0 + pi];
}

// Pool row of the lane's token and its state: 0 = valid, 1 = beyond the chunk (contributes
// zeros, masked out of the softmax), 2 = bad page (contributes NaN).  Invalid lanes read row 0.
__device__ __forceinline__ int64_t tile_row(const DecodeArgs& a, int npages, int tok, int end, int page,
                                            int& state) {
  const int pi = tok / a.page_size;
  const int64_t row = (int64_t)page * a.page_size + (tok - pi * a.page_size);
  state = tok >= end ? 1 : (pi >= npages || page < 0 || row >= a.pool_tokens) ? 2 : 0;
  return state == 0 ? row : 0;
}

template <int FMT>
__device__ __forceinline__ void load_raw(RawTile<FMT>& r, const DecodeArgs& a, int64_t row, int grp) {
  if constexpr (FMT == FMT_FP8) {
    const u32x4* p = reinterpret_cast<const u32x4*>(a.kv + row * kD + 16 * grp);
#pragma unroll
    for (int j = 0; j < 9; ++j) r.d[j] = p[4 * j];
  } else if constexpr (FMT == FMT_NVFP4) {
    const u32x2* p = reinterpret_cast<const u32x2*>(a.kv + row * kNvData + 8 * grp);
#pragma unroll
    for (int j = 0; j < 9; ++j) r.d[j] = p[4 * j];
    const u32x4_a4* s = reinterpret_cast<const u32x4_a4*>(a.kv_scales + row * kNvScale);
    const u32x4 s0 = s[0], s1 = s[1];
    r.s[0] = s0[0]; r.s[1] = s0[1]; r.s[2] = s0[2]; r.s[3] = s0[3];
    r.s[4] = s1[0]; r.s[5] = s1[1]; r.s[6] = s1[2]; r.s[7] = s1[3];
    r.s[8] = reinterpret_cast<const uint32_t*>(a.kv_scales + row * kNvScale)[8];
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.kv) + row * kD + 16 * grp);
#pragma unroll
    for (int j = 0; j < 9; ++j) { r.d[2 * j] = p[8 * j]; r.d[2 * j + 1] = p[8 * j + 1]; }
  }
}

// Replace the data of masked lanes by zeros and of bad-page lanes by NaN codes.
template <int FMT>
__device__ __forceinline__ void fix_raw(RawTile<FMT>& r, int state) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t f = state == 2 ? 0x7f7f7f7fu : 0u;
#pragma unroll
    for (int j = 0; j < 9; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[j][e] = state ? f : r.d[j][e];
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint32_t f = state == 2 ? 0x7f7f7f7fu : 0u;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      r.d[j][0] = state ? 0u : r.d[j][0];
      r.d[j][1] = state ? 0u : r.d[j][1];
      r.s[j] = state ? f : r.s[j];
    }
  } else {
    const uint32_t f = state == 2 ? 0x7fc07fc0u : 0u;
#pragma unroll
    for (int j = 0; j < 18; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) r.d[j][e] = state ? f : r.d[j][e];
  }
}

// The MFMA operand for k-block 2j+H of the lane's token: dims 64j + 16g + 8H .. +8.
template <int FMT, int J, int H>
__device__ __forceinline__ typename OpType<FMT>::type dequant(const RawTile<FMT>& r, uint32_t scale_sel) {
  if constexpr (FMT == FMT_FP8) {
    uint32_t w0 = r.d[J][2 * H], w1 = r.d[J][2 * H + 1];
    f16x2 a = fp8x2_to_f16<false>(w0), b = fp8x2_to_f16<true>(w0);
    f16x2 c = fp8x2_to_f16<false>(w1), d = fp8x2_to_f16<true>(w1);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else if constexpr (FMT == FMT_NVFP4) {
    // block scale: byte g of scale dword J, replicated into both halves -> (s, s) in fp16
    uint32_t sb = __builtin_amdgcn_perm(r.s[J], r.s[J], scale_sel);
    f16x2 s2 = fp8x2_to_f16<false>(sb);
    uint32_t w = r.d[J][H];
    f16x2 a = fp4x2_to_f16<0>(w) * s2, b = fp4x2_to_f16<1>(w) * s2;
    f16x2 c = fp4x2_to_f16<2>(w) * s2, d = fp4x2_to_f16<3>(w) * s2;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    return __builtin_bit_cast(bf16x8, r.d[2 * J + H]);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

template <int FMT, bool DIRECT>
__global__ __launch_bounds__(kThreads, 2) void mla_decode_kernel(DecodeArgs a) {
  typedef typename OpType<FMT>::type Op;
  typedef typename std::conditional<FMT == FMT_BF16, __bf16, _Float16>::type Elem;
  __shared__ __attribute__((aligned(16))) Elem sV[kTile * kVStride];
  __shared__ __attribute__((aligned(16))) float sS[16 * kSStride];

  const int split = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int H = a.num_heads;

  // ---- request bounds (device data, checked without faulting)
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npages = p1 - p0;
  const bool bad = L < 0 || L > a.max_kv_len || p0 < 0 || npages < 0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)npages * a.page_size < (int64_t)L;
  const int t_begin = split * a.chunk_tokens;
  const int t_end = bad ? t_begin : min(L, t_begin + a.chunk_tokens);

  // ---- query operand: lane (head l16, group grp), k-block 2j+h holds dims 64j+16grp+8h..+8
  Op qop[18];
  float score_scale = a.score_scale;
  {
    const uint16_t* qrow = a.q + ((int64_t)b * H + hg * 16 + l16) * kD + 16 * grp;
    u32x4 qraw[18];
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      qraw[2 * j] = reinterpret_cast<const u32x4*>(qrow + 64 * j)[0];
      qraw[2 * j + 1] = reinterpret_cast<const u32x4*>(qrow + 64 * j)[1];
    }
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
      for (int k = 0; k < 18; ++k) qop[k] = __builtin_bit_cast(bf16x8, qraw[k]);
    } else {
      // exact bf16 -> fp16 with a power-of-two prescale 2^s chosen so that max|q| < 2^16
      uint32_t mx = 0;
#pragma unroll
      for (int k = 0; k < 18; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t v = qraw[k][e];
          mx = max(mx, max((v & 0x7fffu) << 16, v & 0x7fff0000u));
        }
      float qmax = wave_max(u2f(mx));
      int ex = (int)((f2u(qmax) >> 23) & 0xff) - 127;       // floor(log2 max|q|), -127 for 0
      int s = (qmax == 0.0f || ex >= 128) ? 0 : min(15 - ex, 64);   // s in [-112, 64]
      const float up = u2f((uint32_t)(127 + s) << 23);
      score_scale = a.score_scale * u2f((uint32_t)(127 - s) << 23);
#pragma unroll
      for (int k = 0; k < 18; ++k) {
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t v = qraw[k][e];
          o[2 * e] = (_Float16)(u2f(v << 16) * up);
          o[2 * e + 1] = (_Float16)(u2f(v & 0xffff0000u) * up);
        }
        qop[k] = o;
      }
    }
  }

  // ---- running state: m, l for head l16 (same in every lane group and wave); O for
  //      heads 4grp+i, dims 128w + 16nt + l16
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // NVFP4: v_perm selector replicating byte grp of a dword into bytes 0 and 1
  const uint32_t scale_sel = (uint32_t)grp | ((uint32_t)grp << 8) | 0x0c0c0000u;

  // ---- tile pipeline.  Two register buffers alternate (A holds even tiles, B odd ones): while
  //      one tile is computed, the other buffer's loads for the next tile are in flight, and the
  //      page id for the tile after that is loaded too.  Loads are issued unconditionally (lanes
  //      without a valid row read row 0), so the code between issue and use is straight-line
  //      and each half-iteration waits only for what the previous one issued.
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
  const int my_tok = 16 * w + l16;
  if (ntiles > 0) {
    RawTile<FMT> bufA, bufB;
    int stA, stB = 0;
    int page = load_page(a, p0, npages, t_begin + my_tok);
    load_raw<FMT>(bufA, a, tile_row(a, npages, t_begin + my_tok, t_end, page, stA), grp);
    page = load_page(a, p0, npages, t_begin + kTile + my_tok);

    auto compute = [&](RawTile<FMT>& cur, int st, int t0) __attribute__((always_inline)) {
      if (__any(st != 0)) fix_raw<FMT>(cur, st);
      // S^T = K Q^T for this wave's 16 tokens; the value dims also go to LDS
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      Elem* vrow = sV + (16 * w + l16) * kVStride + 16 * grp;
#define MLAQ_QK_STEP(J, HH)                                                   \
      {                                                                       \
        Op kop = dequant<FMT, J, HH>(cur, scale_sel);                         \
        s = mfma16x16x32(kop, qop[2 * J + HH], s);                            \
        if (J < 8) *reinterpret_cast<Op*>(vrow + 64 * J + 8 * HH) = kop;      \
      }
      MLAQ_QK_STEP(0, 0) MLAQ_QK_STEP(0, 1) MLAQ_QK_STEP(1, 0) MLAQ_QK_STEP(1, 1)
      MLAQ_QK_STEP(2, 0) MLAQ_QK_STEP(2, 1) MLAQ_QK_STEP(3, 0) MLAQ_QK_STEP(3, 1)
      MLAQ_QK_STEP(4, 0) MLAQ_QK_STEP(4, 1) MLAQ_QK_STEP(5, 0) MLAQ_QK_STEP(5, 1)
      MLAQ_QK_STEP(6, 0) MLAQ_QK_STEP(6, 1) MLAQ_QK_STEP(7, 0) MLAQ_QK_STEP(7, 1)
      MLAQ_QK_STEP(8, 0) MLAQ_QK_STEP(8, 1)
#undef MLAQ_QK_STEP
      // lane holds S for head l16, tokens 4grp+i of this wave's 16
      {
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 16 * w + 4 * grp + i;
          sv[i] = tok < t_end ? s[i] * score_scale : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(sS + l16 * kSStride + 16 * w + 4 * grp) = sv;
      }
      __syncthreads();

      // online softmax over the 64 tokens for head l16; P operands for both K-chunks
      float p[2][8];
      {
        const float* srow = sS + l16 * kSStride + 8 * grp;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(srow), x1 = *reinterpret_cast<const f32x4*>(srow + 4);
        const f32x4 x2 = *reinterpret_cast<const f32x4*>(srow + 32), x3 = *reinterpret_cast<const f32x4*>(srow + 36);
#pragma unroll
        for (int e = 0; e < 4; ++e) { p[0][e] = x0[e]; p[0][4 + e] = x1[e]; p[1][e] = x2[e]; p[1][4 + e] = x3[e]; }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, p[kc][e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = exp2f(m_run - m_new);
      float rsum = 0.0f;
      Op pop[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = exp2f(p[kc][e] - m_new);
          rsum += pe;
          pop[kc][e] = (Elem)pe;
        }
      rsum += __shfl_xor(rsum, 16);
      rsum += __shfl_xor(rsum, 32);
      l_run = l_run * alpha + rsum;
      m_run = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) o[nt][i] *= ai;
        }
      }

      // O += P V over this wave's 128 value dims (V operand by transposed LDS reads)
      {
        const int q4 = l16 & 3, r4 = l16 >> 2;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const Elem* vb = sV + (kc * 32 + grp * 8 + r4) * kVStride + 128 * w + 4 * q4;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) {
            const i16x4 lo = lds_read_tr16(vb + 16 * nt);
            const i16x4 hi = lds_read_tr16(vb + 4 * kVStride + 16 * nt);
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[nt] = mfma16x16x32(pop[kc], __builtin_bit_cast(Op, v8), o[nt]);
          }
        }
      }
      __syncthreads();
    };

    if constexpr (FMT == FMT_BF16) {
      // 16-bit pool (comparison path): one register buffer, the next tile is loaded after
      // the current one is consumed (two 72-register buffers would not fit).
      for (int k = 0; k < ntiles; ++k) {
        const int t0 = t_begin + k * kTile;
        compute(bufA, stA, t0);
        if (k + 1 >= ntiles) break;
        load_raw<FMT>(bufA, a, tile_row(a, npages, t0 + kTile + my_tok, t_end, page, stA), grp);
        page = load_page(a, p0, npages, t0 + 2 * kTile + my_tok);
      }
    } else {
    for (int k = 0; k < ntiles; k += 2) {
      const int t0 = t_begin + k * kTile;
      // tile k+1 -> B, page of tile k+2
      load_raw<FMT>(bufB, a, tile_row(a, npages, t0 + kTile + my_tok, t_end, page, stB), grp);
      page = load_page(a, p0, npages, t0 + 2 * kTile + my_tok);
      compute(bufA, stA, t0);
      if (k + 1 >= ntiles) break;
      // tile k+2 -> A, page of tile k+3
      load_raw<FMT>(bufA, a, tile_row(a, npages, t0 + 2 * kTile + my_tok, t_end, page, stA), grp);
      page = load_page(a, p0, npages, t0 + 3 * kTile + my_tok);
      compute(bufB, stB, t0 + kTile);
    }
    }
  }

  // ---- epilogue
  const int hbase = hg * 16;
  if constexpr (DIRECT) {
    float* outb = a.out + ((int64_t)b * H + hbase) * kDV;
    if (bad) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) outb[(4 * grp + i) * kDV + 128 * w + 16 * nt + l16] = NAN;
      if (a.lse && w == 0 && grp == 0) a.lse[(int64_t)b * H + hbase + l16] = NAN;
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float li = __shfl(l_run, 4 * grp + i);
      float f = li > 0.0f ? a.out_scale / li : 0.0f;
      if (li != li) f = li;   // NaN stays NaN
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) outb[(4 * grp + i) * kDV + 128 * w + 16 * nt + l16] = o[nt][i] * f;
    }
    if (a.lse && w == 0 && grp == 0)
      a.lse[(int64_t)b * H + hbase + l16] = l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2
                                                          : (l_run != l_run ? l_run : -INFINITY);
  } else {
    const int64_t slot = ((int64_t)b * a.num_splits + split) * (H / 16) + hg;
    float* ml = a.part_ml + slot * 32;
    if (w == 0 && grp == 0) {
      ml[l16] = (bad || t_begin >= t_end) ? -INFINITY : m_run;
      ml[16 + l16] = (bad || t_begin >= t_end) ? 0.0f : l_run;
    }
    if (bad || t_begin >= t_end) return;
    float* po = a.part_o + slot * (16 * kDV);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) po[(4 * grp + i) * kDV + 128 * w + 16 * nt + l16] = o[nt][i];
  }
}

// Merge of the split partials of one (request, head, 128-dim chunk) by one wave: weights
// 2^(m_s - M) over the splits, output = sum_s w_s O_s / sum_s w_s l_s, natural-log lse.
constexpr int kMergeDims = 128;
__global__ __launch_bounds__(64) void mla_merge_kernel(DecodeArgs a) {
  __shared__ float sw[1024];
  const int dc = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int H = a.num_heads, hg = h >> 4, hh = h & 15, S = a.num_splits, HG = H / 16;
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const bool bad = L < 0 || L > a.max_kv_len || p0 < 0 || p1 < p0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)(p1 - p0) * a.page_size < (int64_t)L;
  float* outp = a.out + ((int64_t)b * H + h) * kDV + dc * kMergeDims + 2 * lane;
  if (bad) {
    outp[0] = NAN; outp[1] = NAN;
    if (a.lse && dc == 0 && lane == 0) a.lse[(int64_t)b * H + h] = NAN;
    return;
  }
  const int64_t slot0 = (int64_t)b * S * HG + hg;
  float mx = -INFINITY;
  for (int s = lane; s < S; s += 64) mx = fmaxf(mx, a.part_ml[(slot0 + (int64_t)s * HG) * 32 + hh]);
  const float M = wave_max(mx);
  float tot = 0.0f;
  for (int s = lane; s < S; s += 64) {
    const float* ml = a.part_ml + (slot0 + (int64_t)s * HG) * 32;
    const float ms = ml[hh];
    const float ws = ms == -INFINITY ? 0.0f : exp2f(ms - M);
    sw[s] = ws;
    tot += ws * ml[16 + hh];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  __syncthreads();
  const float* po = a.part_o + slot0 * (16 * kDV) + hh * kDV + dc * kMergeDims + 2 * lane;
  const int64_t sstride = (int64_t)HG * 16 * kDV;
  float acc0 = 0.0f, acc1 = 0.0f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    f32x2 v[8];
    float wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      wv[u] = sw[s + u];
      v[u] = wv[u] != 0.0f ? *reinterpret_cast<const f32x2*>(po + (s + u) * sstride) : f32x2{0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) { acc0 += wv[u] * v[u][0]; acc1 += wv[u] * v[u][1]; }
  }
  for (; s < S; ++s) {
    const float ws = sw[s];
    if (ws != 0.0f) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(po + s * sstride);
      acc0 += ws * v[0];
      acc1 += ws * v[1];
    }
  }
  const float f = tot > 0.0f ? a.out_scale / tot : (tot != tot ? tot : 0.0f);
  outp[0] = acc0 * f;
  outp[1] = acc1 * f;
  if (a.lse && dc == 0 && lane == 0)
    a.lse[(int64_t)b * H + h] = tot > 0.0f ? (M + __log2f(tot)) * kLn2 : (tot != tot ? tot : -INFINITY);
}

template <int FMT>
static hipError_t launch_fmt(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  dim3 grid(a.num_splits, a.batch, a.num_heads / 16);
  hipError_t e;
  if (ev.before_split && (e = hipEventRecord(ev.before_split, stream)) != hipSuccess) return e;
  if (a.num_splits == 1) {
    hipLaunchKernelGGL((mla_decode_kernel<FMT, true>), grid, dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev.after_split && (e = hipEventRecord(ev.after_split, stream)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((mla_decode_kernel<FMT, false>), grid, dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev.after_split && (e = hipEventRecord(ev.after_split, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(kDV / kMergeDims, a.num_heads, a.batch), dim3(64), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev.after_merge && (e = hipEventRecord(ev.after_merge, stream)) != hipSuccess) return e;
  return hipSuccess;
}

hipError_t launch_decode(int fmt, const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  switch (fmt) {
    case FMT_FP8: return launch_fmt<FMT_FP8>(a, stream, ev);
    case FMT_NVFP4: return launch_fmt<FMT_NVFP4>(a, stream, ev);
    default: return launch_fmt<FMT_BF16>(a, stream, ev);
  }
}

}  // namespace mlaq
