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
//     both products are dense 16-head contractions on MFMA v_mfma_f32_16x16x32_{f16,bf16};
//   * tile = 64 tokens.  S^T = K Q^T is split over the waves as 4 token groups x 2 halves of
//     the 576 dims (wave w: tokens 16(w%4).., dims 288(w/4)..): each wave holds half of the
//     query operand and converts half of each of its 16 rows; the two partial scores meet in
//     LDS.  O += P V is split as 64 value dims per wave;
//   * K rows go global -> VGPR with 8/16-byte loads issued one tile ahead (two register
//     buffers), and are converted to fp16 in registers (FP8: exact; NVFP4: E2M1 -> fp16 times
//     the fp16 E4M3 block scale, exact since every E2M1 x E4M3 product is an fp16 value); the
//     converted operand feeds the QK MFMA directly, and its value dims are written once to
//     an XOR-swizzled LDS tile, from which the PV operand is read with the gfx950 transposed
//     LDS read (ds_read_b64_tr_b16);
//   * LDS value and score tiles are double-buffered, so one barrier per tile suffices: the
//     QK of tile k+1 in some waves overlaps the PV of tile k in others;
//   * the per-tensor FP8 scale or NVFP4 global scale and a power-of-two query prescale
//     (bf16 queries are converted to fp16 exactly) fold into the score and output scales;
//   * online softmax in fp32 (exp2 domain), kept identically in all 8 waves.
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kTile = 64;       // tokens per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalf = 288;      // dims per QK half
constexpr int kVStride = 512;   // fp16 elements per LDS value row (1024 B); 16-B chunks XOR-swizzled
constexpr int kSStride = 68;    // floats per LDS score row (one head)

// The lane's share of one token row for its dim half dh and lane group g:
//   k-block kb < 8 (m = kb/2, h = kb%2): dims 288dh + 64m + 16g + 8h .. +8;  kb = 8: dims
//   288dh + 256 + 8g .. +8.  (Any order of the 576 dims gives the same dot product; the query
//   operand uses the same map.)
template <int FMT> struct RawTile;
template <> struct RawTile<FMT_FP8> { u32x4 d[4]; u32x2 e; };                  // 4 x 16 B + 8 B
template <> struct RawTile<FMT_NVFP4> { u32x2 d[4]; uint32_t e; uint32_t s[5]; };  // codes + scales
template <> struct RawTile<FMT_BF16> { u32x4 d[9]; };                           // 9 x 16 B

template <int FMT> struct OpType { typedef f16x8 type; typedef _Float16 elem; };
template <> struct OpType<FMT_BF16> { typedef bf16x8 type; typedef __bf16 elem; };

// LDS value tile: row r (token) of 1024 B holds dims 0..511; its 16-byte chunk c is stored at
// chunk c ^ vswz(r), vswz(r) = 2 * ((r & 3) | ((r >> 3) & 1) << 2) | ((r >> 2) & 1).  With this
// map the 16-byte row writes of the QK phase and the transposed 8-byte reads of the PV phase
// touch every bank equally (checked by enumeration for 32 and 64 banks of 4 bytes).
__device__ __forceinline__ int vswz(int r) { return (((r & 3) | (((r >> 3) & 1) << 2)) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ int kb_dim(int dh, int kb, int g) {
  return kb < 8 ? kHalf * dh + 64 * (kb >> 1) + 16 * g + 8 * (kb & 1) : kHalf * dh + 256 + 8 * g;
}

// Page id of the lane's token (clamped into the request's page list, so the load is always
// in bounds; validity is decided separately by tile_row).  With TILEPAGE (pages of 64 or more
// tokens) a tile lies inside one page, so the id is the same for every lane and is read with
// a scalar load.
template <bool TILEPAGE>
__device__ __forceinline__ int load_page(const DecodeArgs& a, int p0, int npages, int t0, int my_tok) {
  const int pi = min((TILEPAGE ? t0 : t0 + my_tok) >> a.page_shift, max(npages - 1, 0));
  return a.kv_indices[p0 + pi];
}

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
    const uint8_t* base = a.kv + row * kD + kHalf * dh;
#pragma unroll
    for (int m = 0; m < 4; ++m) r.d[m] = *reinterpret_cast<const u32x4*>(base + 64 * m + 16 * g);
    r.e = *reinterpret_cast<const u32x2*>(base + 256 + 8 * g);
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint8_t* base = a.kv + row * kNvData + (kHalf / 2) * dh;
#pragma unroll
    for (int m = 0; m < 4; ++m) r.d[m] = *reinterpret_cast<const u32x2*>(base + 32 * m + 8 * g);
    r.e = *reinterpret_cast<const uint32_t*>(base + 128 + 4 * g);
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.kv_scales + row * kNvScale + 16 * dh);
    const u32x4 s4 = *reinterpret_cast<const u32x4_a4*>(sp);
    r.s[0] = s4[0]; r.s[1] = s4[1]; r.s[2] = s4[2]; r.s[3] = s4[3];
    r.s[4] = sp[4];
  } else {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(a.kv) + row * kD + kHalf * dh;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      r.d[2 * m] = *reinterpret_cast<const u32x4*>(base + 64 * m + 16 * g);
      r.d[2 * m + 1] = *reinterpret_cast<const u32x4*>(base + 64 * m + 16 * g + 8);
    }
    r.d[8] = *reinterpret_cast<const u32x4*>(base + 256 + 8 * g);
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

// MFMA operand of k-block KB of the lane's row half.  NVFP4: ssel[0] selects the block scale
// byte of k-blocks 0..7 from the 8-byte scale pair (s[m+1]:s[m]), ssel[1] that of k-block 8
// from s[4]; each selector also replicates the byte into both halves of the fp16 pair.
template <int FMT, int KB>
__device__ __forceinline__ typename OpType<FMT>::type dequant(const RawTile<FMT>& r, const uint32_t* ssel) {
  if constexpr (FMT == FMT_FP8) {
    const uint32_t w0 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1)] : r.e[0];
    const uint32_t w1 = KB < 8 ? r.d[KB >> 1][2 * (KB & 1) + 1] : r.e[1];
    const f16x2 a = fp8x2_to_f16<false>(w0), b = fp8x2_to_f16<true>(w0);
    const f16x2 c = fp8x2_to_f16<false>(w1), d = fp8x2_to_f16<true>(w1);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else if constexpr (FMT == FMT_NVFP4) {
    const uint32_t sb = KB < 8 ? __builtin_amdgcn_perm(r.s[(KB >> 1) + 1], r.s[KB >> 1], ssel[0])
                               : __builtin_amdgcn_perm(r.s[4], r.s[4], ssel[1]);
    const f16x2 s2 = fp8x2_to_f16<false>(sb);
    const uint32_t w = KB < 8 ? r.d[KB >> 1][KB & 1] : r.e;
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

template <int FMT, bool DIRECT, bool TILEPAGE>
__global__ __launch_bounds__(kThreads, 2) void mla_decode_kernel(DecodeArgs a) {
  typedef typename OpType<FMT>::type Op;
  typedef typename OpType<FMT>::elem Elem;
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  __shared__ __attribute__((aligned(16))) Elem sV[2][kTile * kVStride];
  __shared__ __attribute__((aligned(16))) float sS[2][2][16 * kSStride];

  const int split = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int tg = w & 3, dh = w >> 2;   // QK role: token group, dim half
  const int H = a.num_heads;

  // ---- request bounds (device data, checked without faulting)
  const int L = a.kv_lens[b];
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const int npages = p1 - p0;
  const bool bad = L < 0 || L > a.max_kv_len || p0 < 0 || npages < 0 || p1 > a.kv_indptr[a.batch] ||
                   (int64_t)npages * a.page_size < (int64_t)L;
  const int t_begin = split * a.chunk_tokens;
  const int t_end = bad ? t_begin : min(L, t_begin + a.chunk_tokens);

  // ---- running state: m, l for head l16 (same in every lane group and wave); O for
  //      heads 4grp+i, dims 64w + 16nt + l16
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTile - 1) / kTile : 0;
  const int my_tok = 16 * tg + l16;
  if (ntiles > 0) {
    RawTile<FMT> bufA, bufB;
    int stA, stB = 0;
    // prologue, ordered for the in-order load counter: page of tile 0, the query rows, then
    // tile 0's rows and the page of tile 1; the query is converted while those are in flight
    int page = load_page<TILEPAGE>(a, p0, npages, t_begin, my_tok);
    const uint16_t* qrow = a.q + ((int64_t)b * H + hg * 16 + l16) * kD;
    u32x4 qfull[9][2];   // dims 64j + 16grp .. +16: the whole row over the 4 lane groups
#pragma unroll
    for (int j = 0; j < 9; ++j) {
      qfull[j][0] = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * grp);
      qfull[j][1] = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * grp + 8);
    }
    u32x4 qraw[9];       // this wave's half, in the k-block map of RawTile
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) qraw[kb] = *reinterpret_cast<const u32x4*>(qrow + kb_dim(dh, kb, grp));
    load_raw<FMT>(bufA, a, tile_row(a, npages, t_begin + my_tok, t_end, page, stA), dh, grp);
    page = load_page<TILEPAGE>(a, p0, npages, t_begin + kTile, my_tok);

    // query operand; score scale
    Op qop[9];
    float score_scale = a.score_scale;
    if constexpr (FMT == FMT_BF16) {
#pragma unroll
      for (int kb = 0; kb < 9; ++kb) qop[kb] = __builtin_bit_cast(bf16x8, qraw[kb]);
    } else {
      // exact bf16 -> fp16 with a power-of-two prescale 2^s per head, chosen from the whole
      // row (the 4 lane groups of a head are the 4 rows of the wave) so that max|q| < 2^16;
      // 2^-s goes into that head's score scale
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < 9; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t v = qfull[j][hh][e];
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

    // NVFP4 block-scale byte selectors (see dequant): k-blocks 0..7 take byte 2dh + g of the
    // pair (s[m+1]:s[m]); k-block 8 takes byte 2dh + g/2 of s[4]
    uint32_t ssel[2];
    {
      const uint32_t b0 = (uint32_t)(2 * dh + grp), b1 = (uint32_t)(2 * dh + (grp >> 1));
      ssel[0] = b0 | (b0 << 8) | 0x0c0c0000u;
      ssel[1] = b1 | (b1 << 8) | 0x0c0c0000u;
    }
    // LDS offsets (elements).  Value writes: row my_tok, dims kb_dim(dh, kb, grp) (only those
    // below 512 are value dims), chunk XOR vswz(row).  Transposed reads: lane (grp, 4i + q)
    // reads row kc*32 + 8grp + i + 4bb, dims 64w + 16nt + 4q.
    int vw[9];
#pragma unroll
    for (int kb = 0; kb < 9; ++kb) {
      const int d0 = kb_dim(dh, kb, grp);
      vw[kb] = d0 < kDV ? my_tok * kVStride + 8 * ((d0 >> 3) ^ vswz(my_tok)) : -1;
    }
    const int q4 = l16 & 3, r4 = l16 >> 2, ra = r4 | ((grp & 1) << 2);
    int vr[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int row = 8 * grp + r4 + 4 * bb;
      vr[bb] = row * kVStride + 8 * (((8 * w + (q4 >> 1)) ^ vswz(row)) & ~6) + 4 * (q4 & 1);
    }
    // per N-tile: chunk bits 1..2 are nt ^ (ra & 3)
    int vx[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) vx[nt] = 16 * (nt ^ (ra & 3));

    auto compute = [&](RawTile<FMT>& cur, int st, int t0, int buf) __attribute__((always_inline)) {
      if (__any(st != 0)) fix_raw<FMT>(cur, st);
      Elem* v = sV[buf];
      // partial S^T over this wave's dim half for its 16 tokens; value dims to LDS
      f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // two MFMA chains
#define MLAQ_QK_STEP(KB)                                                          \
      {                                                                           \
        const Op kop = dequant<FMT, KB>(cur, ssel);                               \
        sacc[KB & 1] = mfma16x16x32(kop, qop[KB], sacc[KB & 1]);                  \
        if (vw[KB] >= 0) *reinterpret_cast<Op*>(v + vw[KB]) = kop;                \
      }
      MLAQ_QK_STEP(0) MLAQ_QK_STEP(1) MLAQ_QK_STEP(2) MLAQ_QK_STEP(3) MLAQ_QK_STEP(4)
      MLAQ_QK_STEP(5) MLAQ_QK_STEP(6) MLAQ_QK_STEP(7) MLAQ_QK_STEP(8)
#undef MLAQ_QK_STEP
      {
        const f32x4 s = sacc[0] + sacc[1];
        f32x4 sv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 16 * tg + 4 * grp + i;
          sv[i] = tok < t_end ? s[i] * score_scale : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(&sS[buf][dh][l16 * kSStride + 16 * tg + 4 * grp]) = sv;
      }
      __syncthreads();

      // scores of head l16 for tokens kc*32 + 8grp + e (both dim halves), then the value
      // operands of tokens 0-31, whose LDS latency overlaps the softmax
      float p[2][8];
      {
        const float* s0 = &sS[buf][0][l16 * kSStride + 8 * grp];
        const float* s1 = &sS[buf][1][l16 * kSStride + 8 * grp];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const f32x4 a0 = *reinterpret_cast<const f32x4*>(s0 + 32 * kc);
          const f32x4 a1 = *reinterpret_cast<const f32x4*>(s0 + 32 * kc + 4);
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(s1 + 32 * kc);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(s1 + 32 * kc + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { p[kc][e] = a0[e] + b0[e]; p[kc][4 + e] = a1[e] + b1[e]; }
        }
      }
      i16x4 vlo[4], vhi[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        vlo[nt] = lds_read_tr16(v + vr[0] + vx[nt]);
        vhi[nt] = lds_read_tr16(v + vr[1] + vx[nt]);
      }

      float tmax = -INFINITY;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, p[kc][e]);
      tmax = rows_max(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = fast_exp2(m_run - m_new);
      float rsum = 0.0f;
      Op pop[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = fast_exp2(p[kc][e] - m_new);
          rsum += pe;
          pop[kc][e] = (Elem)pe;
        }
      rsum = rows_sum(rsum);
      l_run = l_run * alpha + rsum;
      m_run = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[nt][i] *= ai;
        }
      }

      // O += P V over this wave's 64 value dims: tokens 0-31 with the operands already
      // requested, while those of tokens 32-63 are read
      i16x4 wlo[4], whi[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        wlo[nt] = lds_read_tr16(v + vr[0] + vx[nt] + 32 * kVStride);
        whi[nt] = lds_read_tr16(v + vr[1] + vx[nt] + 32 * kVStride);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const i16x8 v8 = {vlo[nt][0], vlo[nt][1], vlo[nt][2], vlo[nt][3], vhi[nt][0], vhi[nt][1], vhi[nt][2], vhi[nt][3]};
        o[nt] = mfma16x16x32(pop[0], __builtin_bit_cast(Op, v8), o[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const i16x8 v8 = {wlo[nt][0], wlo[nt][1], wlo[nt][2], wlo[nt][3], whi[nt][0], whi[nt][1], whi[nt][2], whi[nt][3]};
        o[nt] = mfma16x16x32(pop[1], __builtin_bit_cast(Op, v8), o[nt]);
      }
    };

    // ---- tile pipeline: two register buffers alternate (A holds even tiles, B odd ones);
    //      while one tile is computed, the other's loads and the next page id are in flight.
    //      Loads are issued unconditionally (lanes without a valid row read row 0), so the
    //      code between issue and use is straight-line.  LDS tiles alternate with the tiles.
    if constexpr (FMT == FMT_BF16) {
      // 16-bit pool (comparison path): one register buffer
      for (int k = 0; k < ntiles; ++k) {
        const int t0 = t_begin + k * kTile;
        compute(bufA, stA, t0, k & 1);
        if (k + 1 >= ntiles) break;
        load_raw<FMT>(bufA, a, tile_row(a, npages, t0 + kTile + my_tok, t_end, page, stA), dh, grp);
        page = load_page<TILEPAGE>(a, p0, npages, t0 + 2 * kTile, my_tok);
      }
    } else {
      for (int k = 0; k < ntiles; k += 2) {
        const int t0 = t_begin + k * kTile;
        load_raw<FMT>(bufB, a, tile_row(a, npages, t0 + kTile + my_tok, t_end, page, stB), dh, grp);
        page = load_page<TILEPAGE>(a, p0, npages, t0 + 2 * kTile, my_tok);
        compute(bufA, stA, t0, 0);
        if (k + 1 >= ntiles) break;
        load_raw<FMT>(bufA, a, tile_row(a, npages, t0 + 2 * kTile + my_tok, t_end, page, stA), dh, grp);
        page = load_page<TILEPAGE>(a, p0, npages, t0 + 3 * kTile, my_tok);
        compute(bufB, stB, t0 + kTile, 1);
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
        for (int nt = 0; nt < 4; ++nt) outb[(4 * grp + i) * kDV + 64 * w + 16 * nt + l16] = NAN;
      if (a.lse && w == 0 && grp == 0) a.lse[(int64_t)b * H + hbase + l16] = NAN;
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l_run, 4 * grp + i);
      float f = li > 0.0f ? a.out_scale / li : 0.0f;
      if (li != li) f = li;   // NaN stays NaN
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) outb[(4 * grp + i) * kDV + 64 * w + 16 * nt + l16] = o[nt][i] * f;
    }
    if (a.lse && w == 0 && grp == 0)
      a.lse[(int64_t)b * H + hbase + l16] = l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2
                                                          : (l_run != l_run ? l_run : -INFINITY);
  } else {
    const int64_t slot = ((int64_t)b * a.num_splits + split) * (H / 16) + hg;
    float* ml = a.part_ml + slot * 32;
    const bool empty = bad || t_begin >= t_end;
    if (w == 0 && grp == 0) {
      ml[l16] = empty ? -INFINITY : m_run;
      ml[16 + l16] = empty ? 0.0f : l_run;
    }
    if (empty) return;
    float* po = a.part_o + slot * (16 * kDV);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) po[(4 * grp + i) * kDV + 64 * w + 16 * nt + l16] = o[nt][i];
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

template <int FMT, bool TILEPAGE>
static hipError_t launch_fmt(const DecodeArgs& a, hipStream_t stream, const ProfileEvents& ev) {
  dim3 grid(a.num_splits, a.batch, a.num_heads / 16);
  hipError_t e;
  if (ev.before_split && (e = hipEventRecord(ev.before_split, stream)) != hipSuccess) return e;
  if (a.num_splits == 1) {
    hipLaunchKernelGGL((mla_decode_kernel<FMT, true, TILEPAGE>), grid, dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev.after_split && (e = hipEventRecord(ev.after_split, stream)) != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((mla_decode_kernel<FMT, false, TILEPAGE>), grid, dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev.after_split && (e = hipEventRecord(ev.after_split, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(kDV / kMergeDims, a.num_heads, a.batch), dim3(64), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ev.after_merge && (e = hipEventRecord(ev.after_merge, stream)) != hipSuccess) return e;
  return hipSuccess;
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
