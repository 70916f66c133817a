// Extend attention over the FP8 workspace with one shared K/V tile per workgroup.
//
// Extend (NVFP4 article on aitop.news, implementation item 2) attends every chunk token of a
// request over the same workspace rows (prefix, then the chunk), causally.  Attending each
// token in its own decode workgroup re-reads and re-converts every row once per token; here a
// workgroup of 8 waves takes 8 consecutive chunk tokens of one request, one wave per token over
// all 576 score dims and all 512 value dims (no partial scores to exchange), and walks the rows
// once for all of them: per tile of 32 rows the 512 threads load the FP8 rows (two tiles
// ahead) and convert them to fp16 into the next of two LDS tile buffers one tile ahead; every
// wave reads its K operands and its transposed V operands from the current one.  A wave holds
// its token's 16 x 512 fp32 accumulator (128 registers) and the query's dims 256 .. 575 (40);
// dims 0 .. 255 stay in LDS, read with the K operands, so that the V operands of the PV
// products can be read four products ahead within two waves per SIMD (256 registers).  One
// barrier per tile, at its end: the buffer the next tile's rows go to was last read before it,
// and the rows stored at the tile's start are visible after it.
// Token i of the request masks rows >= P + i + 1.  A single split writes out and lse;
// several splits write decode-layout partials for the merge kernel.
#include "device_common.h"
#include "mlaq_kernels.h"

namespace mlaq {

constexpr int kXT = 8;                          // chunk tokens per workgroup, one wave each
constexpr int kXWaves = kXT;
constexpr int kXThreads = 64 * kXWaves;         // 512
constexpr int kXRows = 32;                      // rows per tile (two 16-row MFMA blocks)
constexpr int kXRowB = 1152;                    // LDS bytes per tile row: 576 fp16 dims in 72 chunks
constexpr int kXTileB = kXRows * kXRowB;        // 36 KB
constexpr int kXBufs = 2;                       // tile buffers
constexpr int kXQL = 8;                         // query k-blocks (32 dims each) kept in LDS
constexpr int kXQW = 16 * 64 * kXQL;            // a wave's LDS query bytes (16 heads x 256 dims fp16)
constexpr int kXSmem = kXBufs * kXTileB + kXWaves * kXQW;   // 136 KB: one workgroup per CU
constexpr float kXMinusBig = -3.0e38f;
constexpr float kXSlack = 8.0f;
static_assert(kXSmem <= 160 * 1024, "LDS");

// Tile row r, 16-byte chunk c (dims 8c .. 8c+7) lives at chunk (c & ~15) | ((c & 15) ^ s(r))
// for c < 64 and at 64 + ((c & 7) ^ (s(r) & 7)) for the rope chunks, in unpadded 1152-byte
// rows (odd rows start half-way through the 64 banks).  As its bank-conflict counters show, the
// LDS serves a 16-byte read or write in groups of 16 lanes (lanes 8i .. 8i+7 with 8i+32 ..
// 8i+39) and the 8-byte transposed read in groups of 32 lanes; here those groups touch 8
// consecutive rows at chunks c and c ^ 2 (K operands and tile writes) or c and c ^ 1 (V
// operands).  s(r) for r = 0 .. 7 is 0, 11, 9, 14, 12, 2, 5, 7: with the odd rows' half-way
// start these are the eight 4-bit values of even weight, of which no two differ in exactly one
// bit, so every such group spreads over all 64 banks (checked by enumeration; the low 3 bits do
// the same for the rope chunks).
__device__ __forceinline__ int xswz(int r) { return (int)((0x752ce9b0u >> (4 * (r & 7))) & 15u); }
__device__ __forceinline__ int xoff(int r, int c) {
  const int s = xswz(r);
  return r * kXRowB + 16 * (c < 64 ? ((c & ~15) | ((c & 15) ^ s)) : (64 + ((c & 7) ^ (s & 7))));
}
// A wave's LDS query: head h's row of 512 bytes, chunk c (dims 8c .. 8c+7) at (c & ~15) |
// ((c & 15) ^ f(h)), f(h) for h = 0 .. 7 = 0, 1, 4, 5, 8, 9, 12, 13: a read group takes heads h0 ..
// h0+7 at chunks c and c ^ 2, and no two values of f differ by 2 in that bit, so it spreads over
// all banks (checked by enumeration).
__device__ __forceinline__ int qswz(int h) { return (int)((0xdc985410u >> (4 * (h & 7))) & 15u); }
// A value the compiler treats as new in every tile: the per-lane operand addresses derived from
// it are formed where they are used instead of being held in registers across the tile loop,
// which leaves the registers for reading V operands ahead of their products.
__device__ __forceinline__ int opaque(int x) { asm volatile("" : "+v"(x)); return x; }

__global__ __launch_bounds__(kXThreads, 1) void extend_attn_kernel(ExtendAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kXSmem];
  // workgroups in dispatch order take the requests' token blocks from the last (the most rows
  // in a causal chunk) to the first, all requests at each step, so the longest work starts
  // first and the short blocks fill in behind it
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int b = lin % gridDim.y, blk = gridDim.x - 1 - lin / gridDim.y;
  const int H = a.num_heads, HG = H >> 4;        // 16-head groups, each its own workgroups
  const int split = blockIdx.z / HG, hg = blockIdx.z - split * HG;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;

  // ---- request bounds (the checks of the view builder; invalid requests were given NaN there)
  const int P = a.prefix_lens[b], q0 = a.qo_indptr[b], C = a.qo_indptr[b + 1] - q0;
  const int p0 = a.kv_indptr[b], p1 = a.kv_indptr[b + 1];
  const bool ok = P >= 0 && P <= a.max_prefix_len && C >= 0 && C <= a.max_chunk_len && q0 >= 0 &&
                  q0 + C <= a.num_q && p0 >= 0 && p1 >= p0 && p1 <= a.kv_indptr[a.batch] &&
                  (int64_t)(p1 - p0) * a.page_size >= (int64_t)P;
  const int i0 = blk * kXT;
  if (!ok || i0 >= C) return;                    // uniform
  const int ci = i0 + w;                         // this wave's chunk token
  const bool tok = ci < C;                       // wave-uniform
  const int t = q0 + (tok ? ci : C - 1);         // its query row (a valid one for idle waves)
  const int vis = tok ? P + ci + 1 : 0;          // rows it sees
  const int rows_blk = P + min(C, i0 + kXT);     // rows any token of the block sees
  const int tiles_all = (rows_blk + kXRows - 1) / kXRows;
  const int tt0 = split * a.tiles_per_split;
  const int tt1 = min(tiles_all, tt0 + a.tiles_per_split);
  const int ntiles = max(0, tt1 - tt0);

  const uint8_t* reg = a.ws_rows + (int64_t)b * a.region_rows * kD;
  char* const tiles = smem;
  char* const qlds = smem + kXBufs * kXTileB + w * kXQW;   // this wave's query, k-blocks 0 .. kXQL - 1

  // tile loader: thread u of 1152 (16-byte groups; three rounds of 512, the last one partial)
  // takes row u % 32, dims 16(u / 32) .. +15; rows at or past rows_blk read zeros (descriptor limit)
  u32x4 raw[3];
  auto load = [&](int tt) __attribute__((always_inline)) {
    const int r0 = tt * kXRows;
    // uniform, and kept in a scalar register so the descriptor is one too (no per-lane loop)
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(kXRows, rows_blk - r0)));
    const BufferRsrc rs = make_rsrc(reg + (int64_t)r0 * kD, nrows * kD);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int u = tid + kXThreads * j;
      raw[j] = u < 1152 ? buffer_load_b128(rs, (u & 31) * kD + 16 * (u >> 5)) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
    char* tile = tiles + buf * kXTileB;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int u = tid + kXThreads * j;
      if (u < 1152) {
        const int r = u & 31, k = u >> 5;
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const f16x2 a0 = fp8x2_to_f16<false>(raw[j][e]), a1 = fp8x2_to_f16<true>(raw[j][e]);
          lo[2 * e] = __builtin_bit_cast(uint32_t, a0);
          lo[2 * e + 1] = __builtin_bit_cast(uint32_t, a1);
          const f16x2 b0 = fp8x2_to_f16<false>(raw[j][2 + e]), b1 = fp8x2_to_f16<true>(raw[j][2 + e]);
          hi[2 * e] = __builtin_bit_cast(uint32_t, b0);
          hi[2 * e + 1] = __builtin_bit_cast(uint32_t, b1);
        }
        *reinterpret_cast<u32x4*>(tile + xoff(r, 2 * k)) = lo;
        *reinterpret_cast<u32x4*>(tile + xoff(r, 2 * k + 1)) = hi;
      }
    }
  };

  // this token's query as fp16 (exact after a power-of-two prescale per head, folded into the
  // score scale), k-block kb of lane (g, head l16) = dims 32kb + 8g .. +7: blocks 0 .. kXQL - 1
  // go to LDS, the others stay in registers
  auto xdim = [&](int kb) { return 32 * kb + 8 * grp; };
  f16x8 qop[18 - kXQL];
  float score_scale;
  {
    const uint16_t* qrow = a.q + ((int64_t)t * H + 16 * hg + l16) * kD;
    u32x4 qraw[18];
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) qraw[kb] = *reinterpret_cast<const u32x4*>(qrow + xdim(kb));
    uint32_t mx = 0;
#pragma unroll
    for (int kb = 0; kb < 18; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max((qraw[kb][e] & 0x7fffu) << 16, qraw[kb][e] & 0x7fff0000u));
    const float qmax = rows_max(u2f(mx));
    const int ex = (int)((f2u(qmax) >> 23) & 0xff) - 127;
    const int sh = (qmax == 0.0f || ex >= 128) ? 0 : min(15 - ex, 64);
    const float up = u2f((uint32_t)(127 + sh) << 23);
    score_scale = a.score_scale * u2f((uint32_t)(127 - sh) << 23);
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      f16x8 qv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[2 * e] = (_Float16)(u2f(qraw[kb][e] << 16) * up);
        qv[2 * e + 1] = (_Float16)(u2f(qraw[kb][e] & 0xffff0000u) * up);
      }
      if (kb < kXQL) {
        const int c = 4 * kb + grp;
        *reinterpret_cast<f16x8*>(qlds + l16 * (64 * kXQL) + 16 * ((c & ~15) | ((c & 15) ^ qswz(l16)))) = qv;
      } else {
        qop[kb - kXQL] = qv;
      }
    }
  }

  // lane bases: K operand of k-block kb (chunk 4kb + g, or 64 + 4(kb - 16) + g for the rope),
  // rows block tb = krow + 256(kb >> 2) + (kx ^ 64(kb & 3)) + 16 kXRowB tb (kb < 16), krow + 1024 +
  // (kx8 ^ 64(kb - 16)) + 16 kXRowB tb (rope); LDS query block kb = 512 l16 + 256(kb >> 2) + (qx ^
  // 64(kb & 3)); V operand of dims 16nt + 4q of rows 16tb + 4g + i = vrow_b + 256(nt >> 3) + (vx ^
  // 32(nt & 7)) + 16 kXRowB tb
  const int krow = l16 * kXRowB, kx = 16 * (grp ^ xswz(l16)), kx8 = 16 * (grp ^ (xswz(l16) & 7));
  const int qx = 16 * (grp ^ qswz(l16));
  const int q4 = l16 & 3, vrow = 4 * grp + (l16 >> 2);
  const int vrow_b = vrow * kXRowB + 8 * (q4 & 1), vx = 16 * ((q4 >> 1) ^ xswz(vrow));

  // m for head l16; l_run the sum of the lane's own probabilities of head l16
  float m_run = kXMinusBig, l_run = 0.0f;
  f32x4 o[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // pipeline, one barrier per tile: tile k is in LDS buffer k % 2; the rows of tile k + 1
  // arrived in registers during tile k - 1 and are converted into buffer (k + 1) % 2 at the
  // start of tile k (its last readers, the products of tile k - 1, ran before the barrier that
  // ended tile k - 1), and they are visible to every wave after the barrier that ends tile k;
  // then the rows of tile k + 2 are loaded
  if (ntiles > 0) {
    load(tt0);
    store(0);
    if (ntiles > 1) load(tt0 + 1);
    __syncthreads();
  }
  int buf = 0;
  for (int k = 0; k < ntiles; ++k) {
    const int tt = tt0 + k, nbuf = buf ^ 1;
    if (k + 1 < ntiles) {
      store(nbuf);
      if (k + 2 < ntiles) load(tt + 2);
    }
    const char* tile = tiles + buf * kXTileB;
    const int kxk = opaque(kx), kx8k = opaque(kx8), qxk = opaque(qx);
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // QK: the K operands (chunk 4kb + g of the value dims, or 64 + 4(kb - 16) + g of the rope, of
    // row l16 + 16tb) and the LDS query blocks are read five reads ahead of their products
    f16x8 kops[36], qvs[kXQL];
#pragma unroll
    for (int kb = 0; kb < 18; ++kb) {
      if (kb < kXQL) qvs[kb] = *reinterpret_cast<const f16x8*>(qlds + l16 * (64 * kXQL) + 256 * (kb >> 2) + (qxk ^ (64 * (kb & 3))));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int off = kb < 16 ? krow + 256 * (kb >> 2) + (kxk ^ (64 * (kb & 3))) : krow + 1024 + (kx8k ^ (64 * (kb - 16)));
        kops[2 * kb + tb] = *reinterpret_cast<const f16x8*>(tile + off + 16 * kXRowB * tb);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 18; ++kb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) sacc[tb] = mfma16x16x32(kops[2 * kb + tb], kb < kXQL ? qvs[kb] : qop[kb - kXQL], sacc[tb]);
    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < 36 + kXQL - 5) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // scores of this token: lane (g, head l16) holds rows 32tt + 16tb + 4g + j
    float sc[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * tb + j] = sacc[tb][j] * score_scale;
    if (32 * tt + kXRows > P + i0 + 1) {           // uniform: the tile holds a row some token does not see
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (32 * tt + 16 * tb + 4 * grp + j >= vis) sc[4 * tb + j] = -INFINITY;
    }
    // lazy rescale as in the decode kernel: one vote over the lanes' own maxima, the heads'
    // maxima over their lane groups only when some reference must move
    float lmax = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) lmax = fmaxf(lmax, sc[j]);
    if (__any(lmax > m_run + kXSlack)) {
      const float tmax = rows_max(lmax);
      const bool grow = tmax > m_run + kXSlack;
      const float m_new = grow ? tmax : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) o[nt][i] *= ai;
      }
    }
    f16x8 pop;
    float rsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) pop[j] = (_Float16)fast_exp2(sc[j] - m_run);
#pragma unroll
    for (int j = 0; j < 8; j += 2)                 // the rounded probabilities the products use
      rsum = __builtin_amdgcn_fdot2(f16x2{pop[j], pop[j + 1]}, f16x2{(_Float16)1.0f, (_Float16)1.0f}, rsum, false);
    l_run += rsum;   // the lane's own rows; lane groups are added after the last tile
    // PV: the V operands are read four products ahead of their products
    const int vxk = opaque(vx);
    i16x8 vop[32];
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const char* pv = tile + vrow_b + 256 * (nt >> 3) + (vxk ^ (32 * (nt & 7)));
      const i16x4 lo = lds_read_tr16(pv), hi = lds_read_tr16(pv + 16 * kXRowB);
      vop[nt] = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) o[nt] = mfma16x16x32(pop, __builtin_bit_cast(f16x8, vop[nt]), o[nt]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 28; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __syncthreads();   // every wave is done with this tile's buffer; the next tile is visible
    buf = nbuf;
  }

  // ---- outputs of this token: O for heads 4g + i, dims 16nt + l16; (m, l) for head l16
  l_run = rows_sum(l_run);
  if (!tok) return;
  if (a.num_splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      const float L = __shfl(l_run, h);
      float f = L > 0.0f ? a.out_scale / L : 0.0f;
      if (L != L) f = L;
      float* dst = a.out + ((int64_t)t * H + 16 * hg + h) * kDV + l16;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[16 * nt] = o[nt][i] * f;
    }
    if (a.lse && grp == 0)
      a.lse[(int64_t)t * H + 16 * hg + l16] = l_run > 0.0f ? (m_run + __log2f(l_run)) * kLn2
                                                   : (l_run != l_run ? l_run : -INFINITY);
  } else {
    const int64_t slot = ((int64_t)t * a.num_splits + split) * HG + hg;   // the decode partial layout
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* dst = a.part_o + slot * (16 * kDV) + (4 * grp + i) * kDV + l16;
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) dst[16 * nt] = o[nt][i];
    }
    if (grp == 0) {
      a.part_ml[slot * 32 + l16] = ntiles > 0 ? m_run : -INFINITY;
      a.part_ml[slot * 32 + 16 + l16] = l_run;
    }
  }
}

hipError_t launch_extend_attn(const ExtendAttnArgs& a, hipStream_t stream) {
  const int nblk = (a.max_chunk_len + kXT - 1) / kXT;
  hipLaunchKernelGGL(extend_attn_kernel, dim3((unsigned)nblk, (unsigned)a.batch, (unsigned)(a.num_splits * (a.num_heads / 16))),
                     dim3(kXThreads), 0, stream, a);
  return hipGetLastError();
}

int extend_attn_tile_rows() { return kXRows; }
int extend_attn_tokens_per_group() { return kXT; }

}  // namespace mlaq
