// gnf4_grouped_gemm: one launch for all active experts, computing directly on
// the 4-bit packed weights with the codebook decoded in registers (Jordan
// Anderson, jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
// experts-4bit", first bullet: no dequantize-to-bf16 round trip; GitHub
// profile pjordanandrsn, grouped-nf4-gemm bullets).
//
// Two paths, picked on the host from T*k:
//
//  * gemv_kernel (decode, few rows per expert; HBM-bound). Persistent
//    workgroups walk (active expert, row block) items. Each lane owns a fixed
//    set of 16-byte code chunks (32 K values) of a weight row, keeps the
//    matching slice of up to MT token rows in registers as bf16 pairs, and
//    streams rows with coalesced 128-bit loads. NF4 bytes decode through a
//    per-lane-banked LDS table (one v_perm forms the address, one ds_read
//    yields two bf16 codebook values); MXFP4 bytes through
//    v_cvt_scalef32_pk_bf16_fp4. v_dot2c_f32_bf16 accumulates in float32 and
//    the block scale is applied once per 32-value chunk. Rows are reduced
//    across their lanes with DPP and permlane swaps.
//
//  * mfma16_kernel (prefill; a dense contraction per expert). Each workgroup
//    owns a 64 x 256 tile of one expert (tiles enumerated expert by expert,
//    N-tile major, then M-tile; the enumeration is XCD-aware so tiles that
//    share weight columns run on one XCD's L2). Gathered activation rows are
//    staged in LDS (double buffered, XOR-swizzled 16-byte segments); each
//    wave loads whole 64-byte lines of its weight columns, decodes them
//    straight into MFMA B fragments and runs v_mfma_f32_16x16x32_bf16.
//    NF4 / NF4_DQ: the bf16 codebook enters the MFMA and the float32 absmax
//    scales each 64-value partial before accumulation. MXFP4: the e8m0 scale
//    is folded into the (exact) bf16 decode.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace gnf4 {

constexpr int kThreads = 256;  // 4 waves per workgroup for both paths

// Sum over aligned groups of L lanes (L = 8, 16, 32 or 64); every lane of a
// group ends with the group sum. All 64 lanes must be active.
__device__ __forceinline__ float group_sum(float v, int L) {
  auto mov = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              decltype(ctrl)::value, 0xf, 0xf,
                                                              false));
  };
  v += mov(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: xor 1
  v += mov(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: xor 2
  v += mov(v, std::integral_constant<int, 0x141>{});  // row_half_mirror: pairs the quads
  if (L >= 16) v += mov(v, std::integral_constant<int, 0x140>{});  // row_mirror: pairs halves
  if (L >= 32) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, v),
                                              __builtin_bit_cast(unsigned, v), false, false);
    v = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
  if (L >= 64) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                              __builtin_bit_cast(unsigned, v), false, false);
    v = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  }
  return v;
}

// ===================================================================== GEMV

// Routed rows whose source activation row the GEMV caches in LDS.
constexpr int kGemvSrcCache = 1024;

// Per-thread register state of one GEMV item: its weight rows.
template <int U, int C>
struct GemvRows {
  uint4 q[U][C];
  float sc[U][C];
};

// Shape of the GEMV work split, fixed per launch.
struct GemvGeom {
  int L_log2, L, RW, li, seg, wave, KCH, rows_per_item;
  int ustride;   // wave slots between a wave's consecutive row slots (4: the
                 // workgroup's waves interleave; 1: a wave owns its rows)
  int half;      // SwiGLU epilogue: N / 2, the first up row (0 otherwise)
};

// Issue the code and scale loads of the rows of item block n0 of expert e:
// wave slot rows n0 + (u*4 + wave)*RW + seg, chunk li + c*L of each. Rows
// past N and chunks past K/32 load a valid neighbour instead (no predicated
// loads, so no load waits on an earlier one into the same registers); their
// results are discarded where they are used. Addresses are a uniform base of
// the item plus a 32-bit per-lane offset (one expert's packed matrix is
// below 4 GiB).
//
// SwiGLU epilogue (GLU): n0 is the first output column of the item, and the
// first U/2 slots take gate rows n0 + ..., the others the matching up rows
// half + n0 + ..., so that one lane holds each (gate, up) pair.
template <int FMT, int U, int C, bool GLU = false>
__device__ __forceinline__ void gemv_load_rows(const GemmArgs &a, const GemvGeom &g, int e, int n0,
                                               GemvRows<U, C> &R) {
  const int N = a.w.N, K = a.w.K;
  // Callers pass n0 < N (an item past the last row issues no loads); the
  // clamp keeps every row offset non-negative regardless.
  const int rmax = max(N - 1 - n0, 0);
  const int64_t row0 = (int64_t)e * N + n0;
  const uint8_t *cb = a.w.codes + row0 * (K / 2);
  uint32_t r[U], ch[C];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (GLU) {
      constexpr int UH = U / 2;
      const int rel = min(((u % UH) * g.ustride + g.wave) * g.RW + g.seg, g.half - 1 - n0);
      r[u] = (uint32_t)((u / UH) * g.half + rel);
    } else {
      r[u] = (uint32_t)min((u * g.ustride + g.wave) * g.RW + g.seg, rmax);
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) ch[c] = (uint32_t)min(g.li + c * g.L, g.KCH - 1);
  // The small scale loads go first and the code rows after them in row
  // order, so that row u waits only for rows before it.
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if constexpr (FMT == GNF4_MXFP4) {
        const uint8_t *sb = reinterpret_cast<const uint8_t *>(a.w.scales) + row0 * (K / 32);
        R.sc[u][c] = e8m0_to_f32(sb[r[u] * (uint32_t)(K / 32) + ch[c]]);
      } else if constexpr (FMT == GNF4_NF4) {
        const float *sb = reinterpret_cast<const float *>(a.w.scales) + row0 * (K / 64);
        R.sc[u][c] = sb[r[u] * (uint32_t)(K / 64) + (ch[c] >> 1)];
      } else {
        const int64_t blk0 = row0 * (K / 64);
        const uint32_t rb = r[u] * (uint32_t)(K / 64) + (ch[c] >> 1);
        const int8_t q8 = reinterpret_cast<const int8_t *>(a.w.scales)[blk0 + rb];
        R.sc[u][c] = (float)q8 * a.w.scales2[(blk0 + rb) >> 8];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // The codes are read once per call: non-temporal loads (measured 2-6 %
  // faster than default-policy loads on the decode shapes).
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const u32x4_t q = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t *>(cb + (r[u] * (uint32_t)(K / 2) + ch[c] * 16u)));
      R.q[u][c] = make_uint4(q[0], q[1], q[2], q[3]);
    }
  // MXFP4: every load of the item is issued before anything waits for one of
  // them (the compiler otherwise starts converting the first row's scales,
  // and waits for them, before the last code rows are requested): 3.6 %
  // faster on the gpt-oss-shaped one-token GEMV. The NF4 paths measured 0 to
  // 4 % slower with the same barrier and keep the compiler's order.
  if constexpr (FMT == GNF4_MXFP4) __builtin_amdgcn_sched_barrier(0);
}

// Token slices in registers: x[t][c][i] holds the bf16 pair for K values
// 32*ch + 2i, +1 of chunk ch = li + c*L, for routed rows p0 + tg + t (m >= 1
// rows from p0). Rows past the segment and chunks past K/32 load valid
// neighbours; their products are discarded.
template <int MT, int C>
__device__ __forceinline__ void gemv_load_x(const GemmArgs &a, const GemvGeom &g, const int *s_src,
                                            bool src_cached, int p0, int tg, int m,
                                            uint32_t (&x)[MT][C][16]) {
  const int K = a.w.K;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int p = p0 + min(tg + t, m - 1);
    const int src = src_cached ? s_src[p] : (a.gather ? a.perm[p] / a.k : p);
    const uint16_t *xrow = a.X + (int64_t)src * K;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int ch = min(g.li + c * g.L, g.KCH - 1);
      const uint4 *s4 = reinterpret_cast<const uint4 *>(xrow + ch * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = s4[j];
        x[t][c][4 * j + 0] = v.x;
        x[t][c][4 * j + 1] = v.y;
        x[t][c][4 * j + 2] = v.z;
        x[t][c][4 * j + 3] = v.w;
      }
    }
  }
}

// Decode and dot with the token slices; v[u][t] is the product of wave slot
// row u with token t, summed over its L lanes (every lane of the row group
// holds it).
template <int FMT, int MT, int U, int C>
__device__ __forceinline__ void gemv_dot(const GemvGeom &g, const uint32_t *lut, uint32_t lane4,
                                         const GemvRows<U, C> &R, const uint32_t (&x)[MT][C][16],
                                         float (&v)[U][MT]) {
  constexpr bool kLut = FMT != GNF4_MXFP4;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float part[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) part[t] = 0.f;
      const uint32_t qw[4] = {R.q[u][c].x, R.q[u][c].y, R.q[u][c].z, R.q[u][c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t pair;
          if constexpr (kLut) {
            pair = lut_read(lut, lut_addr(qw[j], lane4, i));
          } else {
            if (i == 0) pair = fp4_pair<0>(qw[j], 1.0f);
            else if (i == 1) pair = fp4_pair<1>(qw[j], 1.0f);
            else if (i == 2) pair = fp4_pair<2>(qw[j], 1.0f);
            else pair = fp4_pair<3>(qw[j], 1.0f);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) part[t] = dot2_bf16(pair, x[t][c][4 * j + i], part[t]);
        }
      }
      // A lane past the last chunk adds exactly zero. The mask is applied to
      // both factors with bitwise ANDs rather than a branch, which would let
      // the compiler sink this row's loads into it. NF4: the table holds
      // bf16(s * c), so the block's absmax enters divided by s.
      const uint32_t keep = g.li + c * g.L < g.KCH ? 0xffffffffu : 0u;
      const float sc = kLut ? R.sc[u][c] * kNF4InvScale : R.sc[u][c];
      const float s = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, sc) & keep);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_fmaf(s, __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, part[t]) & keep),
                                acc[t]);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) v[u][t] = group_sum(acc[t], g.L);
  }
}

// Store v[u][t] to row p0 + tg + t (t < m - tg) of Y, column of wave slot row u.
template <int MT, int U>
__device__ __forceinline__ void gemv_store(const GemmArgs &a, const GemvGeom &g,
                                           const float (&v)[U][MT], int n0, int p0, int tg, int m) {
  const int N = a.w.N;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = n0 + (u * g.ustride + g.wave) * g.RW + g.seg;
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (g.li == 0 && r < N && tg + t < m) a.Y[(int64_t)(p0 + tg + t) * N + r] = v[u][t];
  }
}

// SwiGLU epilogue: H[row][col] = bf16(silu(gate) * up) for the item's
// output columns col = n0 + ..., gate in slots u < U/2, up in u + U/2.
template <int MT, int U>
__device__ __forceinline__ void gemv_store_glu(const GemmArgs &a, const GemvGeom &g,
                                               const float (&v)[U][MT], int n0, int p0, int tg,
                                               int m) {
  constexpr int UH = U / 2;
#pragma unroll
  for (int u = 0; u < UH; ++u) {
    const int col = n0 + (u * g.ustride + g.wave) * g.RW + g.seg;
#pragma unroll
    for (int t = 0; t < MT; ++t)
      if (g.li == 0 && col < g.half && tg + t < m)
        a.H[(int64_t)(p0 + tg + t) * g.half + col] = swiglu_bf16(v[u][t], v[u + UH][t]);
  }
}

template <bool GLU, int MT, int U>
__device__ __forceinline__ void gemv_store_any(const GemmArgs &a, const GemvGeom &g,
                                               const float (&v)[U][MT], int n0, int p0, int tg,
                                               int m) {
  if constexpr (GLU) gemv_store_glu<MT, U>(a, g, v, n0, p0, tg, m);
  else gemv_store<MT, U>(a, g, v, n0, p0, tg, m);
}

// Token slice of activation row `src` (one token), chunks li + c*L (past
// K/32: a valid neighbour, discarded by the product mask).
template <int C>
__device__ __forceinline__ void gemv_load_x_row(const GemmArgs &a, const GemvGeom &g, int src,
                                                uint32_t (&x)[1][C][16]) {
  const uint16_t *xrow = a.X + (int64_t)src * a.w.K;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int ch = min(g.li + c * g.L, g.KCH - 1);
    const uint4 *s4 = reinterpret_cast<const uint4 *>(xrow + ch * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = s4[j];
      x[0][c][4 * j + 0] = v.x;
      x[0][c][4 * j + 1] = v.y;
      x[0][c][4 * j + 2] = v.z;
      x[0][c][4 * j + 3] = v.w;
    }
  }
}

// The one-token kernels stage a token row in LDS once per workgroup, so that
// the row is read from L2 once per workgroup rather than once per wave (every
// wave of the grid reads the same row, and a few L2 channels serve it). K is
// at most 64 lanes x 4 chunks x 32 values there.
constexpr int kGemv1MaxK = 8192;

// LDS slot of 16-byte piece j (0..3) of K chunk ch of a staged token row. The
// pieces of a chunk are permuted by the chunk index, so that the lanes that
// read consecutive chunks at one j fall on distinct banks (8 lanes of 16
// bytes cover 32 banks, 16 lanes 64 banks).
__device__ __forceinline__ int xs_slot(int ch, int j) {
  return ch * 4 + (j ^ (((ch >> 1) ^ (ch >> 3)) & 3));
}

// Staging a token row of K / 8 <= 1024 16-byte pieces: piece i is copied
// by thread first + (i mod stride), r = i / stride; at most two per thread
// (stride >= 512). The piece of round r of thread tid, -1 if none.
__device__ __forceinline__ int xs_piece(int tid, int first, int stride, int r, int n) {
  const int i = tid - first + r * stride;
  return (tid >= first && tid - first < stride && i < n) ? i : -1;
}

// A wave's token slice from the row staged in LDS (as gemv_load_x_row).
template <int C>
__device__ __forceinline__ void gemv_lds_x_row(const uint4 *s_x, const GemvGeom &g,
                                               uint32_t (&x)[1][C][16]) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int ch = min(g.li + c * g.L, g.KCH - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = s_x[xs_slot(ch, j)];
      x[0][c][4 * j + 0] = v.x;
      x[0][c][4 * j + 1] = v.y;
      x[0][c][4 * j + 2] = v.z;
      x[0][c][4 * j + 3] = v.w;
    }
  }
}

// GEMV: one workgroup per (active slot, row block) item, blockIdx.x = slot *
// items_per_expert + block; each wave holds U row slots of C chunks per lane
// in flight. The small routing arrays (offsets and the source row of every
// routed row) are read into LDS together with the slot's expert, so that the
// token slices and then the weight rows are issued back to back on the second
// memory round trip; the products of each row start as soon as that row
// has arrived while later rows are still streaming.
template <int FMT, int MT, int C, int U, bool GLU>
__global__ __launch_bounds__(kThreads, 2) void gemv_kernel(GemmArgs a, int L_log2,
                                                           int items_per_expert) {
  static_assert(!GLU || U % 2 == 0, "the SwiGLU epilogue pairs slot u with u + U/2");
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr int kPer = (GNF4_MAX_EXPERTS + kThreads) / kThreads;   // offsets per thread
  constexpr int kSrcPer = kGemvSrcCache / kThreads;
  __shared__ uint32_t lut[kLut ? kLutWords : 1];
  __shared__ int s_off[GNF4_MAX_EXPERTS + 1];
  __shared__ int s_src[kGemvSrcCache];

  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t lane4 = (uint32_t)lane << 2;
  GemvGeom g;
  g.L_log2 = L_log2;
  g.L = 1 << L_log2;
  g.RW = 64 >> L_log2;                          // rows per wave slot
  g.li = lane & (g.L - 1);
  g.seg = lane >> L_log2;
  g.wave = tid >> 6;
  g.ustride = 4;
  g.half = GLU ? a.w.N / 2 : 0;
  g.KCH = a.w.K >> 5;
  g.rows_per_item = 4 * g.RW * (GLU ? U / 2 : U);
  const int E = a.w.E, rows = a.T * a.k;
  const int slot = (int)(blockIdx.x / (unsigned)items_per_expert);
  const int ib = (int)(blockIdx.x - (unsigned)slot * (unsigned)items_per_expert);
  const bool src_cached = rows <= kGemvSrcCache;

  // ---- first round trip: the expert of this slot, offsets, sources -> LDS
  const int e = a.active[slot];
  int vo[kPer], vs[kSrcPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kThreads;
    vo[j] = i <= E ? a.offsets[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < kSrcPer; ++j) {
    const int i = tid + j * kThreads;
    vs[j] = (src_cached && i < rows) ? (a.gather ? a.perm[i] : i) : 0;
  }
  if constexpr (kLut) fill_nf4_lut_256(lut, tid);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + j * kThreads;
    if (i <= E) s_off[i] = vo[j];
  }
#pragma unroll
  for (int j = 0; j < kSrcPer; ++j) {
    const int i = tid + j * kThreads;
    if (src_cached && i < rows) s_src[i] = a.gather ? (vs[j] >= 0 ? vs[j] / a.k : 0) : vs[j];
  }
  __syncthreads();
  if (e < 0) return;                            // slot past the active count

  // ---- second round trip: token slices, then the weight rows
  const int n0 = ib * g.rows_per_item;
  const int p0 = s_off[e];
  const int m = s_off[e + 1] - p0;
  uint32_t x[MT][C][16];
  GemvRows<U, C> R;
  gemv_load_x<MT, C>(a, g, s_src, src_cached, p0, 0, m, x);
  __builtin_amdgcn_sched_barrier(0);
  gemv_load_rows<FMT, U, C, GLU>(a, g, e, n0, R);
  __builtin_amdgcn_sched_barrier(0);
  float v[U][MT];
  gemv_dot<FMT, MT, U, C>(g, lut, lane4, R, x, v);
  gemv_store_any<GLU, MT, U>(a, g, v, n0, p0, 0, m);
  // more routed rows than one token group (an expert routed several times)
  for (int tg = MT; tg < m; tg += MT) {
    gemv_load_x<MT, C>(a, g, s_src, src_cached, p0, tg, m, x);
    gemv_dot<FMT, MT, U, C>(g, lut, lane4, R, x, v);
    gemv_store_any<GLU, MT, U>(a, g, v, n0, p0, tg, m);
  }
}

// GEMV for one token (T = 1): the decode step of a single sequence. The
// only load the weight stream waits for is the slot's expert. The token
// slice is known without the routing: a gathered input has one row (token
// 0); an input already in routed order holds the slot's row at index slot
// whenever every lower active expert has one routed row, which the offsets
// confirm at the end (otherwise the rows are streamed again with the right
// slices). Offsets arrive while the products are computed.
template <int FMT, int C, int U, bool GLU>
__global__ __launch_bounds__(kThreads, 2) void gemv1_kernel(GemmArgs a, int L_log2,
                                                            int items_per_expert) {
  static_assert(!GLU || U % 2 == 0, "the SwiGLU epilogue pairs slot u with u + U/2");
  constexpr bool kLut = FMT != GNF4_MXFP4;
  __shared__ uint32_t lut[kLut ? kLutWords : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t lane4 = (uint32_t)lane << 2;
  GemvGeom g;
  g.L_log2 = L_log2;
  g.L = 1 << L_log2;
  g.RW = 64 >> L_log2;
  g.li = lane & (g.L - 1);
  g.seg = lane >> L_log2;
  g.wave = tid >> 6;
  g.ustride = 4;
  g.half = GLU ? a.w.N / 2 : 0;
  g.KCH = a.w.K >> 5;
  g.rows_per_item = 4 * g.RW * (GLU ? U / 2 : U);
  const int slot = (int)(blockIdx.x / (unsigned)items_per_expert);
  const int ib = (int)(blockIdx.x - (unsigned)slot * (unsigned)items_per_expert);

  const int e = a.active[slot];
  uint32_t x[1][C][16];
  gemv_load_x_row<C>(a, g, a.gather ? 0 : slot, x);
  if constexpr (kLut) fill_nf4_lut_256(lut, tid);
  if (e < 0) return;                            // whole workgroup: slot past the active count
  const int n0 = ib * g.rows_per_item;
  GemvRows<U, C> R;
  __builtin_amdgcn_sched_barrier(0);
  gemv_load_rows<FMT, U, C, GLU>(a, g, e, n0, R);
  __builtin_amdgcn_sched_barrier(0);
  const int p0 = a.offsets[e];
  const int p1 = a.offsets[e + 1];
  __syncthreads();                              // decode table written
  float v[U][1];
  gemv_dot<FMT, 1, U, C>(g, lut, lane4, R, x, v);
  const int m = p1 - p0;
  if (a.gather) {
    // every routed row of this expert is token 0: same products
    for (int t = 0; t < m; ++t) gemv_store_any<GLU, 1, U>(a, g, v, n0, p0 + t, 0, 1);
  } else if (m == 1 && p0 == slot) {
    gemv_store_any<GLU, 1, U>(a, g, v, n0, p0, 0, 1);
  } else {
    for (int t = 0; t < m; ++t) {               // rows streamed again (rare: repeated experts)
      gemv_load_x_row<C>(a, g, p0 + t, x);
      gemv_load_rows<FMT, U, C, GLU>(a, g, e, n0, R);
      gemv_dot<FMT, 1, U, C>(g, lut, lane4, R, x, v);
      gemv_store_any<GLU, 1, U>(a, g, v, n0, p0 + t, 0, 1);
    }
  }
}

// Persistent GEMV for one token's gathered input (T = 1, gather = 1: one
// activation row, every routed row of an expert gets the same products).
// Workgroups of 1024 threads share one decode table, filled once, so that 16
// waves per CU (4 per SIMD) hide each other's load latency: while one wave
// decodes, the others' rows are in flight. Each wave walks its own items (a
// slot and a block of RW * U rows) of the n_active * items_per_expert items,
// interleaved over the CUs. Lane j holds slot j's expert and routed-row
// range, read once: one token has at most 64 slots. The token row is staged
// in LDS once per workgroup.
constexpr int kGemvWaveThreads = 1024;

// Routing of one token's k <= 64 assignments, from the ids alone, computed
// by wave 0 of every workgroup of the fused one-token GEMV; the same result
// as gnf4_route. Lane j holds id e_j. With one ballot per id bit, most
// significant first, each lane finds the valid lanes with the same id (eq)
// and with a smaller id (lt); its stable position is |lt| + |eq below j|,
// the first lane of each id leads its slot, and slot s (experts ascending)
// is led by the lane with |lt & leaders| = s. Slot s's expert, first routed
// row and row count go to LDS for every wave; workgroup 0 writes perm, inv,
// n_active and bad, and the per-expert arrays (counts, offsets, active) are
// written 64 experts per workgroup once its GEMV items are done.
struct OneTokenRoute {
  int exp[64], seg[64], cnt[64];
  int nact, total;
};

// id0: wave 0's lane-j id e_j (-1 past k), loaded by the caller beforehand
// (unused with LOGITS).
template <bool LOGITS>
__device__ __forceinline__ void route_one_token(const GemmArgs &a, OneTokenRoute &sr, int tid,
                                                int id0) {
  const int lane = tid & 63, k = a.k, E = a.w.E;
  if (tid < 64) {
    int e;
    if constexpr (LOGITS) {                       // the router's top-k first (as gnf4_route_logits)
      float wt;
      topk_row<GNF4_MAX_EXPERTS / 64>(a.logits, E, k, lane, e, wt);
      if (blockIdx.x == 0 && lane < k) {
        a.r_topk_ids[lane] = e;
        a.r_topk_w[lane] = wt;
      }
      if (lane >= k) e = -1;
    } else {
      e = id0;
    }
    const bool valid = lane < k && (unsigned)e < (unsigned)E;
    const uint64_t vmask = __ballot(valid);
    uint64_t eq = vmask, lt = 0;
    for (int b = 31 - __builtin_clz((unsigned)max(E - 1, 1)); b >= 0; --b) {
      const bool bit = (e >> b) & 1;
      const uint64_t B = __ballot(valid && bit);
      if (bit) {
        lt |= eq & ~B;
        eq &= B;
      } else {
        eq &= ~B;
      }
    }
    const uint64_t lower = lane ? (~0ull >> (64 - lane)) : 0ull;
    const bool leader = valid && (eq & lower) == 0;
    const uint64_t lmask = __ballot(leader);
    const int pos = __popcll(lt) + __popcll(eq & lower);
    const int nact = __popcll(lmask), total = __popcll(vmask);
    if (leader) {
      const int slot = __popcll(lt & lmask);
      sr.exp[slot] = e;
      sr.seg[slot] = pos;
      sr.cnt[slot] = __popcll(eq);
    }
    if (lane == 0) {
      sr.nact = nact;
      sr.total = total;
    }
    if (blockIdx.x == 0 && lane < k) {
      a.r_inv[lane] = valid ? pos : -1;
      if (valid) a.r_perm[pos] = lane;
      if (lane >= total) a.r_perm[lane] = -1;
      if (lane == 0) {
        a.r_n_active[0] = nact;
        a.r_bad[0] = total != k ? 1 : 0;
      }
    }
  }
  __syncthreads();
}

// The per-expert routing arrays (counts, offsets, active), 64 experts per
// workgroup in turn; called after the GEMV items (nothing in the launch
// reads them).
__device__ __forceinline__ void route_one_token_arrays(const GemmArgs &a, const OneTokenRoute &sr,
                                                       int tid) {
  const int E = a.w.E;
  if (tid < 64) {
    const int nact = sr.nact;
    for (int e = (int)blockIdx.x * 64 + tid; e < E; e += (int)gridDim.x * 64) {
      int off = 0, c = 0;
      for (int s = 0; s < nact; ++s) {
        const int es = sr.exp[s];
        if (es < e) off += sr.cnt[s];
        if (es == e) c = sr.cnt[s];
      }
      a.r_counts[e] = c;
      a.r_offsets[e] = off;
      if (e == E - 1) a.r_offsets[E] = off + c;
      a.r_active[e] = e < nact ? sr.exp[e] : -1;
    }
  }
}

// ROUTE: 0 = routing read from a previous launch, 1 = routing from the k ids,
// 2 = the router's top-k from the logits, then the routing.
template <int FMT, int C, int U, bool GLU, int ROUTE>
__global__ __launch_bounds__(kGemvWaveThreads, 1) void gemv1w_kernel(GemmArgs a, int L_log2,
                                                                     int items_per_expert,
                                                                     int max_slots) {
  static_assert(!GLU || U % 2 == 0, "the SwiGLU epilogue pairs slot u with u + U/2");
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr int kWaves = kGemvWaveThreads / 64;
  __shared__ uint32_t lut[kLut ? kLutWords : 1];
  __shared__ OneTokenRoute sr;
  __shared__ uint4 s_x[kGemv1MaxK / 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t lane4 = (uint32_t)lane << 2;
  GemvGeom g;
  g.L_log2 = L_log2;
  g.L = 1 << L_log2;
  g.RW = 64 >> L_log2;
  g.li = lane & (g.L - 1);
  g.seg = lane >> L_log2;
  g.wave = 0;
  g.ustride = 1;
  g.half = GLU ? a.w.N / 2 : 0;
  g.KCH = a.w.K >> 5;
  g.rows_per_item = g.RW * (GLU ? U / 2 : U);
  const int ipe = items_per_expert;

  int nact, ej, pj0, pj1;                        // slot lane's expert and routed rows
  uint32_t x[1][C][16];
  // the token's ids first (wave 0 routes: the load is in flight during its
  // share of the table fill), then the token row to LDS, loaded by waves
  // 1..; the barrier below publishes it with the table
  int id0 = -1;
  if constexpr (ROUTE == 1) {
    if (tid < 64 && lane < a.k) id0 = a.ids[lane];
  }
  const int xp0 = xs_piece(tid, 64, kGemvWaveThreads - 64, 0, a.w.K / 8);
  const int xp1 = xs_piece(tid, 64, kGemvWaveThreads - 64, 1, a.w.K / 8);
  uint4 xv0, xv1;
  if (xp0 >= 0) xv0 = reinterpret_cast<const uint4 *>(a.X)[xp0];
  if (xp1 >= 0) xv1 = reinterpret_cast<const uint4 *>(a.X)[xp1];
  if constexpr (kLut) fill_nf4_lut<kGemvWaveThreads>(lut, tid);
  if (xp0 >= 0) s_x[xs_slot(xp0 >> 2, xp0 & 3)] = xv0;
  if (xp1 >= 0) s_x[xs_slot(xp1 >> 2, xp1 & 3)] = xv1;
  if constexpr (ROUTE) {
    route_one_token<ROUTE == 2>(a, sr, tid, id0); // ends with a barrier: table written too
    nact = sr.nact;
    const int sl = min(lane, 63);
    ej = lane < nact ? sr.exp[sl] : -1;
    pj0 = lane < nact ? sr.seg[sl] : 0;
    pj1 = lane < nact ? sr.seg[sl] + sr.cnt[sl] : 0;
  } else {
    nact = *a.n_active;
    ej = a.active[min(lane, max_slots - 1)];     // lanes past the active slots: unused
    const int ejc = max(ej, 0);
    pj0 = a.offsets[ejc];
    pj1 = a.offsets[ejc + 1];
    __syncthreads();                              // decode table written
  }
  gemv_lds_x_row<C>(s_x, g, x);

  const int total = nact * ipe;
  const int W = (int)gridDim.x * kWaves;
  GemvRows<U, C> R;
  float v[U][1];
  for (int it = (tid >> 6) * (int)gridDim.x + (int)blockIdx.x; it < total; it += W) {
    const int slot = it / ipe;
    const int n0 = (it - slot * ipe) * g.rows_per_item;
    gemv_load_rows<FMT, U, C, GLU>(a, g, __builtin_amdgcn_readlane(ej, slot), n0, R);
    gemv_dot<FMT, 1, U, C>(g, lut, lane4, R, x, v);
    const int p0 = __builtin_amdgcn_readlane(pj0, slot);
    const int m = __builtin_amdgcn_readlane(pj1, slot) - p0;
    for (int t = 0; t < m; ++t) gemv_store_any<GLU, 1, U>(a, g, v, n0, p0 + t, 0, 1);
  }
  if constexpr (ROUTE) route_one_token_arrays(a, sr, tid);
}

// One token's second projection with the combine as its epilogue (T = 1,
// activation rows in routed order): out[n] = sum_j w[j] * Y[inv[j]][n] over
// j ascending, dropped copies (inv = -1) skipped, where Y[p][n] is the
// float32 product the one-token GEMV forms (same lane geometry, same
// reduction) and the sum uses the combine's operations in its order; so out
// equals gnf4_grouped_gemm followed by gnf4_combine bit for bit, without
// writing or reading Y. One workgroup of 8 waves per G blocks of RW * U
// output rows; a task is (row block, routed row p), one wave each, and the
// products meet in LDS where one thread per output row adds them up.
//
// Routed row p belongs to the p-th active expert whenever every active
// expert has one routed row (a token's k distinct ids), so a task reads
// active[p] and streams that expert's rows at once, with a single memory
// round trip before the weights. The expert's offsets, loaded after the
// weights, confirm it; otherwise (repeated ids, dropped ids) the task finds
// row p's expert by a binary search of the offsets and streams again.
constexpr int kGemvCombineThreads = 512;

// The expert of routed row p (p < k), -1 if there is no such row (dropped
// ids): active[p] when that expert's only row is p, else the last e with
// offsets[e] <= p. Uniform over the wave.
__device__ __forceinline__ int gemv1c_expert(const GemmArgs &a, int p) {
  const int E = a.w.E;
  const int e = p < E ? a.active[p] : -1;
  const int ec = max(e, 0);
  const int o0 = a.offsets[ec], o1 = a.offsets[ec + 1];
  if ((e >= 0) & (o0 == p) & (o1 == p + 1)) return e;
  if (p >= a.offsets[E]) return -1;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.offsets[mid] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int FMT, int C, int U>
__global__ __launch_bounds__(kGemvCombineThreads, 2) void gemv1c_kernel(GemmArgs a, int L_log2,
                                                                        int blocks_per_wg,
                                                                        const float *topk_w,
                                                                        const int32_t *inv,
                                                                        float *out) {
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr int kWaves = kGemvCombineThreads / 64;
  constexpr int kMaxRows = 8 * U;                 // RW <= 8 rows per wave slot
  __shared__ uint32_t lut[kLut ? kLutWords : 1];
  __shared__ int s_ip[64];                        // inv[j]: routed row of copy j
  __shared__ float s_w[64];
  __shared__ float s_y[64][kMaxRows];             // [(block, routed row)][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int N = a.w.N, E = a.w.E, k = a.k;
  GemvGeom g;
  g.L_log2 = L_log2;
  g.L = 1 << L_log2;
  g.RW = 64 >> L_log2;
  g.li = lane & (g.L - 1);
  g.seg = lane >> L_log2;
  g.wave = 0;
  g.ustride = 1;
  g.half = 0;
  g.KCH = a.w.K >> 5;
  g.rows_per_item = g.RW * U;
  const int G = blocks_per_wg;                    // row blocks of this workgroup (G * k <= 64)
  const int nb0 = (int)blockIdx.x * G;

  int vi = 0;
  float vw = 0.f;
  if (tid < k) {
    vi = inv[tid];
    vw = topk_w[tid];
  }
  if constexpr (kLut) fill_nf4_lut<kGemvCombineThreads>(lut, tid);

  // task q = (row block q / k, routed row q % k). The last workgroup may hold
  // fewer than G row blocks (ceil(N / rows per block) need not be a multiple
  // of G): a task whose block starts at or past N loads nothing (the branch
  // is uniform over the wave) and its rows are never stored. Each wave's
  // first task issues its loads before the workgroup barrier, for the
  // speculated expert active[p]; `have` says the registers hold the right
  // expert's rows.
  uint32_t x[1][C][16];
  GemvRows<U, C> R;
  float v[U][1];
  int q = wave;
  bool have = false;
  if (q < G * k && (nb0 + q / k) * g.rows_per_item < N) {
    const int p = q % k;
    const int e = p < E ? a.active[p] : -1;
    const int ec = max(e, 0);
    gemv_load_x_row<C>(a, g, p, x);
    gemv_load_rows<FMT, U, C, false>(a, g, ec, (nb0 + q / k) * g.rows_per_item, R);
    // both offsets in one round trip (no short-circuit between the loads)
    const int o0 = a.offsets[ec], o1 = a.offsets[ec + 1];
    have = (e >= 0) & (o0 == p) & (o1 == p + 1);
  }
  if (tid < k) {
    s_ip[tid] = vi;
    s_w[tid] = vw;
  }
  __syncthreads();                                // decode table, inv and weights in LDS

  for (; q < G * k; q += kWaves) {
    const int b = q / k, p = q - b * k;
    const int n0 = (nb0 + b) * g.rows_per_item;
    if (n0 >= N) continue;
    if (!have) {
      const int e = gemv1c_expert(a, p);
      if (e < 0) continue;                        // no such row (dropped ids): never combined
      gemv_load_x_row<C>(a, g, p, x);
      gemv_load_rows<FMT, U, C, false>(a, g, e, n0, R);
    }
    have = false;
    gemv_dot<FMT, 1, U, C>(g, lut, lane4, R, x, v);
    if (g.li == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) s_y[q][u * g.RW + g.seg] = v[u][0];
    }
  }
  __syncthreads();
  if (tid < G * g.rows_per_item) {               // the combine's operations, j ascending
    const int b = tid / g.rows_per_item, r = tid - b * g.rows_per_item;
    const int n = (nb0 + b) * g.rows_per_item + r;
    if (n < N) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j)
        if (s_ip[j] >= 0) acc = __builtin_fmaf(s_w[j], s_y[b * k + s_ip[j]][r], acc);
      out[n] = acc;
    }
  }
}

// ===================================================================== MFMA

// M tiles of BM rows over all experts (ceil(count / BM) each), the same
// value in every lane. The grid is sized on the host from an upper bound of
// this count; the real count lets each XCD take an equal share.
template <int BM>
__device__ __forceinline__ int total_m_tiles(const GemmArgs &a, int lane) {
  int total = 0;
  for (int e0 = 0; e0 < a.w.E; e0 += 64) {
    const int ee = e0 + lane;
    int t = 0;
    if (ee < a.w.E) t = (a.offsets[ee + 1] - a.offsets[ee] + BM - 1) / BM;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
    total += t;
  }
  return total;
}

// XOR swizzle of the 8 16-byte K segments of activation row r in LDS. An
// MFMA A-fragment read has lanes 0..31 on 32 consecutive rows at one
// logical segment; with r & 7 alone, rows r and r + 8 land on the same banks
// within the lanes the LDS serves together. Folding r >> 3 in separates them.
__device__ __forceinline__ int a_swizzle(int r) { return (r ^ (r >> 3)) & 7; }

// Tile enumeration of the MFMA kernel: expert by expert (ascending),
// ceil(count / BM) M tiles each, N-tile major within the expert. Returns the
// expert of logical tile `bid` (-1 past the last tile), the first logical
// tile of that expert and its M-tile count. Uniform per wave.
template <int BM>
__device__ __forceinline__ void find_tile(const GemmArgs &a, int bid, int n_tiles_n, int lane,
                                          int &e, int &start, int &tiles) {
  e = -1;
  start = 0;
  tiles = 0;
  int base = 0;
  for (int e0 = 0; e0 < a.w.E && e < 0; e0 += 64) {
    const int ee = e0 + lane;
    int t = 0;
    if (ee < a.w.E) t = (a.offsets[ee + 1] - a.offsets[ee] + BM - 1) / BM;
    int incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d, 64);
      if (lane >= d) incl += u;
    }
    const int lo = (base + incl - t) * n_tiles_n, hi = (base + incl) * n_tiles_n;
    const uint64_t hit = __ballot(t > 0 && bid >= lo && bid < hi);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      e = e0 + src;
      start = __shfl(lo, src, 64);
      tiles = __shfl(t, src, 64);
    }
    base += __shfl(incl, 63, 64);
  }
}

// ======================================== MFMA 16x16x32, full-line weight loads

// The prefill kernel for all three formats. Tile 64 activation rows x 256 weight columns per
// workgroup; wave w owns columns [64w, 64w + 64) as four 16-column tiles and
// all 64 rows as four 16-row tiles, with v_mfma_f32_16x16x32_bf16.
//
// Weights advance in stages of 128 K values (two NF4 blocks = one 64-byte
// line per column). Lane L loads 16 bytes, piece p = L >> 4 of the stage, of
// column L & 15 of a column tile: one load instruction covers 16 whole
// lines, and the data already sits in the B operand's lanes (column L & 15,
// K group L >> 4). Pieces 0-1 are block 0 and pieces 2-3 block 1; two
// v_permlane32_swap per tile exchange dwords 2-3 of the low lanes with dwords
// 0-1 of the high lanes, after which every lane holds two dwords of each
// block: block-local K values 32 (p & 1) + 16 (p >> 1) + 8 j + i for MFMA j
// of the block (i < 8). The activation fragments are read from LDS at the
// same K values, so each block's two MFMAs form a partial that the block's
// absmax scales before accumulation.
//
// Scales are read 8 blocks per column at a time: lane (p, c) holds blocks
// 2p, 2p + 1 of the window for column c, and each block's value reaches the
// 4 lanes of its column through ds_bpermute. NF4_DQ loads the two int8
// values and their second-level scales with the window and forms the float32
// absmax when the window comes into use. MXFP4 holds the four e8m0 bytes of
// the two blocks (two 32-K groups each); each lane takes the byte of its own
// group and passes it to the conversion, which makes a scaled partial
// unnecessary. (Reading the bytes block by block instead, one uncoalesced
// byte load per column tile and block, made the MXFP4 call 27 % slower on the
// gpt-oss shape.) Activation rows are
// staged through LDS per block, double buffered. All global reads are
// buffer loads: a uniform base per expert (or the activation tensor) plus a
// fixed 32-bit lane offset and a uniform step offset; reads past a column's
// last block fall on the next column or past the buffer (zero) and are not
// used. Activation tensors of 4 GiB or more (BIGX) are read with 64-bit
// addresses instead; their rows and blocks are clamped in range either way.
//
// SwiGLU epilogue (GLU): a workgroup covers 128 output columns of H = N / 2;
// wave w's column tiles 0, 1 are gate columns c = 32w + 16t + (0..15) and
// tiles 2, 3 the up columns N/2 + c of the same c, so one lane holds each
// (gate, up) pair when storing bf16(silu(gate) * up).
__device__ __forceinline__ int k16_seg(int p, int j) { return 4 * (p & 1) + 2 * (p >> 1) + j; }

constexpr int kBufferDword3 = 0x00020000;   // raw buffer, 32-bit data format

// Rows of a tile: 4 row tiles of 16 (the layout above); the A staging
// buffer is sized for them.
constexpr int kMfmaRowTiles = 4;
constexpr int kMfmaSegs = 16 * kMfmaRowTiles * 8;   // 16-byte A segments per block

// One workgroup's tile (expert e, weight-column tile nt, routed rows row0 +
// [0, rows_valid)) computed with RT row tiles of 16 (rows_valid <= 16 * RT).
template <int FMT, int RT, bool BIGX, bool GLU, bool GATHER>
__device__ __forceinline__ void mfma16_tile(const GemmArgs &a, uint32_t x_bytes, uint32_t *lut,
                                            uint4 (*As)[kMfmaSegs], int e, int nt, int row0,
                                            int rows_valid) {
  // NF4 and NF4_DQ decode through the table and scale each block's partial;
  // MXFP4 folds its scale into the conversion.
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr bool kDQ = FMT == GNF4_NF4_DQ;
  constexpr bool kMX = FMT == GNF4_MXFP4;
  constexpr int BM = 16 * RT, BN = 256;
  static_assert(RT >= 1 && RT <= kMfmaRowTiles, "16 to 64 rows");
  constexpr int kSegs = BM * 8;                 // 16-byte A segments per block
  constexpr int kALoads = (kSegs + kThreads - 1) / kThreads;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.w.N, K = a.w.K;
  const int nb = GLU ? nt * (BN / 2) + wave * 32  // this wave's first (output) column
                     : nt * BN + wave * 64;
  const int half = a.w.N / 2;
  const int p = lane >> 4, c16 = lane & 15;
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int nkb = K / 64;
  const int nst = (nkb + 1) / 2;

  const int64_t erow = (int64_t)e * N;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w.codes + erow * (K / 2)), (short)0, (int)((uint32_t)N * (uint32_t)(K / 2)),
      kBufferDword3);
  // NF4: float32 absmax [N][K/64]; NF4_DQ: int8 [N][K/64]; MXFP4: e8m0 bytes [N][K/32]
  const uint32_t scale_row = kDQ ? (uint32_t)(K / 64) : kMX ? (uint32_t)(K / 32) : (uint32_t)(K / 16);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const uint8_t *>(a.w.scales) + erow * scale_row), (short)0,
      (int)((uint32_t)N * scale_row), kBufferDword3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.X, (short)0, BIGX ? 0 : (int)x_bytes, kBufferDword3);
  // NF4_DQ second-level scales: one float32 per 256 flat blocks of the tensor
  const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.w.scales2, (short)0,
      kDQ ? (int)(uint32_t)((((int64_t)a.w.E * N * nkb + 255) >> 8) * 4) : 0, kBufferDword3);

  // ---- A staging (per 64-K block): byte offsets of this thread's two
  // 16-byte segments in X, and their LDS slots
  uint32_t xoff[kALoads];
  const uint8_t *xptr[kALoads];
  int sdst[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int idx = min(tid + i * kThreads, kSegs - 1);   // a surplus thread repeats the last slot
    const int r = idx >> 3, sg = idx & 7;
    const int pr = row0 + min(r, rows_valid - 1);
    const int src = GATHER ? a.perm[pr] / a.k : pr;
    if constexpr (BIGX)
      xptr[i] = reinterpret_cast<const uint8_t *>(a.X) + (int64_t)src * (K * 2) + sg * 16;
    else
      xoff[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)sg * 16u;
    sdst[i] = r * 8 + (sg ^ a_swizzle(r));
  }

  // ---- weight columns (ragged N: clamped, never stored). NF4 and NF4_DQ
  // scale offset: blocks 2p, 2p + 1 of an 8-block window (NF4_DQ also keeps
  // the flat index of block 2p for its second-level scale); MXFP4: the 32-K
  // group (p & 1) of a block, the block index coming from the step offset.
  uint32_t coff[4], soff[4];
  int64_t fblk[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const uint32_t col = GLU ? (uint32_t)((ct >> 1) * half + min(nb + (ct & 1) * 16 + c16, half - 1))
                             : (uint32_t)min(nb + ct * 16 + c16, N - 1);
    coff[ct] = col * (uint32_t)(K / 2) + 16u * (uint32_t)p;
    soff[ct] = kDQ ? col * scale_row + 2u * (uint32_t)p
               : kMX ? col * scale_row + 4u * (uint32_t)p : col * scale_row + 8u * (uint32_t)p;
    fblk[ct] = (erow + col) * nkb + 2 * p;
  }

  f32x4_t acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // stage slots, raw codes: stage S in slot S mod kSlots. MXFP4 keeps a
  // third stage in flight (about 3 % faster on the gpt-oss shape); the NF4
  // paths have no registers for it.
  constexpr int kSlots = kMX ? 3 : 2;
  uint4 qs0[4], qs1[4], qs2[4];
  uint4 ar0[kALoads], ar1[kALoads];   // A staging ring (even / odd blocks)
  uint2 sw[4], sn[4];                 // absmax window (current / next): blocks 2p, 2p+1
  uint32_t dn[4];                     // NF4_DQ next window: int8 absmax of blocks 2p, 2p+1
  uint2 tn[4];                        //   and their second-level scales
  uint32_t xw[4], xn[4];              // MXFP4 window (current / next): the e8m0 bytes of
                                      //   blocks 2p, 2p+1 (two 32-K groups each)

#define GNF4_LOAD_STAGE(S, Q)                                                             \
  {                                                                                       \
    const int so_ = 64 * min((S), nst - 1);                                               \
    _Pragma("unroll") for (int ct = 0; ct < 4; ++ct)                                     \
        Q[ct] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, coff[ct], so_, 0)); \
  }
#define GNF4_LOAD_A(KB, DST)                                                              \
  {                                                                                       \
    const int so_ = 128 * min((KB), nkb - 1);                                             \
    _Pragma("unroll") for (int i = 0; i < kALoads; ++i) {                                \
      if constexpr (BIGX)                                                                 \
        DST[i] = *reinterpret_cast<const uint4 *>(xptr[i] + so_);                         \
      else                                                                                \
        DST[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[i], so_, 0)); \
    }                                                                                     \
  }
#define GNF4_STORE_A(SLOT, SRC)                                                           \
  _Pragma("unroll") for (int i = 0; i < kALoads; ++i) As[SLOT][sdst[i]] = SRC[i];
#define GNF4_LOAD_WINDOW(W)                                                               \
  _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                     \
    if constexpr (kDQ) {                                                                  \
      /* two byte loads: a 16-bit load at an odd offset would be aligned down */         \
      dn[ct] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, soff[ct], 8 * (W), 0) |  \
               ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, soff[ct], 8 * (W) + 1, 0) << 8); \
      const int64_t f_ = fblk[ct] + 8 * (W);                                              \
      tn[ct].x = __builtin_amdgcn_raw_buffer_load_b32(rs2, (uint32_t)(f_ >> 8) * 4u, 0, 0); \
      tn[ct].y = __builtin_amdgcn_raw_buffer_load_b32(rs2, (uint32_t)((f_ + 1) >> 8) * 4u, 0, 0); \
    } else if constexpr (kMX) {                                                           \
      /* two 16-bit loads (K / 32 is even, so the offsets are too) */                     \
      xn[ct] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, soff[ct], 16 * (W), 0) | \
               ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, soff[ct], 16 * (W) + 2, 0) << 16); \
    } else {                                                                              \
      sn[ct] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, soff[ct], 32 * (W), 0)); \
    }                                                                                     \
  }
  // The window's absmax divided by the operand scale s (the table holds
  // bf16(s * c)); NF4_DQ forms the float32 absmax first, int8 value times its
  // group's scale
#define GNF4_TAKE_WINDOW()                                                                \
  _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                     \
    float a0_ = 0.f, a1_ = 0.f;                                                           \
    if constexpr (kMX) {                                                                  \
      xw[ct] = xn[ct];                                                                    \
      continue;                                                                           \
    } else if constexpr (kDQ) {                                                           \
      a0_ = (float)(int8_t)(dn[ct] & 0xffu) * __builtin_bit_cast(float, tn[ct].x);        \
      a1_ = (float)(int8_t)((dn[ct] >> 8) & 0xffu) * __builtin_bit_cast(float, tn[ct].y); \
    } else {                                                                              \
      a0_ = __builtin_bit_cast(float, sn[ct].x);                                          \
      a1_ = __builtin_bit_cast(float, sn[ct].y);                                          \
    }                                                                                     \
    sw[ct].x = __builtin_bit_cast(uint32_t, a0_ * kNF4InvScale);                          \
    sw[ct].y = __builtin_bit_cast(uint32_t, a1_ * kNF4InvScale);                          \
  }

  GNF4_LOAD_WINDOW(0);
  GNF4_LOAD_STAGE(0, qs0);
  GNF4_LOAD_A(0, ar0);
  GNF4_LOAD_A(1, ar1);
  GNF4_LOAD_STAGE(1, qs1);
  if constexpr (kSlots == 3) GNF4_LOAD_STAGE(2, qs2);
  if constexpr (kLut) fill_nf4_lut_256(lut, tid);
  GNF4_STORE_A(0, ar0);

  // The two B fragments of block B of column tile CT (dwords x, y for block
  // 0, z, w for block 1 after the swap). MXFP4: the scale SC of the lane's
  // 32-K group is applied by the conversion (exact).
#define GNF4_DECODE(Q, B, CT, FB, SC)                                                     \
  {                                                                                       \
    const uint32_t w0_ = (B) == 0 ? Q[CT].x : Q[CT].z;                                    \
    const uint32_t w1_ = (B) == 0 ? Q[CT].y : Q[CT].w;                                    \
    uint32_t d_[8];                                                                       \
    if constexpr (kLut) {                                                                 \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) d_[i] = lut_read(lut, lut_addr(w0_, lane4, i)); \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) d_[4 + i] = lut_read(lut, lut_addr(w1_, lane4, i)); \
    } else {                                                                              \
      d_[0] = fp4_pair<0>(w0_, SC); d_[1] = fp4_pair<1>(w0_, SC);                         \
      d_[2] = fp4_pair<2>(w0_, SC); d_[3] = fp4_pair<3>(w0_, SC);                         \
      d_[4] = fp4_pair<0>(w1_, SC); d_[5] = fp4_pair<1>(w1_, SC);                         \
      d_[6] = fp4_pair<2>(w1_, SC); d_[7] = fp4_pair<3>(w1_, SC);                         \
    }                                                                                     \
    FB[0] = __builtin_bit_cast(bf16x8_t, make_uint4(d_[0], d_[1], d_[2], d_[3]));         \
    FB[1] = __builtin_bit_cast(bf16x8_t, make_uint4(d_[4], d_[5], d_[6], d_[7]));         \
  }

  // One 64-K block KB = 2 S + B of stage S, codes in Q. AC: this block's A
  // staging registers (refilled with block KB + 2); AN: block KB + 1's.
#define GNF4_BLOCK(S, B, Q, AC, AN)                                                       \
  {                                                                                       \
    const int kb = 2 * (S) + (B);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    __syncthreads(); /* As[kb & 1] holds block kb; As[(kb & 1) ^ 1] is free */            \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    if ((B) == 0) {                                                                       \
      if (((S) & 3) == 0) {                                                               \
        GNF4_TAKE_WINDOW();                                                               \
        GNF4_LOAD_WINDOW(((S) >> 2) + 1);                                                 \
      }                                                                                   \
      _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                 \
        auto r0 = __builtin_amdgcn_permlane32_swap(Q[ct].x, Q[ct].z, false, false);      \
        auto r1 = __builtin_amdgcn_permlane32_swap(Q[ct].y, Q[ct].w, false, false);      \
        Q[ct] = make_uint4(r0[0], r1[0], r0[1], r1[1]);                                   \
      }                                                                                   \
    }                                                                                     \
    /* The block's scale for this lane's column sits in window slot kb & 7, */           \
    /* held by lane group (kb & 7) >> 1 = S & 3. NF4, NF4_DQ: the absmax, */              \
    /* element kb & 1 = B. MXFP4: the e8m0 byte of the lane's own 32-K group */           \
    /* (p & 1), byte 2 B + (p & 1) of the group's dword. */                              \
    float scl[4];                                                                         \
    {                                                                                     \
      const int src = (16 * ((S) & 3) + c16) << 2;                                        \
      _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                 \
        if constexpr (kMX) {                                                              \
          const uint32_t w_ = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)xw[ct]);   \
          scl[ct] = e8m0_to_f32((w_ >> (16 * (B) + 8 * (p & 1))) & 0xffu);                \
        } else {                                                                          \
          scl[ct] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(              \
              src, (int)((B) == 0 ? sw[ct].x : sw[ct].y)));                               \
        }                                                                                 \
      }                                                                                   \
    }                                                                                     \
    GNF4_LOAD_A(kb + 2, AC);                                                              \
    const uint4 *Ab = As[kb & 1];                                                         \
    bf16x8_t af[RT][2];                                                                   \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                  \
      const int r = rt * 16 + c16;                                                        \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) af[rt][j] =                          \
          __builtin_bit_cast(bf16x8_t, Ab[r * 8 + (k16_seg(p, j) ^ a_swizzle(r))]);       \
    }                                                                                     \
    /* column tiles in turn: the decode of tile ct + 1 is issued before tile */           \
    /* ct's MFMAs. NF4: tiles t = ct * 4 + rt, the 4 scale FMAs of tile t - 1 */          \
    /* follow tile t's MFMAs so the VALU work overlaps the MFMA pipe; MXFP4 */            \
    /* accumulates in the MFMAs */                                                        \
    bf16x8_t fb[2][2];                                                                    \
    GNF4_DECODE(Q, B, 0, fb[0], scl[0]);                                                  \
    __builtin_amdgcn_s_setprio(1); /* priority while issuing the MFMAs (about 2 % faster) */ \
    f32x4_t Pp[2];                                                                        \
    _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                   \
      __builtin_amdgcn_sched_barrier(0);                                                  \
      if (ct < 3) GNF4_DECODE(Q, B, ct + 1, fb[(ct + 1) & 1], scl[ct + 1]);              \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                \
        if constexpr (kLut) {                                                             \
          constexpr int kT = RT * 4;                                                      \
          const int t = ct * RT + rt;                                                     \
          const int pr = (t + kT - 1) % RT, pc = ((t + kT - 1) / RT) % 4;                 \
          f32x4_t P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][0], fb[ct & 1][0],    \
                                                              f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0); \
          P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][1], fb[ct & 1][1], P, 0, 0, 0); \
          if (t > 0) {                                                                    \
            _Pragma("unroll") for (int r2 = 0; r2 < 4; ++r2) acc[pr][pc][r2] =           \
                __builtin_fmaf(scl[pc], Pp[(t - 1) & 1][r2], acc[pr][pc][r2]);            \
          }                                                                               \
          Pp[t & 1] = P;                                                                  \
        } else {                                                                          \
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][0], fb[ct & 1][0],  \
                                                                acc[rt][ct], 0, 0, 0);    \
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt][1], fb[ct & 1][1],  \
                                                                acc[rt][ct], 0, 0, 0);    \
        }                                                                                 \
      }                                                                                   \
    }                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    __builtin_amdgcn_s_setprio(0);                                                       \
    /* stage S + kSlots reuses this stage's slot once block 1 is decoded */              \
    if ((B) == 1) GNF4_LOAD_STAGE((S) + kSlots, Q);                                       \
    if constexpr (kLut) {                                                                 \
      _Pragma("unroll") for (int r2 = 0; r2 < 4; ++r2) acc[RT - 1][3][r2] =              \
          __builtin_fmaf(scl[3], Pp[(RT * 4 - 1) & 1][r2], acc[RT - 1][3][r2]);           \
    }                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    GNF4_STORE_A((kb & 1) ^ 1, AN);                                                       \
  }

  // stages in groups of kSlots (stage S in slot S mod kSlots); a trailing
  // odd block ends early
  int S = 0;
  if constexpr (kSlots == 3) {
    for (; S + 2 < nst; S += 3) {
      GNF4_BLOCK(S, 0, qs0, ar0, ar1);
      GNF4_BLOCK(S, 1, qs0, ar1, ar0);
      GNF4_BLOCK(S + 1, 0, qs1, ar0, ar1);
      GNF4_BLOCK(S + 1, 1, qs1, ar1, ar0);
      GNF4_BLOCK(S + 2, 0, qs2, ar0, ar1);
      if (2 * (S + 2) + 1 < nkb) GNF4_BLOCK(S + 2, 1, qs2, ar1, ar0);
    }
    if (S < nst) {
      GNF4_BLOCK(S, 0, qs0, ar0, ar1);
      if (2 * S + 1 < nkb) GNF4_BLOCK(S, 1, qs0, ar1, ar0);
    }
    if (S + 1 < nst) {
      GNF4_BLOCK(S + 1, 0, qs1, ar0, ar1);
      if (2 * (S + 1) + 1 < nkb) GNF4_BLOCK(S + 1, 1, qs1, ar1, ar0);
    }
  } else {
    for (; S + 1 < nst; S += 2) {
      GNF4_BLOCK(S, 0, qs0, ar0, ar1);
      GNF4_BLOCK(S, 1, qs0, ar1, ar0);
      GNF4_BLOCK(S + 1, 0, qs1, ar0, ar1);
      if (2 * (S + 1) + 1 < nkb) GNF4_BLOCK(S + 1, 1, qs1, ar1, ar0);
    }
    if (S < nst) {
      GNF4_BLOCK(S, 0, qs0, ar0, ar1);
      if (2 * S + 1 < nkb) GNF4_BLOCK(S, 1, qs0, ar1, ar0);
    }
  }
#undef GNF4_BLOCK
#undef GNF4_DECODE
#undef GNF4_TAKE_WINDOW
#undef GNF4_LOAD_WINDOW
#undef GNF4_STORE_A
#undef GNF4_LOAD_A
#undef GNF4_LOAD_STAGE

  // ---- store: register r of a 16x16 tile holds row 4 p + r, column c16
  if constexpr (GLU) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int col = nb + ct * 16 + c16;
        if (col >= half) continue;
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const int r = rt * 16 + 4 * p + r2;
          if (r < rows_valid)
            a.H[(int64_t)(row0 + r) * half + col] = swiglu_bf16(acc[rt][ct][r2], acc[rt][ct + 2][r2]);
        }
      }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = nb + ct * 16 + c16;
        if (col >= N) continue;
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) {
          const int r = rt * 16 + 4 * p + r2;
          if (r < rows_valid) a.Y[(int64_t)(row0 + r) * N + col] = acc[rt][ct][r2];
        }
      }
  }
}

// Tiles are enumerated expert by expert with 64-row M tiles; an expert's
// last tile holds count % 64 rows (when not 0), so the tile body is compiled
// for 1 to 4 row tiles of 16 and each workgroup runs the smallest that
// holds its rows: a tile of 20 rows issues the MFMAs, activation loads and
// scale multiplies of 32 rows, not 64 (the B decode is the same). The
// branch is uniform over the workgroup.
template <int FMT, int RT, bool BIGX, bool GLU, bool GATHER>
__global__ __launch_bounds__(kThreads, 2) void mfma16_kernel(GemmArgs a, int n_tiles_n,
                                                             uint32_t x_bytes) {
  static_assert(RT == kMfmaRowTiles, "64-row tiles");
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr int BM = 16 * RT;
  __shared__ uint32_t lut[kLut ? kLutWords : 1];
  __shared__ uint4 As[2][kMfmaSegs];

  const int lane = threadIdx.x & 63;
  // Logical tile id from the hardware workgroup id: workgroups are dealt
  // round-robin over the 8 XCDs, so XCD x (bid & 7) runs bid >> 3 = 0, 1, ...
  // in turn; it takes the x-th eighth of the real tiles, consecutive ids, and
  // its workgroups past that share exit. (An eighth of the grid's upper bound
  // instead left the last XCD most of the empty tail: about 10 % longer.)
  const int total = total_m_tiles<BM>(a, lane) * n_tiles_n;
  const int per = (total + 7) >> 3;
  const int j = (int)(blockIdx.x >> 3);
  const int bid = (int)(blockIdx.x & 7) * per + j;
  if (j >= per || bid >= total) return;
  int e, start, tiles;
  find_tile<BM>(a, bid, n_tiles_n, lane, e, start, tiles);
  if (e < 0) return;
  const int local = bid - start;
  const int nt = local / tiles, mt = local - nt * tiles;
  const int seg_start = a.offsets[e];
  const int count = a.offsets[e + 1] - seg_start;
  const int row0 = seg_start + mt * BM;
  const int rows_valid = min(BM, count - mt * BM);
  const int rt = (rows_valid + 15) >> 4;
  if (rt >= 4)
    mfma16_tile<FMT, 4, BIGX, GLU, GATHER>(a, x_bytes, lut, As, e, nt, row0, rows_valid);
  else if (rt == 3)
    mfma16_tile<FMT, 3, BIGX, GLU, GATHER>(a, x_bytes, lut, As, e, nt, row0, rows_valid);
  else if (rt == 2)
    mfma16_tile<FMT, 2, BIGX, GLU, GATHER>(a, x_bytes, lut, As, e, nt, row0, rows_valid);
  else
    mfma16_tile<FMT, 1, BIGX, GLU, GATHER>(a, x_bytes, lut, As, e, nt, row0, rows_valid);
}

// ============================================================ host launch

// Rows per wave slot U compiled for each (tokens per group MT, chunks per lane
// C): register budget U * C * 5 + MT * C * 16 per lane.
struct GemvVariant {
  int MT, C, nu;
  int U[3];
};
static const GemvVariant kGemvVariants[] = {
    {1, 1, 3, {4, 8, 16}}, {1, 2, 2, {4, 8, 0}}, {1, 3, 2, {2, 4, 0}}, {1, 4, 1, {2, 0, 0}},
    {2, 1, 2, {2, 4, 0}},  {2, 2, 1, {2, 0, 0}}, {2, 3, 2, {1, 2, 0}},
    {4, 1, 1, {2, 0, 0}},  {4, 2, 2, {1, 2, 0}}, {8, 1, 1, {2, 0, 0}},
};

// NF4_DQ rebuilds each absmax from two loads and needs more registers: its
// rows per wave slot stop at U * C <= 8.
static bool gemv_fits(int fmt, int C, int U) { return fmt != GNF4_NF4_DQ || C * U <= 8; }

static const GemvVariant *gemv_variant(int MT, int C) {
  for (const auto &v : kGemvVariants)
    if (v.MT == MT && v.C == C) return &v;
  return nullptr;
}

// Output columns of a call: N, or N / 2 with the SwiGLU epilogue.
static int out_cols(const GemmArgs &a) { return a.H ? a.w.N / 2 : a.w.N; }

// One token, gathered input: the persistent kernel, one workgroup per CU (or
// as many as are resident at once).
template <int FMT, int C, int U, bool GLU, int ROUTE>
static hipError_t gemv1w_go(const GemmArgs &a, int L_log2, int max_slots, hipStream_t s) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv1w_kernel<FMT, C, U, GLU, ROUTE>,
                                                     kGemvWaveThreads, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  const int rows_per_item = (64 >> L_log2) * (GLU ? U / 2 : U);
  const int items = (out_cols(a) + rows_per_item - 1) / rows_per_item;
  const int64_t waves = (int64_t)max_slots * items;
  const int64_t grid = std::min<int64_t>((int64_t)per_cu * device_cu_count(),
                                         (waves + kGemvWaveThreads / 64 - 1) / (kGemvWaveThreads / 64));
  hipLaunchKernelGGL((gemv1w_kernel<FMT, C, U, GLU, ROUTE>), dim3((unsigned)grid),
                     dim3(kGemvWaveThreads), 0, s, a, L_log2, items, max_slots);
  return hipGetLastError();
}

template <int FMT, int MT, int C, int U, bool GLU>
static hipError_t gemv_go(const GemmArgs &a, int L_log2, int max_slots, hipStream_t s) {
  const int L = 1 << L_log2;
  const int rows_per_item = 4 * (64 / L) * (GLU ? U / 2 : U);
  const int items = (out_cols(a) + rows_per_item - 1) / rows_per_item;
  const int64_t grid = (int64_t)max_slots * items;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (MT == 1) {
    // one token in routed order (a gathered one takes gemv1w_kernel)
    if (a.T == 1) {
      hipLaunchKernelGGL((gemv1_kernel<FMT, C, U, GLU>), dim3((unsigned)grid), dim3(kThreads), 0,
                         s, a, L_log2, items);
      return hipGetLastError();
    }
  }
  // Two or more tokens take one token per group only when K needs 4 chunks
  // per lane (K > 6144).
  if constexpr (MT == 1 && C < 4) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((gemv_kernel<FMT, MT, C, U, GLU>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, a, L_log2, items);
    return hipGetLastError();
  }
}

// The SwiGLU epilogue pairs slot u with u + U/2, so it takes even U only.
#define GNF4_GEMV_CASE(mt, c, u)                                                       \
  if constexpr (FMT != GNF4_NF4_DQ || c * u <= 8)                                      \
    if (MT == mt && C == c && U == u) {                                                \
      if (!a.H) return gemv_go<FMT, mt, c, u, false>(a, L_log2, max_slots, s);         \
      if constexpr (u % 2 == 0) return gemv_go<FMT, mt, c, u, true>(a, L_log2, max_slots, s); \
      return hipErrorInvalidValue;                                                     \
    }

template <int FMT>
static hipError_t gemv_dispatch(const GemmArgs &a, int MT, int C, int U, int L_log2, int max_slots,
                                hipStream_t s) {
  GNF4_GEMV_CASE(1, 1, 4) GNF4_GEMV_CASE(1, 1, 8) GNF4_GEMV_CASE(1, 1, 16)
  GNF4_GEMV_CASE(1, 2, 4) GNF4_GEMV_CASE(1, 2, 8) GNF4_GEMV_CASE(1, 3, 2) GNF4_GEMV_CASE(1, 3, 4)
  GNF4_GEMV_CASE(1, 4, 2)
  GNF4_GEMV_CASE(2, 1, 2) GNF4_GEMV_CASE(2, 1, 4) GNF4_GEMV_CASE(2, 2, 2) GNF4_GEMV_CASE(2, 3, 1)
  GNF4_GEMV_CASE(2, 3, 2)
  GNF4_GEMV_CASE(4, 1, 2) GNF4_GEMV_CASE(4, 2, 1) GNF4_GEMV_CASE(4, 2, 2) GNF4_GEMV_CASE(8, 1, 2)
  return hipErrorInvalidValue;
}
#undef GNF4_GEMV_CASE

// Chunks-per-lane values compiled for each token count. One token covers
// K <= 64 lanes * 4 chunks * 32 = 8192.
static int gemv_c_options(int MT, int *out) {
  int n = 0;
  for (const auto &v : kGemvVariants)
    if (v.MT == MT) out[n++] = v.C;
  return n;
}

// Lanes per row L (8..64) and chunks per lane C covering K/32 chunks with the
// least idle lanes, larger L on ties. Returns false if K is too large.
bool gemv_shape(int K, int MT, int *L_log2, int *C) {
  const int kch = K / 32;
  int opts[8];
  const int nopt = gemv_c_options(MT, opts);
  double best = -1.0;
  for (int lg = 6; lg >= 3; --lg) {
    for (int i = 0; i < nopt; ++i) {
      const int c = opts[i];
      const int cap = (1 << lg) * c;
      if (cap < kch) continue;
      const double util = (double)kch / cap;
      if (util > best + 1e-9) {
        best = util;
        *L_log2 = lg;
        *C = c;
      }
      break;  // larger C only adds idle lanes for this L
    }
  }
  return best > 0.0;
}

int gemv_tokens(int T) { return T >= 5 ? 8 : (T >= 3 ? 4 : (T >= 2 ? 2 : 1)); }

// Rows per wave slot: the smallest compiled U (that fits the format's
// registers, and is even for the SwiGLU epilogue) whose grid fits the
// resident workgroups (two per CU), else the largest that fits; 0 if none
// does. cols: output columns (N, or N / 2 with the epilogue).
static int gemv_pick_u(const GemvVariant &v, int fmt, int cols, int L_log2, int max_slots,
                       bool glu) {
  const int64_t target = 2LL * device_cu_count();
  int last = 0;
  for (int i = 0; i < v.nu; ++i) {
    if (!gemv_fits(fmt, v.C, v.U[i])) break;
    if (glu && v.U[i] % 2) continue;
    last = v.U[i];
    const int per = 4 * (64 >> L_log2) * (glu ? v.U[i] / 2 : v.U[i]);
    const int64_t items = (int64_t)max_slots * ((cols + per - 1) / per);
    if (items <= target) return v.U[i];
  }
  return last;
}

// Rows per wave slot of the one-token gathered kernel for C chunks per lane
// (measured fastest on the workload shapes, and free of register spills).
// The SwiGLU epilogue needs an even U (slot u pairs with u + U/2). C = 2 (K
// of 4096, the Qwen3-235B-shaped gate_up): U = 3 gives each wave exactly two
// items at 8 routed experts x 3072 rows, 4 % faster than U = 4 (1.5 items
// per wave, the second round of half the waves in the tail); U = 2, 6 and 8
// and issuing both items' loads before either's products were slower.
template <int FMT, bool GLU, int ROUTE>
static hipError_t gemv1w_dispatch(const GemmArgs &a, int C, int L_log2, int max_slots,
                                  hipStream_t s) {
  switch (C) {
    case 1: return gemv1w_go<FMT, 1, 4, GLU, ROUTE>(a, L_log2, max_slots, s);
    case 2:
      if constexpr (GLU) return gemv1w_go<FMT, 2, 4, GLU, ROUTE>(a, L_log2, max_slots, s);
      else return gemv1w_go<FMT, 2, 3, GLU, ROUTE>(a, L_log2, max_slots, s);
    case 3: return gemv1w_go<FMT, 3, 2, GLU, ROUTE>(a, L_log2, max_slots, s);
    case 4:
      if constexpr (FMT != GNF4_MXFP4 && !GLU) return gemv1w_go<FMT, 4, 1, GLU, ROUTE>(a, L_log2, max_slots, s);
      else return gemv1w_go<FMT, 4, 2, GLU, ROUTE>(a, L_log2, max_slots, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, bool GLU>
static hipError_t gemv1w_route(const GemmArgs &a, int C, int L_log2, int max_slots, hipStream_t s) {
  if (a.logits) return gemv1w_dispatch<FMT, GLU, 2>(a, C, L_log2, max_slots, s);
  if (a.ids) return gemv1w_dispatch<FMT, GLU, 1>(a, C, L_log2, max_slots, s);
  return gemv1w_dispatch<FMT, GLU, 0>(a, C, L_log2, max_slots, s);
}

template <int FMT>
static hipError_t gemv1w_any(const GemmArgs &a, int C, int L_log2, int max_slots, hipStream_t s) {
  return a.H ? gemv1w_route<FMT, true>(a, C, L_log2, max_slots, s)
             : gemv1w_route<FMT, false>(a, C, L_log2, max_slots, s);
}

template <int FMT, int C, int U>
static hipError_t gemv1c_go(const GemmArgs &a, int L_log2, const float *topk_w,
                            const int32_t *inv, float *out, hipStream_t s) {
  const int rows_per_item = (64 >> L_log2) * U;
  const int items = (a.w.N + rows_per_item - 1) / rows_per_item;
  const int G = a.k < 8 ? 8 / a.k : 1;            // row blocks per workgroup
  const int wgs = (items + G - 1) / G;
  hipLaunchKernelGGL((gemv1c_kernel<FMT, C, U>), dim3((unsigned)wgs), dim3(kGemvCombineThreads), 0,
                     s, a, L_log2, G, topk_w, inv, out);
  return hipGetLastError();
}

// Rows per wave slot: the smallest U (1, 2, 4) whose workgroup count is at
// most two per CU (fewer, larger workgroups amortize the table fill and the
// routing read; more keep every CU busy).
template <int FMT, int C>
static hipError_t gemv1c_pick(const GemmArgs &a, int L_log2, const float *topk_w,
                              const int32_t *inv, float *out, hipStream_t s) {
  // The smallest U whose workgroup count is at most two per CU and either
  // fits the CUs or is a whole multiple of them: a count in between leaves
  // some CUs one workgroup more than the rest (measured: the gpt-oss-shaped
  // down projection, 360 workgroups at U = 2, takes 14 % longer per decode
  // step than 180 at U = 4).
  const int G = a.k < 8 ? 8 / a.k : 1;
  const int64_t cus = device_cu_count(), target = 2 * cus;
  int U = 4;
  for (int u = 1; u <= 4; u <<= 1) {
    const int64_t rows = (int64_t)(64 >> L_log2) * u * G;
    const int64_t wgs = (a.w.N + rows - 1) / rows;
    if (wgs <= target && (wgs <= cus || wgs % cus == 0)) {
      U = u;
      break;
    }
  }
  if (U == 1) return gemv1c_go<FMT, C, 1>(a, L_log2, topk_w, inv, out, s);
  if (U == 2) return gemv1c_go<FMT, C, 2>(a, L_log2, topk_w, inv, out, s);
  return gemv1c_go<FMT, C, 4>(a, L_log2, topk_w, inv, out, s);
}

template <int FMT>
static hipError_t gemv1c_dispatch(const GemmArgs &a, int C, int L_log2, const float *topk_w,
                                  const int32_t *inv, float *out, hipStream_t s) {
  switch (C) {
    case 1: return gemv1c_pick<FMT, 1>(a, L_log2, topk_w, inv, out, s);
    case 2: return gemv1c_pick<FMT, 2>(a, L_log2, topk_w, inv, out, s);
    case 3: return gemv1c_pick<FMT, 3>(a, L_log2, topk_w, inv, out, s);
    case 4: return gemv1c_pick<FMT, 4>(a, L_log2, topk_w, inv, out, s);
    default: return hipErrorInvalidValue;
  }
}

bool gemv_combine_fits(const GemmArgs &a) {
  int L_log2 = 6, C = 1;
  return a.T == 1 && !a.gather && a.k <= 64 && gemv_shape(a.w.K, 1, &L_log2, &C);
}

hipError_t launch_gemv_combine(const GemmArgs &a, const float *topk_w, const int32_t *inv,
                               float *out, hipStream_t s) {
  int L_log2 = 6, C = 1;
  if (!gemv_combine_fits(a) || !gemv_shape(a.w.K, 1, &L_log2, &C)) return hipErrorInvalidValue;
  switch (a.w.format) {
    case GNF4_NF4: return gemv1c_dispatch<GNF4_NF4>(a, C, L_log2, topk_w, inv, out, s);
    case GNF4_NF4_DQ: return gemv1c_dispatch<GNF4_NF4_DQ>(a, C, L_log2, topk_w, inv, out, s);
    default: return gemv1c_dispatch<GNF4_MXFP4>(a, C, L_log2, topk_w, inv, out, s);
  }
}

hipError_t launch_gemv(const GemmArgs &a, hipStream_t s) {
  if (a.T == 1 && a.gather) {
    int L_log2 = 6, C = 1;
    if (!gemv_shape(a.w.K, 1, &L_log2, &C)) return hipErrorInvalidValue;
    const int max_slots = std::min<int>(a.w.E, a.k);
    switch (a.w.format) {
      case GNF4_NF4:
        return gemv1w_any<GNF4_NF4>(a, C, L_log2, max_slots, s);
      case GNF4_NF4_DQ:
        return gemv1w_any<GNF4_NF4_DQ>(a, C, L_log2, max_slots, s);
      default:
        return gemv1w_any<GNF4_MXFP4>(a, C, L_log2, max_slots, s);
    }
  }
  int MT = gemv_tokens(a.T);
  int L_log2 = 6, C = 1;
  while (!gemv_shape(a.w.K, MT, &L_log2, &C)) {
    if (MT == 1) return hipErrorInvalidValue;
    MT >>= 1;
  }
  const GemvVariant *v = gemv_variant(MT, C);
  if (!v) return hipErrorInvalidValue;
  const int max_slots = std::min<int>(a.w.E, a.T * a.k);
  const int U = gemv_pick_u(*v, a.w.format, out_cols(a), L_log2, max_slots, a.H != nullptr);
  if (U == 0) return hipErrorInvalidValue;
  switch (a.w.format) {
    case GNF4_NF4: return gemv_dispatch<GNF4_NF4>(a, MT, C, U, L_log2, max_slots, s);
    case GNF4_NF4_DQ: return gemv_dispatch<GNF4_NF4_DQ>(a, MT, C, U, L_log2, max_slots, s);
    default: return gemv_dispatch<GNF4_MXFP4>(a, MT, C, U, L_log2, max_slots, s);
  }
}

// Bytes of the activation tensor the GEMM reads (gathered: T rows, else T*k).
static int64_t x_bytes(const GemmArgs &a) {
  return (a.gather ? (int64_t)a.T : (int64_t)a.T * a.k) * a.w.K * 2;
}

template <int FMT, int RT, bool BIGX, bool GLU, bool GATHER>
static hipError_t mfma16_go(const GemmArgs &a, hipStream_t s) {
  constexpr int BM = 16 * RT, BN = GLU ? 128 : 256;    // output columns per tile
  const int rows = a.T * a.k;
  const int n_tiles_n = (out_cols(a) + BN - 1) / BN;
  const int64_t m_tiles = (rows + BM - 1) / BM + std::min<int>(a.w.E, rows);
  int64_t grid = m_tiles * n_tiles_n;
  grid = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((mfma16_kernel<FMT, RT, BIGX, GLU, GATHER>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     a, n_tiles_n, BIGX ? 0u : (uint32_t)x_bytes(a));
  return hipGetLastError();
}

// The activation gather is a compile-time choice: the gathered first
// projection and the routed-order second one are distinct kernels (also in
// a profile's per-kernel rows).
template <int FMT, bool GATHER>
static hipError_t mfma_pick_g(const GemmArgs &a, hipStream_t s) {
  // 32-bit buffer offsets reach activation tensors below 4 GiB
  const bool big = x_bytes(a) >= ((int64_t)1 << 32);
  if (a.H)
    return big ? mfma16_go<FMT, 4, true, true, GATHER>(a, s) : mfma16_go<FMT, 4, false, true, GATHER>(a, s);
  return big ? mfma16_go<FMT, 4, true, false, GATHER>(a, s) : mfma16_go<FMT, 4, false, false, GATHER>(a, s);
}

template <int FMT>
static hipError_t mfma_pick(const GemmArgs &a, hipStream_t s) {
  return a.gather ? mfma_pick_g<FMT, true>(a, s) : mfma_pick_g<FMT, false>(a, s);
}

hipError_t launch_mfma(const GemmArgs &a, hipStream_t s) {
  switch (a.w.format) {
    case GNF4_NF4: return mfma_pick<GNF4_NF4>(a, s);
    case GNF4_NF4_DQ: return mfma_pick<GNF4_NF4_DQ>(a, s);
    default: return mfma_pick<GNF4_MXFP4>(a, s);
  }
}

}  // namespace gnf4
