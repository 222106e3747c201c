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
//  * mfma_kernel (prefill; a dense contraction per expert). Each workgroup
//    owns a BM x BN tile of one expert (tiles enumerated expert by expert,
//    N-tile major, then M-tile; the enumeration is XCD-aware so tiles that
//    share weight columns run on one XCD's L2). Gathered activation rows are
//    staged in LDS (double buffered, XOR-swizzled 16-byte segments); each
//    wave decodes its weight columns straight into MFMA B fragments and runs
//    v_mfma_f32_32x32x16_bf16. NF4: the bf16 codebook enters the MFMA and
//    the float32 absmax scales each 64-value partial before accumulation.
//    MXFP4: the e8m0 scale is folded into the (exact) bf16 decode.
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

// Block scale of 32-value chunk `ch` of weight row `row` (flat e*N + n).
template <int FMT>
__device__ __forceinline__ float chunk_scale(const Weights &w, int64_t row, int ch) {
  if constexpr (FMT == GNF4_MXFP4) {
    return e8m0_to_f32(reinterpret_cast<const uint8_t *>(w.scales)[row * (w.K / 32) + ch]);
  } else if constexpr (FMT == GNF4_NF4) {
    return reinterpret_cast<const float *>(w.scales)[row * (w.K / 64) + (ch >> 1)];
  } else {
    const int64_t blk = row * (w.K / 64) + (ch >> 1);
    return (float)reinterpret_cast<const int8_t *>(w.scales)[blk] * w.scales2[blk >> 8];
  }
}

// ===================================================================== GEMV

// Rows in flight per wave-row-slot: about 128 bytes of code loads per lane
// outstanding for one token, fewer as the token slices take registers.
template <int MT, int C>
struct GemvUnroll {
  static constexpr int raw = (MT >= 4 ? 4 : 8) / (C * (MT >= 2 ? 2 : 1));
  static constexpr int value = raw < 1 ? 1 : raw;
};

template <int FMT, int MT, int C>
__global__ __launch_bounds__(kThreads, 2) void gemv_kernel(GemmArgs a, int L_log2,
                                                           int items_per_expert, int max_slots) {
  constexpr int U = GemvUnroll<MT, C>::value;
  constexpr bool kLut = FMT != GNF4_MXFP4;
  __shared__ uint32_t lut[kLut ? kLutWords : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t lane4 = (uint32_t)lane << 2;
  const int L = 1 << L_log2;
  const int RW = 64 >> L_log2;                  // rows per wave slot
  const int li = lane & (L - 1), seg = lane >> L_log2;
  const int N = a.w.N, K = a.w.K, KCH = K >> 5;
  const int rows_per_item = 4 * RW * U;
  const int64_t nitems = (int64_t)max_slots * items_per_expert;
  bool lut_ready = !kLut;

  uint4 q[U][C];
  float sc[U][C];
  // All code and scale loads of one item (rows n0 + (u*4 + wave)*RW + seg).
#define GNF4_GEMV_LOAD_ROWS()                                                             \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                        \
    const int r = n0 + (u * 4 + wave) * RW + seg;                                         \
    const int64_t row = (int64_t)e * N + r;                                               \
    _Pragma("unroll") for (int c = 0; c < C; ++c) {                                      \
      const int ch = li + c * L;                                                          \
      if (r < N && ch < KCH) {                                                            \
        q[u][c] = *reinterpret_cast<const uint4 *>(a.w.codes + row * (K / 2) + ch * 16);  \
        sc[u][c] = chunk_scale<FMT>(a.w, row, ch);                                        \
      } else {                                                                            \
        q[u][c] = make_uint4(0u, 0u, 0u, 0u);                                             \
        sc[u][c] = 0.f;                                                                   \
      }                                                                                   \
    }                                                                                     \
  }

  for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int slot = (int)(item / items_per_expert);
    const int ib = (int)(item - (int64_t)slot * items_per_expert);
    // The only load the weight stream waits for: the expert of this slot
    // (-1 past the active count).
    const int e = a.active[slot];
    if (e < 0) continue;
    const int n0 = ib * rows_per_item;
    GNF4_GEMV_LOAD_ROWS();
    const int p0 = a.offsets[e];
    const int m = a.offsets[e + 1] - p0;

    for (int tg = 0; tg < m; tg += MT) {
      if (tg > 0) GNF4_GEMV_LOAD_ROWS();   // more tokens than MT: stream the rows again

      // Token slices in registers: x[t][c][i] holds the bf16 pair for K values
      // 32*ch + 2i, +1 of chunk ch = li + c*L.
      uint32_t x[MT][C][16];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const bool has = tg + t < m;
        const int p = p0 + tg + t;
        const int src = has ? (a.gather ? a.perm[p] / a.k : p) : 0;
        const uint16_t *xrow = a.X + (int64_t)src * K;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int ch = li + c * L;
          if (has && ch < KCH) {
            const uint4 *s4 = reinterpret_cast<const uint4 *>(xrow + ch * 32);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint4 v = s4[j];
              x[t][c][4 * j + 0] = v.x;
              x[t][c][4 * j + 1] = v.y;
              x[t][c][4 * j + 2] = v.z;
              x[t][c][4 * j + 3] = v.w;
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[t][c][i] = 0u;
          }
        }
      }

      // The decode table is built once per workgroup, while the first loads
      // are in flight.
      if constexpr (kLut) {
        if (!lut_ready) {
          fill_nf4_lut_256(lut, tid);
          __syncthreads();
          lut_ready = true;
        }
      }

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
          const uint32_t qw[4] = {q[u][c].x, q[u][c].y, q[u][c].z, q[u][c].w};
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
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[t] = __builtin_fmaf(sc[u][c], part[t], acc[t]);
        }
        const int r = n0 + (u * 4 + wave) * RW + seg;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const float v = group_sum(acc[t], L);
          if (li == 0 && r < N && tg + t < m) a.Y[(int64_t)(p0 + tg + t) * N + r] = v;
        }
      }
    }
  }
#undef GNF4_GEMV_LOAD_ROWS
}

// ===================================================================== MFMA

// Logical tile id from the hardware workgroup id: consecutive logical ids on
// the same XCD (workgroups are dealt round-robin over the 8 XCDs). The grid
// is a multiple of 8, so the map is a bijection.
__device__ __forceinline__ int xcd_remap(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Tile: BM = 32*TM activation rows x BN = 4*32*TN weight rows (output
// columns). The 4 waves split N: wave w owns columns [w*32*TN, (w+1)*32*TN)
// and all BM rows, so every weight column is decoded by exactly one wave.
// K advances 64 values (one NF4 block, two MXFP4 blocks) per step; A and B
// are prefetched two steps ahead (register staging, A double-buffered in LDS).
template <int FMT, int TM, int TN>
__global__ __launch_bounds__(kThreads, 2) void mfma_kernel(GemmArgs a, int n_tiles_n) {
  constexpr int BM = 32 * TM;
  constexpr int BN = 4 * 32 * TN;
  constexpr bool kLut = FMT != GNF4_MXFP4;
  constexpr int kSegs = BM * 8;              // 16-byte A segments per K step
  constexpr int kALoads = kSegs / kThreads;  // per thread
  static_assert(kSegs % kThreads == 0, "BM must be a multiple of 32");
  __shared__ uint32_t lut[kLut ? kLutWords : 1];
  __shared__ uint4 As[2][kSegs];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.w.E, N = a.w.N, K = a.w.K;

  // ---- which tile: walk experts, ceil(count/BM) M-tiles x n_tiles_n N-tiles each
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  int e = -1, start = 0, tiles = 0;
  {
    int base = 0;
    for (int e0 = 0; e0 < E && e < 0; e0 += 64) {
      const int ee = e0 + lane;
      int t = 0;
      if (ee < E) t = (a.offsets[ee + 1] - a.offsets[ee] + BM - 1) / BM;
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
  if (e < 0) return;                        // past the last tile (uniform per workgroup)
  const int local = bid - start;
  const int nt = local / tiles, mt = local - nt * tiles;
  const int seg_start = a.offsets[e];
  const int count = a.offsets[e + 1] - seg_start;
  const int row0 = seg_start + mt * BM;
  const int rows_valid = min(BM, count - mt * BM);
  const int n0 = nt * BN + wave * 32 * TN;  // this wave's first column
  const uint32_t lane4 = (uint32_t)lane << 2;

  // ---- A (gathered activation rows): per-thread sources, fixed over K
  const uint16_t *xsrc[kALoads];
  int sdst[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int idx = tid + i * kThreads;
    const int r = idx >> 3, sg = idx & 7;
    const int p = row0 + min(r, rows_valid - 1);          // padding rows repeat a valid row
    const int src = a.gather ? a.perm[p] / a.k : p;
    xsrc[i] = a.X + (int64_t)src * K + sg * 8;
    sdst[i] = r * 8 + (sg ^ (r & 7));
  }

  // ---- B: lane (g, nn) holds K values [32g, 32g + 32) of column nn of each N sub-tile
  const int g = lane >> 5, nn = lane & 31;
  const uint8_t *bsrc[TN];
  int64_t brow[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int n = min(n0 + tn * 32 + nn, N - 1);           // ragged N: clamp, never stored
    brow[tn] = (int64_t)e * N + n;
    bsrc[tn] = a.w.codes + brow[tn] * (K / 2) + g * 16;
  }

  const int nkb = K / 64;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  // Two-slot rings (slot 0 holds even steps, slot 1 odd steps), as separate
  // named arrays so that they stay in registers.
  static_assert(kALoads == 2, "A staging holds two 16-byte segments per thread (BM = 64)");
  uint4 areg0_0, areg0_1, areg1_0, areg1_1;
  uint4 bq0[TN], bq1[TN];
  uint2 bs0[TN], bs1[TN];   // raw block-scale bits (x; NF4_DQ: y = scale2)

#define GNF4_LOAD_A(KB, DST)                                                              \
  DST##_0 = *reinterpret_cast<const uint4 *>(xsrc[0] + (KB) * 64);                       \
  DST##_1 = *reinterpret_cast<const uint4 *>(xsrc[1] + (KB) * 64);
#define GNF4_LOAD_B(KB, BQ)                                                               \
  _Pragma("unroll") for (int tn = 0; tn < TN; ++tn)                                      \
      BQ[tn] = *reinterpret_cast<const uint4 *>(bsrc[tn] + (KB) * 32);
#define GNF4_LOAD_S(KB, BS)                                                               \
  _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) {                                    \
    /* raw scale bits only: converting here would wait for the load */                  \
    if constexpr (FMT == GNF4_MXFP4) {                                                    \
      BS[tn].x = reinterpret_cast<const uint8_t *>(a.w.scales)[brow[tn] * (K / 32) + 2 * (KB) + g]; \
    } else if constexpr (FMT == GNF4_NF4) {                                               \
      BS[tn].x = reinterpret_cast<const uint32_t *>(a.w.scales)[brow[tn] * (K / 64) + (KB)]; \
    } else {                                                                              \
      const int64_t blk = brow[tn] * (K / 64) + (KB);                                     \
      BS[tn].x = (uint32_t)(int32_t)reinterpret_cast<const int8_t *>(a.w.scales)[blk];    \
      BS[tn].y = __builtin_bit_cast(uint32_t, a.w.scales2[blk >> 8]);                     \
    }                                                                                     \
  }

  GNF4_LOAD_B(0, bq0);
  GNF4_LOAD_S(0, bs0);
  GNF4_LOAD_A(0, areg0);
  GNF4_LOAD_B(min(1, nkb - 1), bq1);
  GNF4_LOAD_S(min(1, nkb - 1), bs1);
  GNF4_LOAD_A(min(1, nkb - 1), areg1);
  if constexpr (kLut) fill_nf4_lut_256(lut, tid);
  As[0][sdst[0]] = areg0_0; As[0][sdst[1]] = areg0_1;

  // One K step. S: ring slot of this step; AC/BQ/BS: this step's ring
  // entries (refilled with step KB + 2); AN: the next step's A staging.
#define GNF4_MFMA_STEP(KB, S, AC, AN, BQ, BS)                                             \
  {                                                                                       \
    /* no instruction crosses a step boundary: a decode hoisted into the */              \
    /* previous step would wait on loads issued only one step earlier */                 \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    __syncthreads(); /* As[S] holds step KB; As[S ^ 1] is no longer read */               \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    bf16x8_t bf[TN][4];                                                                   \
    float scl[TN];                                                                        \
    _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) {                                  \
      const uint32_t qw[4] = {BQ[tn].x, BQ[tn].y, BQ[tn].z, BQ[tn].w};                    \
      if constexpr (FMT == GNF4_MXFP4) scl[tn] = e8m0_to_f32(BS[tn].x);                   \
      else if constexpr (FMT == GNF4_NF4) scl[tn] = __builtin_bit_cast(float, BS[tn].x);  \
      else scl[tn] = (float)(int32_t)BS[tn].x * __builtin_bit_cast(float, BS[tn].y);      \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                    \
        uint32_t d[4];                                                                    \
        if constexpr (kLut) {                                                             \
          _Pragma("unroll") for (int i = 0; i < 4; ++i) d[i] =                           \
              lut_read(lut, lut_addr(qw[j], lane4, i));                                   \
        } else {                                                                          \
          d[0] = fp4_pair<0>(qw[j], scl[tn]);                                             \
          d[1] = fp4_pair<1>(qw[j], scl[tn]);                                             \
          d[2] = fp4_pair<2>(qw[j], scl[tn]);                                             \
          d[3] = fp4_pair<3>(qw[j], scl[tn]);                                             \
        }                                                                                 \
        bf[tn][j] = __builtin_bit_cast(bf16x8_t, make_uint4(d[0], d[1], d[2], d[3]));     \
      }                                                                                   \
    }                                                                                     \
    {                                                                                     \
      const int kn = min((KB) + 2, nkb - 1);                                              \
      GNF4_LOAD_B(kn, BQ);                                                                \
      GNF4_LOAD_A(kn, AC);                                                                \
    }                                                                                     \
    const uint4 *Ab = As[S];                                                              \
    bf16x8_t af[TM][4];                                                                   \
    _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) {                                  \
      const int r = tm * 32 + nn;                                                         \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) af[tm][j] =                          \
          __builtin_bit_cast(bf16x8_t, Ab[r * 8 + ((4 * g + j) ^ (r & 7))]);              \
    }                                                                                     \
    if constexpr (kLut) {                                                                 \
      /* tiles in order t = tn * TM + tm; partials alternate between two register */     \
      /* sets so the scale FMAs of one tile overlap the MFMAs of the next */             \
      f32x16_t Pp[2];                                                                     \
      _Pragma("unroll") for (int t = 0; t < TM * TN; ++t) {                              \
        const int tm = t % TM, tn = t / TM;                                               \
        f32x16_t P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm][0], bf[tn][0],        \
                                                             f32x16_t{}, 0, 0, 0);        \
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm][1], bf[tn][1], P, 0, 0, 0);    \
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm][2], bf[tn][2], P, 0, 0, 0);    \
        P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm][3], bf[tn][3], P, 0, 0, 0);    \
        if (t > 0) {                                                                      \
          const int pm = (t - 1) % TM, pn = (t - 1) / TM;                                 \
          _Pragma("unroll") for (int r2 = 0; r2 < 16; ++r2) acc[pm][pn][r2] =            \
              __builtin_fmaf(scl[pn], Pp[(t - 1) & 1][r2], acc[pm][pn][r2]);              \
        }                                                                                 \
        Pp[t & 1] = P;                                                                    \
      }                                                                                   \
      {                                                                                   \
        constexpr int t = TM * TN - 1;                                                    \
        const int pm = t % TM, pn = t / TM;                                               \
        _Pragma("unroll") for (int r2 = 0; r2 < 16; ++r2) acc[pm][pn][r2] =              \
            __builtin_fmaf(scl[pn], Pp[t & 1][r2], acc[pm][pn][r2]);                      \
      }                                                                                   \
    } else {                                                                              \
      _Pragma("unroll") for (int tn = 0; tn < TN; ++tn)                                  \
      _Pragma("unroll") for (int tm = 0; tm < TM; ++tm)                                  \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[tm][tn] =                        \
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm][j], bf[tn][j], acc[tm][tn], 0, 0, 0); \
    }                                                                                     \
    As[(S) ^ 1][sdst[0]] = AN##_0; As[(S) ^ 1][sdst[1]] = AN##_1;                          \
    /* the scales of step KB + 2 are loaded after this step's last use of BS, so */      \
    /* the loop-carried register is refilled in place */                                  \
    GNF4_LOAD_S(min((KB) + 2, nkb - 1), BS);                                              \
  }

  int kb = 0;
  for (; kb + 1 < nkb; kb += 2) {
    GNF4_MFMA_STEP(kb, 0, areg0, areg1, bq0, bs0);
    GNF4_MFMA_STEP(kb + 1, 1, areg1, areg0, bq1, bs1);
  }
  if (kb < nkb) GNF4_MFMA_STEP(kb, 0, areg0, areg1, bq0, bs0);
#undef GNF4_MFMA_STEP
#undef GNF4_LOAD_A
#undef GNF4_LOAD_B
#undef GNF4_LOAD_S

  // ---- store: C fragment register r = 4i + j holds row 8i + 4g + j, column nn
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int col = n0 + tn * 32 + nn;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = tm * 32 + 8 * i + 4 * g + j;
          if (r < rows_valid) a.Y[(int64_t)(row0 + r) * N + col] = acc[tm][tn][4 * i + j];
        }
    }
}

// ============================================================ host launch

static int floor_log2(int v) {
  int r = 0;
  while ((2 << r) <= v) ++r;
  return r;
}

template <int FMT, int MT, int C>
static hipError_t gemv_go(const GemmArgs &a, int L_log2, int max_slots, hipStream_t s) {
  const int L = 1 << L_log2;
  const int rows_per_item = 4 * (64 / L) * GemvUnroll<MT, C>::value;
  const int items = (a.w.N + rows_per_item - 1) / rows_per_item;
  const int64_t upper = (int64_t)max_slots * items;
  const int64_t grid = std::min<int64_t>(upper, 2LL * device_cu_count());
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemv_kernel<FMT, MT, C>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     L_log2, items, max_slots);
  return hipGetLastError();
}

template <int FMT, int MT>
static hipError_t gemv_pick_c(const GemmArgs &a, int C, int L_log2, int max_slots, hipStream_t s) {
  switch (C) {
    case 1: return gemv_go<FMT, MT, 1>(a, L_log2, max_slots, s);
    case 2: if constexpr (MT <= 4) return gemv_go<FMT, MT, 2>(a, L_log2, max_slots, s); break;
    case 3: if constexpr (MT <= 2) return gemv_go<FMT, MT, 3>(a, L_log2, max_slots, s); break;
    case 4: if constexpr (MT <= 1) return gemv_go<FMT, MT, 4>(a, L_log2, max_slots, s); break;
  }
  return hipErrorInvalidValue;
}

template <int FMT>
static hipError_t gemv_pick_mt(const GemmArgs &a, int MT, int C, int L_log2, int max_slots,
                               hipStream_t s) {
  switch (MT) {
    case 1: return gemv_pick_c<FMT, 1>(a, C, L_log2, max_slots, s);
    case 2: return gemv_pick_c<FMT, 2>(a, C, L_log2, max_slots, s);
    case 4: return gemv_pick_c<FMT, 4>(a, C, L_log2, max_slots, s);
    default: return gemv_pick_c<FMT, 8>(a, C, L_log2, max_slots, s);
  }
}

// Chunks-per-lane values compiled for each token count (x registers:
// MT * C * 16 <= 96 per lane, so that no variant spills). One token covers
// K <= 64 lanes * 4 chunks * 32 = 8192.
static int gemv_c_options(int MT, int *out) {
  static const int c1[] = {1, 2, 3, 4}, c2[] = {1, 2, 3}, c4[] = {1, 2}, c8[] = {1};
  const int *src = MT == 1 ? c1 : MT == 2 ? c2 : MT == 4 ? c4 : c8;
  const int n = MT == 1 ? 4 : MT == 2 ? 3 : MT == 4 ? 2 : 1;
  for (int i = 0; i < n; ++i) out[i] = src[i];
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

hipError_t launch_gemv(const GemmArgs &a, hipStream_t s) {
  int MT = gemv_tokens(a.T);
  int L_log2 = 6, C = 1;
  while (!gemv_shape(a.w.K, MT, &L_log2, &C)) {
    if (MT == 1) return hipErrorInvalidValue;
    MT >>= 1;
  }
  const int max_slots = std::min<int>(a.w.E, a.T * a.k);
  switch (a.w.format) {
    case GNF4_NF4: return gemv_pick_mt<GNF4_NF4>(a, MT, C, L_log2, max_slots, s);
    case GNF4_NF4_DQ: return gemv_pick_mt<GNF4_NF4_DQ>(a, MT, C, L_log2, max_slots, s);
    default: return gemv_pick_mt<GNF4_MXFP4>(a, MT, C, L_log2, max_slots, s);
  }
}

template <int FMT, int TM, int TN>
static hipError_t mfma_go(const GemmArgs &a, hipStream_t s) {
  constexpr int BM = 32 * TM, BN = 4 * 32 * TN;
  const int rows = a.T * a.k;
  const int n_tiles_n = (a.w.N + BN - 1) / BN;
  const int64_t m_tiles = (rows + BM - 1) / BM + std::min<int>(a.w.E, rows);
  int64_t grid = m_tiles * n_tiles_n;
  grid = (grid + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((mfma_kernel<FMT, TM, TN>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                     n_tiles_n);
  return hipGetLastError();
}

template <int FMT>
static hipError_t mfma_pick(const GemmArgs &a, hipStream_t s) {
  return mfma_go<FMT, 2, 2>(a, s);
}

hipError_t launch_mfma(const GemmArgs &a, hipStream_t s) {
  switch (a.w.format) {
    case GNF4_NF4: return mfma_pick<GNF4_NF4>(a, s);
    case GNF4_NF4_DQ: return mfma_pick<GNF4_NF4_DQ>(a, s);
    default: return mfma_pick<GNF4_MXFP4>(a, s);
  }
}

}  // namespace gnf4
