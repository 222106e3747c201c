// gnf4_grouped_gemm_dx: the input gradient of the grouped GEMM through the
// frozen packed expert weights, in one launch for all active experts, reading
// the 4-bit codes as stored (Jordan Anderson, jordananderson-pages.pages.dev,
// section "grouped-nf4-gemm & experts-4bit", fourth bullet: the kernel is
// differentiable, fine-tuning computes on the packed weights rather than
// unpacking them in the backward pass, and the backward is a single launch).
//
// For expert e and each routed row p of its segment,
//
//     dA[p, :] = dY[p, :] @ W'[e]        dY bf16 [rows, N], W'[e] [N, K]
//
// contracts over the N output features of the forward call. The packed
// codes are contiguous along K, the output dimension here, so the MFMA B
// operand (8 consecutive contraction values of one output column per lane)
// needs values from 8 different weight rows: the transposed access of the
// forward kernel's.
//
// mfma_dx_kernel. A workgroup owns 16 RT rows of one expert's segment and
// 256 output columns; wave w takes columns [64 w, 64 w + 64), which is one
// NF4 block of every weight row (two MXFP4 blocks). The contraction advances
// 32 weight rows per step. Lane (c, g) = (lane & 15, lane >> 4) reads the two
// code bytes of columns 4c .. 4c+3 of the wave's slice in rows 8g .. 8g+7 of
// the step and decodes them into the B fragments of four MFMA tiles: tile t
// stands for the output columns 4c + t (c = 0..15), so a lane's four tiles
// cover four adjacent columns and its accumulators store as 16-byte runs.
//
// The absmax (NF4, NF4_DQ) varies along the contraction, one value per
// weight row, so it cannot scale a partial sum as in the forward kernel: each
// weight is formed as the float32 product w = c[q] * absmax (the dequantized
// value exactly) and enters the MFMA as bf16 hi + lo, hi = bf16(w) and
// lo = bf16(w - hi), two MFMAs per tile; what is left out is below 2^-16 of
// |w|. MXFP4 weights e2m1 * 2^(s-127) are exact in bf16 and take one MFMA.
// NF4 bytes decode through an LDS table of float32 codebook pairs (one copy
// per lane of a half wave, so each lane reads its own banks); MXFP4 through
// v_cvt_scalef32_pk_f32_fp4.
//
// The gradient rows dY of the tile are staged in LDS per step (double
// buffered, XOR-swizzled 16-byte chunks) and shared by the four waves. Rows
// past the segment are clamped (their outputs are not stored); contraction
// rows past N enter as zero on both sides.
//
// Tiles are enumerated expert by expert, K tile major, then row tile, so
// the row tiles that read the same weight columns are neighbours; the
// kernel counts the tiles that exist and deals them to the 8 XCDs in
// contiguous runs, so tiles that share weight columns and gradient rows run
// on one XCD's L2 and no XCD is left idle by the host's upper bound.
#include <algorithm>

#include "common.h"

namespace gnf4 {

constexpr int kDxThreads = 256;
constexpr int kDxPairCopies = 32;                  // table copies: lanes 0..31 read their own
constexpr int kDxPairWords = 256 * kDxPairCopies * 2;

// float32 codebook value of code q, selected among compile-time constants.
__device__ __forceinline__ uint32_t nf4_f32_bits(uint32_t q) {
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) v = (q == (uint32_t)i) ? kNF4Bits[i] : v;
  return v;
}

// Table entry b (an NF4 byte), copy j: the float32 pair (c[b >> 4], c[b & 15]),
// the value of element 2i (high nibble) first, at byte offset b * 256 + j * 8.
// Thread t writes float2 slots t + 256 i (i < 32): entry (t + 256 i) / 32.
__device__ __forceinline__ void fill_dx_table(float *tab, int tid) {
#pragma unroll 4
  for (int i = 0; i < 256 * kDxPairCopies / kDxThreads; ++i) {
    const uint32_t slot = (uint32_t)tid + kDxThreads * i, b = slot / kDxPairCopies;
    tab[2 * slot] = __builtin_bit_cast(float, nf4_f32_bits(b >> 4));
    tab[2 * slot + 1] = __builtin_bit_cast(float, nf4_f32_bits(b & 15u));
  }
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Tile of logical id `logical` (see the file comment). Every lane of the
// wave returns the same values; e = -1 when the id is past the last tile.
template <int BM>
__device__ __forceinline__ void dx_find_tile(const int32_t *offsets, int E, int n_tiles_k,
                                             int logical, int lane, int &e, int &start,
                                             int &mtiles) {
  e = -1;
  start = 0;
  mtiles = 0;
  int base = 0;
  for (int e0 = 0; e0 < E && e < 0; e0 += 64) {
    const int ee = e0 + lane;
    int t = 0;
    if (ee < E) t = (offsets[ee + 1] - offsets[ee] + BM - 1) / BM;
    int incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(incl, d, 64);
      if (lane >= d) incl += u;
    }
    const int lo = (base + incl - t) * n_tiles_k, hi = (base + incl) * n_tiles_k;
    const uint64_t hit = __ballot(t > 0 && logical >= lo && logical < hi);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      e = e0 + src;
      start = __shfl(lo, src, 64);
      mtiles = __shfl(t, src, 64);
    }
    base += __shfl(incl, 63, 64);
  }
}

template <int BM>
__device__ __forceinline__ int dx_total_tiles(const int32_t *offsets, int E, int n_tiles_k,
                                              int lane) {
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int ee = e0 + lane;
    int t = 0;
    if (ee < E) t = (offsets[ee + 1] - offsets[ee] + BM - 1) / BM;
    total += wave_sum_i(t);
  }
  return total * n_tiles_k;
}

// Swizzled position of 16-byte chunk q (8 contraction values) of staged row r.
__device__ __forceinline__ int dy_chunk(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

__device__ __forceinline__ uint32_t pack_bf16_pair(float lo_half, float hi_half) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo_half, hi_half};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16 hi + lo split of two float32 weights of one column in rows n, n+1:
// hi = RNE bf16 of each, lo = RNE bf16 of the (exact) float32 remainder.
__device__ __forceinline__ void split_pair(float w0, float w1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16_pair(w0, w1);
  const float h0 = __builtin_bit_cast(float, hi << 16);
  const float h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = pack_bf16_pair(w0 - h0, w1 - h1);
}

template <int FMT, int RT>
__global__ __launch_bounds__(kDxThreads, 2) void mfma_dx_kernel(DxArgs a, int n_tiles_k) {
  constexpr bool kNF = FMT != GNF4_MXFP4;
  constexpr bool kDQ = FMT == GNF4_NF4_DQ;
  constexpr int BM = 16 * RT;
  constexpr int kChunks = BM * 4;                 // 16-byte dY chunks per step
  constexpr int kChunkLoads = (kChunks + kDxThreads - 1) / kDxThreads;
  __shared__ float tab[kNF ? kDxPairWords : 1];
  __shared__ uint4 Ds[2][kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.w.N, K = a.w.K, E = a.w.E;

  // logical tile id: contiguous runs of the real tile count per XCD
  const int total = dx_total_tiles<BM>(a.offsets, E, n_tiles_k, lane);
  const int per = (total + 7) >> 3;
  const int bid = blockIdx.x, j = bid >> 3;
  const int logical = (bid & 7) * per + j;
  if (j >= per || logical >= total) return;
  int e, start, mtiles;
  dx_find_tile<BM>(a.offsets, E, n_tiles_k, logical, lane, e, start, mtiles);
  if (e < 0) return;
  const int local = logical - start;
  const int kt = local / mtiles, mt = local - kt * mtiles;
  const int seg0 = a.offsets[e];
  const int count = a.offsets[e + 1] - seg0;
  const int row0 = mt * BM;                       // first row of the tile within the segment

  if constexpr (kNF) fill_dx_table(tab, tid);

  const int c = lane & 15, g = lane >> 4;
  const int colbase = kt * 256 + wave * 64;
  const int mycol = colbase + 4 * c;              // this lane's 4 output columns
  const bool col_ok = mycol < K;
  const int ldcol = col_ok ? mycol : 0;           // clamped for loads
  const int64_t half_k = K >> 1;
  const uint8_t *codes_e = a.w.codes + (int64_t)e * N * half_k + (ldcol >> 1);
  const int nkb = K >> 6, ngrp = K >> 5;
  const int kb = ldcol >> 6, grp = ldcol >> 5;
  const int64_t row_e = (int64_t)e * N;           // flat weight row of this expert's row 0

  // gradient rows: chunk loads of this thread for the step starting at n0
  auto load_dy = [&](int n0, uint4 (&v)[kChunkLoads]) {
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const int ch = tid + kDxThreads * i;
      v[i] = make_uint4(0, 0, 0, 0);
      if (ch < kChunks) {
        const int r = ch >> 2, q = ch & 3;
        const int p = seg0 + min(row0 + r, count - 1);
        const int n = n0 + 8 * q;
        if (n < N) v[i] = *reinterpret_cast<const uint4 *>(a.dY + (int64_t)p * N + n);
      }
    }
  };
  auto store_dy = [&](int buf, const uint4 (&v)[kChunkLoads]) {
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const int ch = tid + kDxThreads * i;
      if (ch < kChunks) Ds[buf][dy_chunk(ch >> 2, ch & 3)] = v[i];
    }
  };
  // weight rows n0 + 8g + i (i < 8): two code bytes and the row's scale
  uint32_t code[8];
  float scl[8];
  int8_t q8[8];
  float s2[8];
  uint32_t sb[8];
  auto load_w = [&](int n0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + 8 * g + i;
      const int nn = n < N ? n : N - 1;
      code[i] = *reinterpret_cast<const uint16_t *>(codes_e + (int64_t)nn * half_k);
      const int64_t fr = row_e + nn;              // flat weight row
      if constexpr (FMT == GNF4_NF4) {
        scl[i] = static_cast<const float *>(a.w.scales)[fr * nkb + kb];
      } else if constexpr (kDQ) {
        const int64_t blk = fr * nkb + kb;
        q8[i] = static_cast<const int8_t *>(a.w.scales)[blk];
        s2[i] = a.w.scales2[blk >> 8];
      } else {
        sb[i] = static_cast<const uint8_t *>(a.w.scales)[fr * ngrp + grp];
      }
    }
  };

  f32x4_t acc[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[r][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nsteps = (N + 31) >> 5;
  {
    uint4 v[kChunkLoads];
    load_dy(0, v);
    store_dy(0, v);
  }
  load_w(0);
  __syncthreads();

  const uint32_t lane8 = (uint32_t)(lane & 31) * 8u;
  for (int s = 0; s < nsteps; ++s) {
    const int n0 = s * 32;
    // this step's weights from registers, then the next step's loads
    uint32_t cw[8];
    float aw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cw[i] = code[i];
      float av;
      if constexpr (FMT == GNF4_NF4) av = scl[i];
      else if constexpr (kDQ) av = (float)q8[i] * s2[i];
      else av = e8m0_to_f32(sb[i]);
      aw[i] = (n0 + 8 * g + i < N) ? av : 0.0f;   // rows past N contribute zero
    }
    uint4 dyv[kChunkLoads];
    const bool more = s + 1 < nsteps;
    if (more) {
      load_dy(n0 + 32, dyv);
      load_w(n0 + 32);
    }

    // B fragments: tile t, rows 8g .. 8g+7 of column 4c + t, as bf16 pairs
    uint32_t bhi[4][4], blo[4][4];
    float w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (kNF) {
        const float2 p0 = *reinterpret_cast<const float2 *>(
            reinterpret_cast<const char *>(tab) + __builtin_amdgcn_perm(cw[i], lane8, 0x0c0c0400u));
        const float2 p1 = *reinterpret_cast<const float2 *>(
            reinterpret_cast<const char *>(tab) + __builtin_amdgcn_perm(cw[i], lane8, 0x0c0c0500u));
        w[i][0] = p0.x * aw[i];
        w[i][1] = p0.y * aw[i];
        w[i][2] = p1.x * aw[i];
        w[i][3] = p1.y * aw[i];
      } else {
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], aw[i], 0);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[i], aw[i], 1);
        w[i][0] = v0[0];
        w[i][1] = v0[1];
        w[i][2] = v1[0];
        w[i][3] = v1[1];
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if constexpr (kNF) split_pair(w[2 * h][t], w[2 * h + 1][t], bhi[t][h], blo[t][h]);
        else bhi[t][h] = pack_bf16_pair(w[2 * h][t], w[2 * h + 1][t]);
      }

    const int buf = s & 1;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint4 av = Ds[buf][dy_chunk(16 * r + c, g)];
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(bhi[t]));
        acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[r][t], 0, 0, 0);
        if constexpr (kNF) {
          const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(blo[t]));
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[r][t], 0, 0, 0);
        }
      }
    }
    if (more) store_dy(buf ^ 1, dyv);
    __syncthreads();
  }

  // lane (c, g) holds rows 4g + i of each 16-row tile, columns 4c + t
  if (!col_ok) return;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = row0 + 16 * r + 4 * g + i;
      if (lr < count) {
        const float4 o = make_float4(acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]);
        *reinterpret_cast<float4 *>(a.dA + (int64_t)(seg0 + lr) * K + mycol) = o;
      }
    }
}

template <int FMT, int RT>
static hipError_t dx_go(const DxArgs &a, hipStream_t s) {
  constexpr int BM = 16 * RT;
  const int rows = a.rows;
  const int n_tiles_k = (a.w.K + 255) / 256;
  const int64_t m_tiles = (rows + BM - 1) / BM + std::min<int>(a.w.E, rows);
  const int64_t bound = m_tiles * n_tiles_k;
  const int64_t grid = (bound + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((mfma_dx_kernel<FMT, RT>), dim3((unsigned)grid), dim3(kDxThreads), 0, s, a,
                     n_tiles_k);
  return hipGetLastError();
}

// Row tile from the mean rows per active expert (a host-side estimate: the
// routing stays on the device).
template <int FMT>
static hipError_t dx_pick(const DxArgs &a, hipStream_t s) {
  const int64_t experts = std::min<int64_t>(a.w.E, a.rows);
  const int64_t mean = experts > 0 ? (a.rows + experts - 1) / experts : 0;
  if (mean <= 16) return dx_go<FMT, 1>(a, s);
  if (mean <= 32) return dx_go<FMT, 2>(a, s);
  if (mean <= 64) return dx_go<FMT, 4>(a, s);
  return dx_go<FMT, 8>(a, s);
}

hipError_t launch_gemm_dx(const DxArgs &a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  switch (a.w.format) {
    case GNF4_NF4: return dx_pick<GNF4_NF4>(a, s);
    case GNF4_NF4_DQ: return dx_pick<GNF4_NF4_DQ>(a, s);
    default: return dx_pick<GNF4_MXFP4>(a, s);
  }
}

}  // namespace gnf4
