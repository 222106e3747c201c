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
#include <type_traits>

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
// Thread t writes float2 slots t + 256 i (i < 32), i.e. entry b = t / 32 + 8 i
// copy t % 32: its high nibble is i / 2 (a constant of the unrolled loop) and
// its low nibble t / 32 + 8 (i & 1), one of two values per thread.
__device__ __forceinline__ void fill_dx_table(float *tab, int tid) {
  const uint32_t t5 = (uint32_t)tid >> 5;
  const float lo0 = __builtin_bit_cast(float, nf4_f32_bits(t5));
  const float lo1 = __builtin_bit_cast(float, nf4_f32_bits(t5 + 8u));
#pragma unroll
  for (int i = 0; i < 256 * kDxPairCopies / kDxThreads; ++i) {
    const uint32_t slot = (uint32_t)tid + kDxThreads * i;
    *reinterpret_cast<float2 *>(tab + 2 * slot) =
        make_float2(__builtin_bit_cast(float, kNF4Bits[i >> 1]), (i & 1) ? lo1 : lo0);
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

// One halving step of a cross-lane reduction: the lane keeps half of its
// first 2 CNT values (the upper half when lane & d), adds the partner's copy
// of that half (lane ^ d) and leaves the sums in v[0 .. CNT).
template <int CNT>
__device__ __forceinline__ void halve(float *v, int d, int lane) {
  const bool upper = (lane & d) != 0;
#pragma unroll
  for (int i = 0; i < CNT; ++i) {
    const float send = upper ? v[i] : v[i + CNT];
    const float keep = upper ? v[i + CNT] : v[i];
    v[i] = keep + __shfl_xor(send, d, 64);
  }
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

constexpr int kDxBufferDword3 = 0x00020000;   // raw buffer, 32-bit data format

template <int FMT, int RT, int CT>
__global__ __launch_bounds__(kDxThreads, 2) void mfma_dx_kernel(DxArgs a, int n_tiles_k) {
  constexpr bool kNF = FMT != GNF4_MXFP4;
  constexpr bool kDQ = FMT == GNF4_NF4_DQ;
  constexpr int BM = 16 * RT;
  static_assert(CT == 2 || CT == 4, "2 or 4 column tiles per wave");
  constexpr int BN = 64 * CT;                     // columns per workgroup (16 CT per wave)
  constexpr int kChunks = BM * 4;                 // 16-byte dY chunks per step
  constexpr int kChunkLoads = (kChunks + kDxThreads - 1) / kDxThreads;
  __shared__ float tab[kNF ? kDxPairWords : 1];
  __shared__ uint4 Ds[2][kChunks];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar offsets
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
  const int colbase = kt * BN + wave * 16 * CT;
  const int mycol = colbase + CT * c;             // this lane's CT output columns
  const bool col_ok = mycol < K;
  const uint32_t ldcol = col_ok ? (uint32_t)mycol : 0u;   // clamped for loads
  const uint32_t half_k = (uint32_t)K >> 1, nkb = (uint32_t)K >> 6, ngrp = (uint32_t)K >> 5;
  const uint32_t kb = ldcol >> 6, grp = ldcol >> 5;
  // bytes per weight row of the scales: float32 absmax, int8 q8, e8m0 byte
  const uint32_t scale_row = FMT == GNF4_NF4 ? nkb * 4u : kDQ ? nkb : ngrp;
  const uint32_t scale_col = FMT == GNF4_NF4 ? kb * 4u : kDQ ? kb : grp;
  const int64_t erow = (int64_t)e * N;            // flat weight row of this expert's row 0

  // buffer views: the expert's codes and scales, the tensor's second-level
  // scales, the segment's gradient rows; every access below stays in range
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w.codes + erow * half_k), (short)0, (int)((uint32_t)N * half_k), kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const uint8_t *>(a.w.scales) + erow * scale_row), (short)0,
      (int)((uint32_t)N * scale_row), kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.w.scales2, (short)0,
      kDQ ? (int)(uint32_t)((((int64_t)E * N * nkb + 255) >> 8) * 4) : 0, kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.dY + (int64_t)seg0 * N), (short)0, (int)((uint32_t)count * (uint32_t)N * 2u),
      kDxBufferDword3);

  // this lane's weight rows 8g + i of a step: code bytes at coff + row * half_k
  const uint32_t coff = (uint32_t)(8 * g) * half_k + (ldcol >> 1);
  const uint32_t soff = (uint32_t)(8 * g) * scale_row + scale_col;
  // this thread's gradient chunks: row r (clamped to the segment), chunk q
  uint32_t dyoff[kChunkLoads];
  int dyq[kChunkLoads];
#pragma unroll
  for (int i = 0; i < kChunkLoads; ++i) {
    const int ch = tid + kDxThreads * i;
    const int r = ch >> 2;
    dyq[i] = ch & 3;
    dyoff[i] = (uint32_t)min(row0 + r, count - 1) * (uint32_t)N * 2u + (uint32_t)dyq[i] * 16u;
  }

  // Main loop: pairs of full 32-row steps, every load unconditional and in
  // range (the prefetch step index is clamped with scalar arithmetic); the
  // rest (an odd full step, a partial last step) runs after it without
  // prefetch, each lane clamping its rows to N - 1 and zeroing rows past N.
  const int nfull = N >> 5;
  const int npair = nfull >> 1;
  uint32_t cw[2][8], sv[2][8];
  float s2v[2][8];
  uint4 dreg[2][kChunkLoads];

  // weights of step s into register set S; `clamp`: rows of a step that may
  // reach past N are clamped per lane (else step s must be full)
  auto issue_w = [&](auto SET, int s, bool clamp) {
    constexpr int S = decltype(SET)::value;
    const uint32_t n0 = (uint32_t)s * 32u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t vc = coff, vs = soff, so_c = (n0 + i) * half_k, so_s = (n0 + i) * scale_row;
      uint32_t row = n0 + 8 * g + i;
      if (clamp) {
        row = min(row, (uint32_t)N - 1u);
        vc = row * half_k + (ldcol >> 1);
        vs = row * scale_row + scale_col;
        so_c = 0;
        so_s = 0;
      }
      if constexpr (CT == 4) cw[S][i] = __builtin_amdgcn_raw_buffer_load_b16(rc, vc, so_c, 0);
      else cw[S][i] = __builtin_amdgcn_raw_buffer_load_b8(rc, vc, so_c, 0);
      if constexpr (FMT == GNF4_NF4) {
        sv[S][i] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs, so_s, 0);
      } else {
        sv[S][i] = __builtin_amdgcn_raw_buffer_load_b8(rs, vs, so_s, 0);
      }
      if constexpr (kDQ) {
        const int64_t blk = (erow + row) * nkb + kb;
        s2v[S][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rs2, (uint32_t)(blk >> 8) * 4u, 0, 0));
      }
    }
  };
  // gradient rows of full step s into register set S (threads without a
  // chunk load a duplicate of a valid one and do not store it)
  auto issue_dy = [&](auto SET, int s) {
    constexpr int S = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i)
      dreg[S][i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, dyoff[i], (uint32_t)s * 64u, 0));
  };
  auto store_dy = [&](auto SET, int buf) {
    constexpr int S = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const int ch = tid + kDxThreads * i;
      if (ch < kChunks) Ds[buf][dy_chunk(ch >> 2, dyq[i])] = dreg[S][i];
    }
  };

  f32x4_t acc[RT][CT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[r][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const uint32_t lane8 = (uint32_t)(lane & 31) * 8u;
  // B fragments of register set S for the step starting at n0, then the
  // MFMAs against LDS buffer `buf`
  auto compute = [&](auto SET, int n0, int buf) {
    constexpr int S = decltype(SET)::value;
    float aw[8];
    uint32_t cwv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cwv[i] = cw[S][i];
      if constexpr (FMT == GNF4_NF4) aw[i] = __builtin_bit_cast(float, sv[S][i]);
      else if constexpr (kDQ) aw[i] = (float)(int8_t)sv[S][i] * s2v[S][i];
      else aw[i] = e8m0_to_f32(sv[S][i]);
    }
    if (n0 + 32 > N) {                            // rows past N contribute zero
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (n0 + 8 * g + i >= N) aw[i] = 0.0f;
    }
    uint32_t bhi[CT][4], blo[CT][4];
    {
      float w[8][CT];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (kNF) {
          const float2 p0 = *reinterpret_cast<const float2 *>(
              reinterpret_cast<const char *>(tab) + __builtin_amdgcn_perm(cwv[i], lane8, 0x0c0c0400u));
          w[i][0] = p0.x * aw[i];
          w[i][1] = p0.y * aw[i];
          if constexpr (CT == 4) {
            const float2 p1 = *reinterpret_cast<const float2 *>(
                reinterpret_cast<const char *>(tab) + __builtin_amdgcn_perm(cwv[i], lane8, 0x0c0c0500u));
            w[i][2] = p1.x * aw[i];
            w[i][3] = p1.y * aw[i];
          }
        } else {
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cwv[i], aw[i], 0);
          w[i][0] = v0[0];
          w[i][1] = v0[1];
          if constexpr (CT == 4) {
            const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cwv[i], aw[i], 1);
            w[i][2] = v1[0];
            w[i][3] = v1[1];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if constexpr (kNF) split_pair(w[2 * h][t], w[2 * h + 1][t], bhi[t][h], blo[t][h]);
          else bhi[t][h] = pack_bf16_pair(w[2 * h][t], w[2 * h + 1][t]);
        }
    }
    // all hi products, then all lo products: 4 RT independent MFMAs separate
    // the two that update one accumulator
    return [&, bhi, blo, buf]() {
      bf16x8_t af[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) af[r] = __builtin_bit_cast(bf16x8_t, Ds[buf][dy_chunk(16 * r + c, g)]);
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(bhi[t]));
#pragma unroll
        for (int r = 0; r < RT; ++r)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bh, acc[r][t], 0, 0, 0);
      }
      if constexpr (kNF) {
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(blo[t]));
#pragma unroll
          for (int r = 0; r < RT; ++r)
            acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bl, acc[r][t], 0, 0, 0);
        }
      }
    };
  };

  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  if (npair > 0) {
    issue_dy(Set0{}, 0);
    issue_w(Set0{}, 0, false);
    issue_dy(Set1{}, 1);
    issue_w(Set1{}, 1, false);
    store_dy(Set0{}, 0);
    __syncthreads();
    const int last = 2 * npair - 1;               // last step of the main loop
    for (int s = 0; s < 2 * npair; s += 2) {
      // step s: set 0, LDS buffer 0; its registers are reloaded for s + 2
      {
        auto mma = compute(Set0{}, s * 32, 0);
        issue_w(Set0{}, min(s + 2, last), false);
        issue_dy(Set0{}, min(s + 2, last));
        mma();
        store_dy(Set1{}, 1);                      // step s + 1's rows
        __syncthreads();
      }
      // step s + 1: set 1, LDS buffer 1; reloaded for s + 3
      {
        auto mma = compute(Set1{}, s * 32 + 32, 1);
        issue_w(Set1{}, min(s + 3, last), false);
        issue_dy(Set1{}, min(s + 3, last));
        mma();
        store_dy(Set0{}, 0);                      // step s + 2's rows (unused after the last)
        __syncthreads();
      }
    }
  }
  // the rest: at most one full step and one partial step
  for (int s = 2 * npair; s < (N + 31) >> 5; ++s) {
    const int n0 = s * 32;
    issue_w(Set0{}, s, true);
#pragma unroll
    for (int i = 0; i < kChunkLoads; ++i) {
      const int ch = tid + kDxThreads * i;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ch < kChunks && n0 + 8 * dyq[i] < N)
        v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, dyoff[i], (uint32_t)n0 * 2u, 0));
      if (ch < kChunks) Ds[0][dy_chunk(ch >> 2, dyq[i])] = v;
    }
    __syncthreads();
    auto mma = compute(Set0{}, n0, 0);
    mma();
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
        float *dst = a.dA + (int64_t)(seg0 + lr) * K + mycol;
        if constexpr (CT == 4)
          *reinterpret_cast<float4 *>(dst) = make_float4(acc[r][0][i], acc[r][1][i], acc[r][2][i], acc[r][3][i]);
        else
          *reinterpret_cast<float2 *>(dst) = make_float2(acc[r][0][i], acc[r][1][i]);
      }
    }
}

// ================================================ few rows per expert

constexpr int kGemvDxMaxRows = 64;   // routed rows (T*k) up to which the GEMV path is used

// gemv_dx_kernel: the few-row path. One workgroup of 8 waves per item
// (expert e, up to MT routed rows of its segment, 32 * LPR output columns).
// LPR lanes share a weight row: lane l reads the 16 code bytes of chunk
// l % LPR of the item (32 columns) in row RPG * R + l / LPR, RPG = 64 / LPR,
// for the row groups R = w, w + 8, ... of wave w, so one 128-bit load covers
// RPG rows with LPR lanes on consecutive bytes of each. The lane also reads
// the row's scale and dY[p][n] of its MT rows p, and accumulates
// s * c[q] in float32 with s = dY[p][n] * absmax (exact codebook values, no
// bf16 rounding of the weights; MXFP4 decodes exactly with its e8m0 scale).
// Rows advance in batches of U per lane, two batches in flight: every load
// of the main loop is unconditional and in range; the remaining groups
// (including a partial last one) run after it with each lane's row clamped
// to N - 1 and its contribution zeroed. Each wave reduces over the RPG lanes
// of each chunk by halving exchanges; the 8 waves' sums meet in LDS, added
// in wave order.
constexpr int kDxGemvThreads = 512;

template <int FMT, int MT, int LPR>
__global__ __launch_bounds__(kDxGemvThreads, MT == 1 ? 4 : 2) void gemv_dx_kernel(DxArgs a) {
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  constexpr bool kNF = FMT != GNF4_MXFP4;
  constexpr bool kDQ = FMT == GNF4_NF4_DQ;
  constexpr int kWaves = kDxGemvThreads / 64;
  constexpr int U = MT == 1 ? 2 : (MT >= 4 ? 2 : 4);   // rows per lane per batch
  constexpr int RPG = 64 / LPR;                   // weight rows per load (one per LPR lanes)
  constexpr int BC = 32 * LPR;                    // output columns per item
  __shared__ float tab[kNF ? kDxPairWords : 1];
  __shared__ float red[kWaves][MT][BC];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar offsets
  const int N = a.w.N, K = a.w.K, E = a.w.E;
  // items: expert by expert, row block, then 64-column block (fastest),
  // dealt to the XCDs in contiguous runs of the real item count
  const int nchunk = K >> 5, nblk = (nchunk + LPR - 1) / LPR;
  const int total = dx_total_tiles<MT>(a.offsets, E, nblk, lane);
  const int per = (total + 7) >> 3;
  const int bid = blockIdx.x, jb = bid >> 3;
  const int logical = (bid & 7) * per + jb;
  if (jb >= per || logical >= total) return;      // whole workgroup
  int e, start, mtiles;
  dx_find_tile<MT>(a.offsets, E, nblk, logical, lane, e, start, mtiles);
  if (e < 0) return;
  const int local = logical - start;
  const int rb = local / nblk, cb = local - rb * nblk;
  const int seg0 = a.offsets[e];
  const int count = a.offsets[e + 1] - seg0;
  const int prow0 = rb * MT;                      // first row of the item within the segment

  // this lane's chunk; MXFP4 with an odd chunk count: the last block's
  // second chunk is past K (loads clamped to chunk nchunk - 1, no sums kept)
  const int par = lane & (LPR - 1);
  const int kc_raw = LPR * cb + par;
  const bool chunk_ok = kc_raw < nchunk;
  const uint32_t kc = (uint32_t)min(kc_raw, nchunk - 1);
  const uint32_t half_k = (uint32_t)K >> 1, nkb = (uint32_t)K >> 6, ngrp = (uint32_t)K >> 5;
  const uint32_t col0 = kc * 32u;
  const uint32_t kb = col0 >> 6;
  const uint32_t scale_row = FMT == GNF4_NF4 ? nkb * 4u : kDQ ? nkb : ngrp;
  const uint32_t scale_col = FMT == GNF4_NF4 ? kb * 4u : kDQ ? kb : kc;
  const int64_t erow = (int64_t)e * N;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w.codes + erow * half_k), (short)0, (int)((uint32_t)N * half_k), kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(reinterpret_cast<const uint8_t *>(a.w.scales) + erow * scale_row), (short)0,
      (int)((uint32_t)N * scale_row), kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rs2 = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.w.scales2, (short)0,
      kDQ ? (int)(uint32_t)((((int64_t)E * N * nkb + 255) >> 8) * 4) : 0, kDxBufferDword3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.dY + (int64_t)seg0 * N), (short)0, (int)((uint32_t)count * (uint32_t)N * 2u),
      kDxBufferDword3);
  uint32_t dyrow[MT];                             // byte offset of row p, element 0
#pragma unroll
  for (int m = 0; m < MT; ++m) dyrow[m] = (uint32_t)min(prow0 + m, count - 1) * (uint32_t)N * 2u;

  // this wave's 32-row groups: R = wave + 8 i; the first `nfull_w` are whole
  const int rl = lane / LPR;                      // row within a group
  const int groups = (N + RPG - 1) / RPG;
  const int nfull_w = (N / RPG - wave + kWaves - 1) / kWaves > 0 ? (N / RPG - wave + kWaves - 1) / kWaves : 0;
  const int nall_w = (groups - wave + kWaves - 1) / kWaves > 0 ? (groups - wave + kWaves - 1) / kWaves : 0;
  const int nb = nfull_w / U;                     // full batches of this wave

  uint4 cq[2][U];
  uint32_t sq[2][U], yq[2][U][MT];
  float tq[2][U];
  auto issue = [&](auto SET, int i0, bool clamp) {
    constexpr int S = decltype(SET)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t g0 = (uint32_t)(RPG * (wave + kWaves * (i0 + u)));   // first row of the group
      uint32_t row = g0 + (uint32_t)rl;
      if (clamp) row = min(row, (uint32_t)N - 1u);
      const uint32_t lr = clamp ? row : (uint32_t)rl;
      const uint32_t vc = lr * half_k + col0 / 2u;
      const uint32_t vs = lr * scale_row + scale_col;
      const uint32_t sc = clamp ? 0u : g0 * half_k, ss = clamp ? 0u : g0 * scale_row;
      cq[S][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, vc, sc, 0));
      if constexpr (FMT == GNF4_NF4) sq[S][u] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs, ss, 0);
      else sq[S][u] = __builtin_amdgcn_raw_buffer_load_b8(rs, vs, ss, 0);
      if constexpr (kDQ) {
        const int64_t blk = (erow + row) * nkb + kb;
        tq[S][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rs2, (uint32_t)(blk >> 8) * 4u, 0, 0));
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        yq[S][u][m] = __builtin_amdgcn_raw_buffer_load_b16(rd, dyrow[m] + lr * 2u,
                                                           clamp ? 0u : g0 * 2u, 0);
    }
  };

  float acc[MT][32];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[m][j] = 0.0f;
  const uint32_t lane8 = (uint32_t)(lane & 31) * 8u;

  auto consume = [&](auto SET, int i0, bool clamp) {
    constexpr int S = decltype(SET)::value;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sc;
      if constexpr (FMT == GNF4_NF4) sc = __builtin_bit_cast(float, sq[S][u]);
      else if constexpr (kDQ) sc = (float)(int8_t)sq[S][u] * tq[S][u];
      else sc = e8m0_to_f32(sq[S][u]);
      const int row = RPG * (wave + kWaves * (i0 + u)) + rl;
      const bool live = !clamp || (i0 + u < nall_w && row < N);
      float sv[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float y = __builtin_bit_cast(float, yq[S][u][m] << 16);
        if constexpr (kNF) sv[m] = live ? y * sc : 0.0f;
        else sv[m] = live ? y : 0.0f;
      }
      const uint32_t wd[4] = {cq[S][u].x, cq[S][u].y, cq[S][u].z, cq[S][u].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v0, v1;
          if constexpr (kNF) {
            const float2 pr = *reinterpret_cast<const float2 *>(
                reinterpret_cast<const char *>(tab) +
                __builtin_amdgcn_perm(wd[d], lane8, 0x0c0c0000u | ((4u + (uint32_t)b) << 8)));
            v0 = pr.x;
            v1 = pr.y;
          } else {
            typedef float f32x2_t __attribute__((ext_vector_type(2)));
            f32x2_t pv;
            if (b == 0) pv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], sc, 0);
            else if (b == 1) pv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], sc, 1);
            else if (b == 2) pv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], sc, 2);
            else pv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd[d], sc, 3);
            v0 = pv[0];
            v1 = pv[1];
          }
          const int j = 8 * d + 2 * b;           // columns j, j + 1 of the chunk
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            acc[m][j] = __builtin_fmaf(sv[m], v0, acc[m][j]);
            acc[m][j + 1] = __builtin_fmaf(sv[m], v1, acc[m][j + 1]);
          }
        }
      }
    }
  };

  if (nb > 0) issue(Set0{}, 0, false);            // in flight while the table fills
  if constexpr (kNF) {
    if (tid < kDxThreads) fill_dx_table(tab, tid);
  }
  __syncthreads();
  for (int b = 0; b < nb; b += 2) {
    issue(Set1{}, U * min(b + 1, nb - 1), false);
    consume(Set0{}, U * b, false);
    if (b + 1 < nb) {
      issue(Set0{}, U * min(b + 2, nb - 1), false);
      consume(Set1{}, U * (b + 1), false);
    }
  }
  for (int i0 = nb * U; i0 < nall_w; i0 += U) {
    issue(Set0{}, i0, true);
    consume(Set0{}, i0, true);
  }

  // reduce over the RPG lanes of each chunk (lane bits 5 .. log2 LPR): values
  // are ordered v = j * MT + m, so the halvings leave the lane with chunk par
  // and group row rl holding columns (32 / RPG) * rl + i, i < 32 / RPG
  constexpr int KEEP = 32 / RPG;                  // columns per lane after the halvings
  float v[32 * MT];
#pragma unroll
  for (int j = 0; j < 32; ++j)
#pragma unroll
    for (int m = 0; m < MT; ++m) v[j * MT + m] = chunk_ok ? acc[m][j] : 0.0f;
  halve<16 * MT>(v, 32, lane);
  halve<8 * MT>(v, 16, lane);
  halve<4 * MT>(v, 8, lane);
  if constexpr (LPR <= 4) halve<2 * MT>(v, 4, lane);
  if constexpr (LPR <= 2) halve<MT>(v, 2, lane);
#pragma unroll
  for (int i = 0; i < KEEP; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][32 * par + KEEP * rl + i] = v[i * MT + m];
  __syncthreads();
  // threads 0 .. BC MT - 1: row m = tid / BC, column tid % BC, waves in order
  for (int t = tid; t < BC * MT; t += kDxGemvThreads) {
    const int m = t / BC, c = t % BC;
    float sum = red[0][m][c];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w][m][c];
    const int col = BC * cb + c;
    if (prow0 + m < count && col < K) a.dA[(int64_t)(seg0 + prow0 + m) * K + col] = sum;
  }
}

template <int FMT, int MT, int LPR>
static hipError_t gemv_dx_go(const DxArgs &a, hipStream_t s) {
  const int rows = a.rows;
  const int nblk = (a.w.K / 32 + LPR - 1) / LPR;
  const int64_t items = ((int64_t)(rows + MT - 1) / MT + std::min<int>(a.w.E, rows)) * nblk;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((gemv_dx_kernel<FMT, MT, LPR>), dim3((unsigned)grid), dim3(kDxGemvThreads), 0, s,
                     a);
  return hipGetLastError();
}

// Lanes per weight row: 4 (128-column items, half the lines per load of 2)
// when that still gives every CU an item, else 2 (measured: 4 wins on the
// Qwen3-235B shape, 2 on the OLMoE, Qwen3-30B and gpt-oss shapes).
template <int FMT, int MT>
static hipError_t gemv_dx_pick(const DxArgs &a, hipStream_t s) {
  const int64_t experts = std::min<int64_t>(a.w.E, a.rows);
  const int64_t items4 = experts * ((a.w.K / 32 + 3) / 4);
  if (items4 >= device_cu_count()) return gemv_dx_go<FMT, MT, 4>(a, s);
  return gemv_dx_go<FMT, MT, 2>(a, s);
}

template <int FMT, int RT, int CT>
static hipError_t dx_go(const DxArgs &a, hipStream_t s) {
  constexpr int BM = 16 * RT;
  const int rows = a.rows;
  const int n_tiles_k = (a.w.K + 64 * CT - 1) / (64 * CT);
  const int64_t m_tiles = (rows + BM - 1) / BM + std::min<int>(a.w.E, rows);
  const int64_t bound = m_tiles * n_tiles_k;
  const int64_t grid = (bound + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((mfma_dx_kernel<FMT, RT, CT>), dim3((unsigned)grid), dim3(kDxThreads), 0, s, a,
                     n_tiles_k);
  return hipGetLastError();
}

// Row tile from the mean rows per active expert (a host-side estimate: the
// routing stays on the device).
template <int FMT>
static hipError_t dx_pick(const DxArgs &a, hipStream_t s) {
  const int64_t experts = std::min<int64_t>(a.w.E, a.rows);
  const int64_t mean = experts > 0 ? (a.rows + experts - 1) / experts : 0;
  if (a.rows <= kGemvDxMaxRows) {
    if (mean <= 1) return gemv_dx_pick<FMT, 1>(a, s);
    if (mean <= 2) return gemv_dx_pick<FMT, 2>(a, s);
    if (mean <= 4) return gemv_dx_pick<FMT, 4>(a, s);
  }
  if (mean <= 16) return dx_go<FMT, 1, 4>(a, s);
  if (mean <= 32) return dx_go<FMT, 2, 4>(a, s);
  if (mean <= 96) return dx_go<FMT, 4, 4>(a, s);
  return dx_go<FMT, 8, 2>(a, s);
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
