// Shared device-side definitions for the gnf4 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gnf4.h"

namespace gnf4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// NF4 codebook, float32 bit patterns, index = 4-bit code. These are the 16
// NormalFloat-4 values of the QLoRA construction (8 positive and 7 negative
// N(0,1) quantiles from offset (1-1/30 + 1-1/32)/2, an exact zero, normalised
// to [-1, 1]) rounded to float32.
static constexpr uint32_t kNF4Bits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

// bfloat16 bits of a float32 value (round to nearest even).
__host__ __device__ constexpr uint32_t bf16_rne(uint32_t f) {
  return (f + 0x7fffu + ((f >> 16) & 1u)) >> 16;
}

// The bf16 operand of the NF4 contractions. bf16 keeps 8 significant bits,
// so each codebook value enters the products with a fixed rounding error,
// and these errors add up over K in every output. The kernels use
// bf16(s * c[q]) instead and scale each 64-value partial by absmax / s:
//   y = sum_blocks fp32(absmax * (1/s)) * sum_k x[k] * bf16(s * c[q[k]]).
// s is the float32 in [1, 2) that minimizes the mean over the 16 codes of
// (bf16(fp32(s * c[q])) / s - c[q])^2: 2.9x below the unscaled codebook's
// (s = 1), which the error of an output grows with (a sum of x * absmax *
// rounding error over K). The extra float32 rounding of absmax / s is 2^-24
// relative.
static constexpr float kNF4Scale = 1.43700611591339111328125f;   // 0x3fb7efd1
static constexpr float kNF4InvScale = 1.0f / kNF4Scale;

__host__ __device__ constexpr uint32_t nf4_bf16_bits(uint32_t q) {
  return bf16_rne(__builtin_bit_cast(uint32_t, __builtin_bit_cast(float, kNF4Bits[q & 15u]) * kNF4Scale));
}

// e2m1 magnitudes by the low three code bits.
static constexpr float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

// float32 value 2^(s-127) of an e8m0 byte: s = 0 is the subnormal 2^-127,
// s = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t bits = (s == 0u) ? 0x00400000u : (s == 255u ? 0x7fc00000u : (s << 23));
  return __builtin_bit_cast(float, bits);
}

// Kernel-side view of the weights.
struct Weights {
  int32_t format, E, N, K;
  const uint8_t *codes;
  const void *scales;
  const float *scales2;
};

struct GemmArgs {
  Weights w;
  const uint16_t *X;
  int32_t gather;
  const int32_t *offsets;
  const int32_t *perm;
  const int32_t *active;
  const int32_t *n_active;
  int32_t T, k;
  float *Y;          // float32 output [T*k][N] (plain GEMM)
  uint16_t *H;       // bf16 output [T*k][N/2] (SwiGLU epilogue; then Y is unused)
  // Routing fused into the one-token GEMV: the token's k ids and where the
  // routing outputs go (as gnf4_route writes them); ids == NULL when the
  // routing was done beforehand (offsets / active / n_active are read).
  const int32_t *ids;
  int32_t *r_counts, *r_offsets, *r_perm, *r_inv, *r_active, *r_n_active, *r_bad;
  // ... or the router's logits [1][E] (then the top-k ids and softmax weights
  // are formed first and written to r_topk_ids / r_topk_w)
  const float *logits;
  int32_t *r_topk_ids;
  float *r_topk_w;
};

// Input gradient of the grouped GEMM: dA [rows][K] from dY [rows][N], both
// in routed (permuted) order, segments given by offsets.
struct DxArgs {
  Weights w;
  const uint16_t *dY;
  const int32_t *offsets;
  int32_t rows;
  float *dA;
};

// Copy of listed experts' packed bytes into cache slots: segment g of expert
// e is seg_units[g] 16-byte units at src[g] + e * seg_units[g] (codes,
// scales, and for NF4_DQ scales2), written to dst[g] + s * seg_units[g].
struct CacheFillArgs {
  const void *src[3];
  void *dst[3];
  int64_t seg_units[3];
  int nseg;
  int64_t units;                 // sum of seg_units
  int64_t chunks;                // workgroups per copy
  int E, S;
  const int32_t *copies;         // [0] count, then (expert, slot) pairs
};

// SwiGLU (the activation between a mixture-of-experts layer's projections;
// not described on the pages, the form of the public models the workloads
// follow): bf16 of silu(g) * u, silu(x) = x / (1 + exp(-x)), rounded once
// from the float64 value. Shared by gnf4_swiglu and the GEMM's epilogue so
// that both round alike.
// float64 -> bfloat16 bits, nearest with ties to even, straight from the
// float64 significand (no float32 step, which could round twice). A finite
// x = m53 * 2^(e - 52) with the 53-bit significand m53; bf16 keeps the
// significand n = m53 / 2^s rounded, s = 45 + (E - e), where E = max(e, -126)
// is the bf16 exponent (-126 for its subnormals). NaN gives 0x7FC0.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  const int ex = (int)((b >> 52) & 0x7ff);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7ff) return man ? (uint16_t)0x7FC0 : (uint16_t)(sign | 0x7F80);
  if (ex == 0) return (uint16_t)sign;           // zero or below 2^-1022: rounds to zero
  const int e = ex - 1023;
  int E = e > -126 ? e : -126;
  const int sh = 45 + (E - e);
  const uint64_t m53 = (1ull << 52) | man;
  uint32_t n;
  if (sh >= 64) {
    n = 0;                                      // below a quarter of the smallest subnormal
  } else {
    n = (uint32_t)(m53 >> sh);
    const uint64_t rem = m53 & ((1ull << sh) - 1), half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (n & 1u))) ++n;
  }
  if (n == 256) {
    n = 128;
    ++E;
  }
  if (E > 127) return (uint16_t)(sign | 0x7F80);
  if (n < 128) return (uint16_t)(sign | n);     // subnormal (E = -126)
  return (uint16_t)(sign | ((uint32_t)(E + 127) << 7) | (n - 128));
}

// bf16 of silu(g) * u as the float64 product rounds it. The float32
// estimate (g * u) * rcp(1 + expf(-g)) carries a few float32 ulps of
// relative error (expf and v_rcp_f32 within 1-2 ulps each, three roundings
// of half an ulp), so it rounds to the same bf16 as the exact value unless
// it lies within that error of a rounding midpoint; those values, and the
// ranges where the estimate loses its relative accuracy (exp(-g) overflowing,
// a gate or result near the float32 subnormal or overflow range, non-finite
// values), are redone in float64. With |g| >= 2^-100, g > -80 and the result
// between 2^-99 and 2^100 every intermediate is a normal float32, and the
// error stays below 11 ulps of h; the margin is 16.
__device__ __forceinline__ uint16_t swiglu_bf16(float g, float u) {
  const float h = (g * u) * __builtin_amdgcn_rcpf(1.0f + expf(-g));
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const uint32_t ex = (hb >> 23) & 0xffu;
  const uint32_t gex = (__builtin_bit_cast(uint32_t, g) >> 23) & 0xffu;
  const int32_t mid = (int32_t)(hb & 0xffffu) - 0x8000;
  const bool easy = g > -80.0f && gex > 26u && ex > 27u && ex < 227u && (mid > 16 || mid < -16);
  if (easy) return (uint16_t)((hb + 0x7fffu + ((hb >> 16) & 1u)) >> 16);
  const double x = (double)g;
  return f64_to_bf16_rne(x / (1.0 + exp(-x)) * (double)u);
}


// ------------------------------------------------ router top-k of one token

// Order of a logit as an unsigned integer that increases with its value:
// the float's bits mapped monotonically, -0 taken as +0 (so that the two tie
// like equal values), NaN as 1 (below -inf); 0 marks an absent or already
// chosen entry. Equal orders rank the lower expert first.
__device__ __forceinline__ uint32_t topk_ord(float x) {
  const uint32_t u = x == 0.0f ? 0u : __builtin_bit_cast(uint32_t, x);
  return (x != x) ? 1u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
}

// The logit of an order (the map inverted; 1 gives a NaN).
__device__ __forceinline__ float topk_logit(uint32_t ord) {
  return __builtin_bit_cast(float, (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// 64-bit value of lane l (a uniform lane index): two readlanes.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
  return __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, x), l));
}

// max(v, the value of the lane CTRL names), a DPP row shift; lanes without a
// source read 0, the smallest value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
  return o > v ? o : v;
}

// The largest value of the wave, the same in every lane: four DPP right
// shifts by 1, 2, 4, 8 within each row of 16 lanes leave the row's maximum in
// its last lane (15, 31, 47, 63), read with readlanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0x111>(v);                    // row_shr:1
  v = dpp_max_u32<0x112>(v);                    // row_shr:2
  v = dpp_max_u32<0x114>(v);                    // row_shr:4
  v = dpp_max_u32<0x118>(v);                    // row_shr:8
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t m1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t m2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t m3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  return max(max(m0, m1), max(m2, m3));
}

// k rounds of the router's top-k over the first M orders of each lane (the
// ones past M are 0): round r takes the largest remaining order and, among
// the entries that hold it, the lowest expert (first the lowest j, then the
// lowest lane); its owner lane clears it, and lane r keeps the expert and
// the order.
template <int M, int NPL>
__device__ __forceinline__ void topk_rounds(uint32_t (&ord)[NPL], int k, int lane, int &mine,
                                            uint32_t &mine_ord) {
  for (int r = 0; r < k; ++r) {
    uint32_t best = ord[0];
#pragma unroll
    for (int j = 1; j < M; ++j) best = max(best, ord[j]);
    best = wave_max_u32(best);
    int e = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      const uint64_t hit = __ballot(ord[j] == best);
      if (!found && hit) {
        e = 64 * j + __builtin_ctzll(hit);
        found = true;
      }
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (j == (e >> 6)) ord[j] = 0;
    }
    if (lane == r) {
      mine = e;
      mine_ord = best;
    }
  }
}

// The router's choice for one token's logits row[0 .. E) (E <= 64 NPL), by
// one whole wave: lane l holds the orders of experts l + 64 j (j < NPL); k
// rounds each take the largest remaining one, over as many orders per lane
// as E needs (a uniform branch picks the compiled width). Lane j < k returns
// the j-th choice and its softmax weight, formed in float64 (the largest
// chosen logit subtracted, the exponentials summed in rank order by every
// lane alike) and rounded to float32. The result does not depend on NPL.
template <int NPL>
__device__ __forceinline__ void topk_row(const float *row, int E, int k, int lane, int &id,
                                         float &wt) {
  const int npl = (E + 63) >> 6;                // orders in use per lane (NPL is the most)
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) v[j] = row[min(lane + 64 * j, E - 1)];   // all loads in flight at once
  uint32_t ord[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) ord[j] = lane + 64 * j < E ? topk_ord(v[j]) : 0u;
  int mine = 0;                                 // lane r: the expert chosen in round r
  uint32_t mine_ord = 0;                        // and its order
  constexpr int M2 = NPL < 2 ? NPL : 2, M4 = NPL < 4 ? NPL : 4, M8 = NPL < 8 ? NPL : 8;
  if (npl <= 1) topk_rounds<1, NPL>(ord, k, lane, mine, mine_ord);
  else if (npl <= 2) topk_rounds<M2, NPL>(ord, k, lane, mine, mine_ord);
  else if (npl <= 4) topk_rounds<M4, NPL>(ord, k, lane, mine, mine_ord);
  else if (npl <= 8) topk_rounds<M8, NPL>(ord, k, lane, mine, mine_ord);
  else topk_rounds<NPL, NPL>(ord, k, lane, mine, mine_ord);
  const double x = lane < k ? (double)topk_logit(mine_ord) : 0.0;   // the chosen logit
  const double m = readlane_f64(x, 0);
  const double ex = exp(x - m);
  double s = 0.0;
  for (int j = 0; j < k; ++j) s += readlane_f64(ex, j);
  id = mine;
  wt = (float)(ex / s);
}

// NF4 byte -> two bf16 operand values (nf4_bf16_bits) as one dword (element
// 2i, the high nibble, in the low half): the operand layout of v_dot2 and of
// the MFMA fragments, where consecutive K values sit low half first.
__host__ __device__ constexpr uint32_t nf4_pair(uint32_t byte) {
  return nf4_bf16_bits(byte >> 4) | (nf4_bf16_bits(byte & 15u) << 16);
}

// LDS decode table of NF4 byte pairs, replicated once per lane of a wave so
// that every lane reads its own bank: entry b of copy c lives at byte offset
// b * 256 + c * 4. 256 entries x 64 copies x 4 B = 64 KiB.
constexpr int kLutCopies = 64;
constexpr int kLutWords = 256 * kLutCopies;

// bf16 operand value of code q (0..15) without memory: the 16 values packed
// into four 64-bit constants.
__device__ __forceinline__ uint32_t nf4_bf16(uint32_t q) {
  constexpr uint64_t w0 = (uint64_t)nf4_bf16_bits(0) | ((uint64_t)nf4_bf16_bits(1) << 16) |
                          ((uint64_t)nf4_bf16_bits(2) << 32) | ((uint64_t)nf4_bf16_bits(3) << 48);
  constexpr uint64_t w1 = (uint64_t)nf4_bf16_bits(4) | ((uint64_t)nf4_bf16_bits(5) << 16) |
                          ((uint64_t)nf4_bf16_bits(6) << 32) | ((uint64_t)nf4_bf16_bits(7) << 48);
  constexpr uint64_t w2 = (uint64_t)nf4_bf16_bits(8) | ((uint64_t)nf4_bf16_bits(9) << 16) |
                          ((uint64_t)nf4_bf16_bits(10) << 32) | ((uint64_t)nf4_bf16_bits(11) << 48);
  constexpr uint64_t w3 = (uint64_t)nf4_bf16_bits(12) | ((uint64_t)nf4_bf16_bits(13) << 16) |
                          ((uint64_t)nf4_bf16_bits(14) << 32) | ((uint64_t)nf4_bf16_bits(15) << 48);
  const uint64_t w = (q < 8u) ? ((q < 4u) ? w0 : w1) : ((q < 12u) ? w2 : w3);
  return (uint32_t)(w >> ((q & 3u) * 16u)) & 0xffffu;
}

// Fill the table with a 256-thread workgroup. Thread t writes 16-byte groups
// g = t + 256 i (i = 0..15), i.e. 4 copies of entry b = g / 16 = t / 16 + 16 i.
// For that entry the high nibble (element 2i of the pair) is i and the low
// nibble is t / 16, so each thread decodes one value and ORs in constants;
// consecutive lanes write consecutive 16-byte groups (no bank conflicts).
__device__ __forceinline__ void fill_nf4_lut_256(uint32_t *lut, int tid) {
  const uint32_t lo = nf4_bf16((uint32_t)tid >> 4) << 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = nf4_bf16_bits(i) | lo;
    *reinterpret_cast<uint4 *>(lut + (tid + 256 * i) * 4) = make_uint4(v, v, v, v);
  }
}

// Fill the table with a workgroup of NT threads (NT divides 4096): thread t
// writes the 16-byte groups g = t + NT i, each 4 copies of entry g / 16.
template <int NT>
__device__ __forceinline__ void fill_nf4_lut(uint32_t *lut, int tid) {
  static_assert(4096 % NT == 0, "16-byte groups per thread");
#pragma unroll
  for (int i = 0; i < 4096 / NT; ++i) {
    const uint32_t grp = (uint32_t)tid + NT * i, b = grp >> 4;
    const uint32_t v = nf4_bf16(b >> 4) | (nf4_bf16(b & 15u) << 16);
    *reinterpret_cast<uint4 *>(lut + grp * 4) = make_uint4(v, v, v, v);
  }
}

// Byte offset into the table for byte i (0..3) of dword w, for this lane:
// v_perm_b32 places byte i of w in bits 8..15 and this lane's copy offset
// (lane * 4, < 256) in bits 0..7, so one instruction forms the address.
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, uint32_t lane4, int i) {
  return __builtin_amdgcn_perm(w, lane4, 0x0c0c0000u | ((4u + (uint32_t)i) << 8));
}

__device__ __forceinline__ uint32_t lut_read(const uint32_t *lut, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lut) + byte_off);
}

// MXFP4 byte i (0..3) of dword w -> two bf16 (low nibble first), times scale.
template <int I>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, I));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Host-side launchers (one per kernel family), defined in the .hip files.
hipError_t launch_route(const int32_t *ids, int32_t T, int32_t k, int32_t E, int32_t *counts,
                        int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                        int32_t *n_active, int32_t *bad, void *workspace, hipStream_t s);
// Workspace bytes the route of n assignments over E experts needs (0 when
// one workgroup routes them).
size_t route_workspace_bytes(int64_t n, int32_t E);
// The per-device file-scope route workspace (gnf4_route_noalloc): its size,
// and its device address on the current device (resolved once per device).
size_t route_scratch_bytes();
void *route_scratch_ptr(hipError_t *err);
hipError_t launch_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids,
                       float *w, hipStream_t s);
hipError_t launch_swiglu(const float *Y, int32_t rows, int32_t I, uint16_t *H, hipStream_t s);
hipError_t launch_gemv(const GemmArgs &a, hipStream_t s);
hipError_t launch_mfma(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_dx(const DxArgs &a, hipStream_t s);
// One token's second projection with the combine fused (T = 1, routed-order
// rows); gemv_combine_fits says whether that kernel takes the call.
bool gemv_combine_fits(const GemmArgs &a);
hipError_t launch_cache_reset(int32_t *state, int32_t E, int32_t S, hipStream_t s);
hipError_t launch_cache_stage(const int32_t *ids, int32_t n, int32_t E, int32_t S, int32_t *state,
                              int32_t *slot_ids, int32_t *copies, hipStream_t s);
hipError_t launch_cache_fill(const CacheFillArgs &f, int32_t max_copies, hipStream_t s);
int64_t cache_fill_chunks(int64_t units);
hipError_t launch_gemv_combine(const GemmArgs &a, const float *topk_w, const int32_t *inv,
                               float *out, hipStream_t s);
hipError_t launch_combine(const float *Y, const int32_t *inv, const float *w, int32_t T,
                          int32_t k, int32_t N, float *out, hipStream_t s);
hipError_t launch_dequant(const Weights &w, int32_t e, float *out, hipStream_t s);
hipError_t launch_dequant_bf16(const Weights &w, const int32_t *experts, const int32_t *count,
                               int32_t max_experts, uint16_t *out, hipStream_t s);
hipError_t launch_quantize(int32_t fmt, const float *W, int32_t rows, int32_t K, uint8_t *codes,
                           void *scales, float *scales2, hipStream_t s);

hipError_t launch_read_probe(const void *src, int64_t nbytes, int32_t workgroups, uint32_t *sink,
                             hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace gnf4
