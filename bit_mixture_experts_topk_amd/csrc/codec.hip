// Packing and unpacking of the 4-bit weight formats.
//
//  * dequant_kernel: decodes one expert to float32 (the bit-exact test aid).
//  * quantize kernels: pack float32 weights into NF4, NF4 with an int8
//    double-quantized absmax, or MXFP4 (offline step, not on the hot path).
//
// Formats: NF4 on the bitsandbytes layout and MXFP4 on the released bytes
// (Jordan Anderson, jordananderson-pages.pages.dev, section
// "grouped-nf4-gemm & experts-4bit", first and third bullets; e2m1 + e8m0
// per "MoE Training on Consumer GPUs -- Loggetta & Cerin Amroth", Task guides
// table). The NF4 values are the QLoRA NormalFloat-4 construction; the MXFP4
// conversion follows the OCP Microscaling v1.0 rule.
#include "common.h"

namespace gnf4 {

__device__ __forceinline__ float nf4_value(uint32_t q) {
  return __builtin_bit_cast(float, kNF4Bits[q & 15u]);
}

__device__ __forceinline__ float e2m1_value(uint32_t q) {
  const float m = kE2M1[q & 7u];
  return (q & 8u) ? -m : m;
}

// ---------------------------------------------------------------- dequant ---

constexpr int kCodecThreads = 256;

// One thread per 16 packed bytes (32 values) of expert e.
__global__ __launch_bounds__(kCodecThreads) void dequant_kernel(Weights w, int e,
                                                                float *__restrict__ out) {
  const int64_t chunks_per_row = w.K / 32;
  const int64_t chunk = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
  if (chunk >= (int64_t)w.N * chunks_per_row) return;
  const int64_t n = chunk / chunks_per_row, c = chunk % chunks_per_row;
  const int64_t row = (int64_t)e * w.N + n;
  const uint4 q4 = *reinterpret_cast<const uint4 *>(w.codes + row * (w.K / 2) + c * 16);
  const uint32_t qw[4] = {q4.x, q4.y, q4.z, q4.w};
  float *dst = out + n * w.K + c * 32;
  if (w.format == GNF4_MXFP4) {
    const uint32_t s = reinterpret_cast<const uint8_t *>(w.scales)[row * (w.K / 32) + c];
    const float sc = e8m0_to_f32(s);
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = (qw[i >> 2] >> ((i & 3) * 8)) & 0xffu;
      dst[2 * i] = e2m1_value(b & 15u) * sc;        // element 2i: low nibble
      dst[2 * i + 1] = e2m1_value(b >> 4) * sc;
    }
  } else {
    const int64_t blk = row * (w.K / 64) + c / 2;
    float a;
    if (w.format == GNF4_NF4) {
      a = reinterpret_cast<const float *>(w.scales)[blk];
    } else {
      const int q8 = reinterpret_cast<const int8_t *>(w.scales)[blk];
      a = (float)q8 * w.scales2[blk >> 8];
    }
    for (int i = 0; i < 16; ++i) {
      const uint32_t b = (qw[i >> 2] >> ((i & 3) * 8)) & 0xffu;
      dst[2 * i] = nf4_value(b >> 4) * a;             // element 2i: high nibble
      dst[2 * i + 1] = nf4_value(b & 15u) * a;
    }
  }
}

// The decode of the dequantize-then-matmul comparison path: the experts
// listed in experts[0 .. min(*count, max_experts)) decoded to bf16 (the
// exact float32 value rounded to nearest even; NaN stays a quiet NaN) into
// out[slot][N][K]. One thread per 4 packed bytes (8 values, one 16-byte
// store), so a wave's loads and stores each cover one contiguous span. The
// 16 code values sit in lanes 0..15 of a register and reach each lane
// through ds_bpermute (no select chain, no bank conflicts). Every lane of a
// wave takes part in the permutes; lanes without work skip loads and stores.
__global__ __launch_bounds__(kCodecThreads) void dequant_bf16_kernel(
    Weights w, const int32_t *__restrict__ experts, const int32_t *__restrict__ count,
    int32_t max_experts, uint16_t *__restrict__ out) {
  const int64_t per_expert = (int64_t)w.N * (w.K / 8);      // 8-value groups
  const int64_t grp = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool mx = w.format == GNF4_MXFP4;
  const float table = mx ? e2m1_value((uint32_t)lane) : nf4_value((uint32_t)lane);
  const int slot = (int)(grp / per_expert);
  int e = -1;
  if (slot < max_experts && slot < *count) e = experts[slot];
  const bool live = e >= 0 && e < w.E;
  if (!__any(live)) return;                     // whole wave idle
  const int64_t rem = grp - (int64_t)slot * per_expert;
  const int64_t n = rem / (w.K / 8), j = rem % (w.K / 8);    // 8-value group j of row n
  const int64_t row = (int64_t)(live ? e : 0) * w.N + (live ? n : 0);
  uint32_t q = 0;
  float sc = 0.0f;
  if (live) {
    q = reinterpret_cast<const uint32_t *>(w.codes + row * (w.K / 2))[j];
    if (mx) {
      sc = e8m0_to_f32(reinterpret_cast<const uint8_t *>(w.scales)[row * (w.K / 32) + j / 4]);
    } else {
      const int64_t blk = row * (w.K / 64) + j / 8;
      sc = w.format == GNF4_NF4
               ? reinterpret_cast<const float *>(w.scales)[blk]
               : (float)reinterpret_cast<const int8_t *>(w.scales)[blk] * w.scales2[blk >> 8];
    }
  }
  const int tbits = __builtin_bit_cast(int, table);
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (q >> (8 * i)) & 0xffu;
    // element 2i: NF4 high nibble, MXFP4 low nibble
    const uint32_t q0 = mx ? (b & 15u) : (b >> 4), q1 = mx ? (b >> 4) : (b & 15u);
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((int)(q0 << 2), tbits)) * sc;
    const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((int)(q1 << 2), tbits)) * sc;
    const uint32_t u0 = __builtin_bit_cast(uint32_t, v0), u1 = __builtin_bit_cast(uint32_t, v1);
    const uint32_t r0 = (v0 != v0) ? 0x7fc0u : ((u0 + 0x7fffu + ((u0 >> 16) & 1u)) >> 16);
    const uint32_t r1 = (v1 != v1) ? 0x7fc0u : ((u1 + 0x7fffu + ((u1 >> 16) & 1u)) >> 16);
    h[i] = r0 | (r1 << 16);
  }
  if (!live) return;
  *reinterpret_cast<uint4 *>(out + ((int64_t)slot * w.N + n) * w.K + j * 8) =
      make_uint4(h[0], h[1], h[2], h[3]);
}

hipError_t launch_dequant_bf16(const Weights &w, const int32_t *experts, const int32_t *count,
                               int32_t max_experts, uint16_t *out, hipStream_t s) {
  const int64_t groups = (int64_t)max_experts * w.N * (w.K / 8);
  const int64_t blocks = (groups + kCodecThreads - 1) / kCodecThreads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_bf16_kernel, dim3((unsigned)blocks), dim3(kCodecThreads), 0, s, w,
                     experts, count, max_experts, out);
  return hipGetLastError();
}

hipError_t launch_dequant(const Weights &w, int32_t e, float *out, hipStream_t s) {
  const int64_t chunks = (int64_t)w.N * (w.K / 32);
  const int64_t blocks = (chunks + kCodecThreads - 1) / kCodecThreads;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(kCodecThreads), 0, s, w, e, out);
  return hipGetLastError();
}

// --------------------------------------------------------------- quantize ---

// NF4 code of x = w / absmax (float64): the number of codebook midpoints
// strictly below x, i.e. the nearest value with ties to the lower code.
__device__ __forceinline__ uint32_t nf4_encode(double x) {
  uint32_t q = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    const double mid = 0.5 * ((double)nf4_value(i) + (double)nf4_value(i + 1));
    q += (x > mid) ? 1u : 0u;
  }
  return q;
}

// Absmax and codes of one 64-value block; writes 32 packed bytes.
__device__ float nf4_block(const float *__restrict__ src, uint8_t *__restrict__ dst) {
  float a = 0.f;
  for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(src[i]));
  uint32_t words[8];
  for (int j = 0; j < 8; ++j) {
    uint32_t wv = 0;
    for (int bi = 0; bi < 4; ++bi) {
      const int i = j * 8 + bi * 2;
      uint32_t q0 = 7u, q1 = 7u;
      if (a > 0.f) {
        q0 = nf4_encode((double)src[i] / (double)a);
        q1 = nf4_encode((double)src[i + 1] / (double)a);
      }
      wv |= ((q0 << 4) | q1) << (bi * 8);
    }
    words[j] = wv;
  }
  uint4 *d = reinterpret_cast<uint4 *>(dst);
  d[0] = make_uint4(words[0], words[1], words[2], words[3]);
  d[1] = make_uint4(words[4], words[5], words[6], words[7]);
  return a;
}

__global__ __launch_bounds__(kCodecThreads) void quantize_nf4_kernel(
    const float *__restrict__ W, int64_t nblocks, uint8_t *__restrict__ codes,
    float *__restrict__ absmax) {
  const int64_t b = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
  if (b >= nblocks) return;
  absmax[b] = nf4_block(W + b * 64, codes + b * 32);
}

// NF4 with double-quantized absmax: one workgroup per group of 256 blocks.
// scale2 = fp32(max / 127) (float64 division), q8 = clip(rint(a / scale2), 0, 127).
__global__ __launch_bounds__(kCodecThreads) void quantize_nf4dq_kernel(
    const float *__restrict__ W, int64_t nblocks, uint8_t *__restrict__ codes,
    int8_t *__restrict__ q8, float *__restrict__ scales2) {
  __shared__ float red[kCodecThreads / 64];
  const int64_t b = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
  float a = 0.f;
  if (b < nblocks) a = nf4_block(W + b * 64, codes + b * 32);
  float m = a;
  for (int d = 32; d > 0; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s2 = (float)((double)m / 127.0);
  if (threadIdx.x == 0) scales2[blockIdx.x] = s2;
  if (b < nblocks) {
    int q = 0;
    if (s2 > 0.f) {
      const double r = __builtin_rint((double)a / (double)s2);
      q = (int)fmin(fmax(r, 0.0), 127.0);
    }
    q8[b] = (int8_t)q;
  }
}

// e2m1 code of a float64 value: nearest magnitude, ties to the even
// mantissa, saturating at 6; the sign bit is taken from `neg`.
__device__ __forceinline__ uint32_t e2m1_encode(double v, bool neg) {
  const double m = fmin(fabs(v), 6.0);
  // Midpoints between consecutive magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t q = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    // above the midpoint: the upper neighbour; exactly on it: the even code
    if (m > mids[i] || (m == mids[i] && ((i + 1) & 1) == 0)) q = i + 1;
  }
  return q | (neg ? 8u : 0u);
}

// One thread per 32-value block: shared exponent floor(log2 amax) - 2 taken
// from the float32 bits, s = clamp(e + 127, 0, 254), then per-value rounding
// of w * 2^(127 - s) (exact in float64).
__global__ __launch_bounds__(kCodecThreads) void quantize_mxfp4_kernel(
    const float *__restrict__ W, int64_t nblocks, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * kCodecThreads + threadIdx.x;
  if (b >= nblocks) return;
  const float *src = W + b * 32;
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(src[i]));
  int s = 0;
  if (amax > 0.f) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
    const int ex = (int)(bits >> 23);
    const int fl = ex > 0 ? ex - 127 : (31 - __builtin_clz(bits & 0x7fffffu)) - 149;
    s = min(max(fl - 2 + 127, 0), 254);
  }
  const double inv = __builtin_bit_cast(double, (uint64_t)(1023 + 127 - s) << 52);  // 2^(127-s)
  uint32_t words[4];
  for (int j = 0; j < 4; ++j) {
    uint32_t wv = 0;
    for (int bi = 0; bi < 4; ++bi) {
      const int i = j * 8 + bi * 2;
      const float x0 = src[i], x1 = src[i + 1];
      const uint32_t q0 = e2m1_encode((double)x0 * inv, __builtin_bit_cast(uint32_t, x0) >> 31);
      const uint32_t q1 = e2m1_encode((double)x1 * inv, __builtin_bit_cast(uint32_t, x1) >> 31);
      wv |= (q0 | (q1 << 4)) << (bi * 8);                // element 2i: low nibble
    }
    words[j] = wv;
  }
  *reinterpret_cast<uint4 *>(codes + b * 16) = make_uint4(words[0], words[1], words[2], words[3]);
  scales[b] = (uint8_t)s;
}

hipError_t launch_quantize(int32_t fmt, const float *W, int32_t rows, int32_t K, uint8_t *codes,
                           void *scales, float *scales2, hipStream_t s) {
  if (fmt == GNF4_MXFP4) {
    const int64_t nb = (int64_t)rows * (K / 32);
    if (nb == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)((nb + kCodecThreads - 1) / kCodecThreads)),
                       dim3(kCodecThreads), 0, s, W, nb, codes, (uint8_t *)scales);
    return hipGetLastError();
  }
  const int64_t nb = (int64_t)rows * (K / 64);
  if (nb == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nb + kCodecThreads - 1) / kCodecThreads);
  if (fmt == GNF4_NF4) {
    hipLaunchKernelGGL(quantize_nf4_kernel, dim3(grid), dim3(kCodecThreads), 0, s, W, nb, codes,
                       (float *)scales);
  } else {
    hipLaunchKernelGGL(quantize_nf4dq_kernel, dim3(grid), dim3(kCodecThreads), 0, s, W, nb, codes,
                       (int8_t *)scales, scales2);
  }
  return hipGetLastError();
}

}  // namespace gnf4
