// The steps either side of the grouped GEMM in a mixture-of-experts FFN
// layer: the router's top-k choice from logits (before gnf4_route) and the
// SwiGLU step between the two projections. The pages put the fused kernel
// behind a real router (Jordan Anderson, jordananderson-pages.pages.dev,
// section "grouped-nf4-gemm & experts-4bit", demonstration paragraph of the
// first bullet) without describing either step; the definitions here are
// those of the public models the workloads are shaped after.
#include "common.h"

namespace gnf4 {

// ---------------------------------------------------------------- top-k

// Order key of (logit, expert): larger keys rank first. The high half maps
// the float's bits to an unsigned integer that increases with the value
// (NaN maps to 0, below -inf); the low half is ~e, so that on equal logits
// the lower expert ranks first. Absent and already chosen entries use key 0,
// below every real entry (whose low half is at least ~1023).
__device__ __forceinline__ uint64_t topk_key(float x, int e) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t ord = (x != x) ? 0u : ((u & 0x80000000u) ? ~u : (u | 0x80000000u));
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token; lane l holds the logits of experts l + 64 j (j < NPL).
// k rounds each take the largest remaining key. Lane j < k then forms the
// softmax weight of the j-th choice in float64: the largest chosen logit
// subtracted, the exponentials summed in rank order by every lane alike.
template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                           // whole wave
  const float *row = logits + (int64_t)t * E;
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? topk_key(row[e], e) : 0ull;
  }
  int mine = 0;                                 // lane r: the expert chosen in round r
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)~(uint32_t)best;
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < NPL; ++j)
        if (j == (e >> 6)) key[j] = 0;
    }
    if (lane == r) mine = e;
  }
  const double x = lane < k ? (double)row[mine] : 0.0;
  const double m = __shfl(x, 0, 64);
  const double ex = exp(x - m);
  double s = 0.0;
  for (int j = 0; j < k; ++j) s += __shfl(ex, j, 64);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = mine;
    w[(int64_t)t * k + lane] = (float)(ex / s);
  }
}

hipError_t launch_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *ids,
                       float *w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 512) hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- SwiGLU

// H[p][i] = bf16(silu(g) * u), g = Y[p][i], u = Y[p][I + i], silu(x) =
// x / (1 + exp(-x)), rounded once from the float64 value. Four consecutive i
// per thread (float4 reads of both halves, one 8-byte store); I % 4 == 0.
__global__ __launch_bounds__(256) void swiglu_kernel(const float *__restrict__ Y, int64_t rows,
                                                     int I, uint16_t *__restrict__ H) {
  const int q = I >> 2;                         // float4 groups per half row
  const int64_t total = rows * q;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = g / q;
    const int c = (int)(g - p * q) * 4;
    const float *yr = Y + p * (2 * (int64_t)I);
    const float4 gv = *reinterpret_cast<const float4 *>(yr + c);
    const float4 uv = *reinterpret_cast<const float4 *>(yr + I + c);
    const float ga[4] = {gv.x, gv.y, gv.z, gv.w}, ua[4] = {uv.x, uv.y, uv.z, uv.w};
    uint16_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = swiglu_bf16(ga[i], ua[i]);
    *reinterpret_cast<uint2 *>(H + p * I + c) =
        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  }
}

hipError_t launch_swiglu(const float *Y, int32_t rows, int32_t I, uint16_t *H, hipStream_t s) {
  const int64_t total = (int64_t)rows * (I / 4);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid), dim3(256), 0, s, Y, (int64_t)rows, I, H);
  return hipGetLastError();
}

}  // namespace gnf4
