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

// One wave per token (topk_row in common.h): four tokens per workgroup.
template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                           // whole wave
  int id;
  float wt;
  topk_row<NPL>(logits + (int64_t)t * E, E, k, lane, id, wt);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = id;
    w[(int64_t)t * k + lane] = wt;
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
