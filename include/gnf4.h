/* gnf4.h -- grouped 4-bit mixture-of-experts GEMM for AMD MI355X (gfx950).
 *
 * The operation. A mixture-of-experts layer whose experts are stored 4-bit
 * packed: one call computes every active expert's matmul directly on the
 * packed bytes, decoding the 16-entry codebook in registers, without writing
 * dequantized bf16 weights anywhere (Jordan Anderson,
 * jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
 * first bullet; GitHub profile pjordanandrsn, grouped-nf4-gemm bullets). The
 * packed bytes are consumed as stored: NF4 on the bitsandbytes layout and
 * MXFP4 on a checkpoint's released bytes (same section, third bullet).
 *
 * A layer step is three calls on one stream:
 *   gnf4_route          top-k expert ids -> per-expert row segments
 *   gnf4_grouped_gemm   Y[p] = A[p] . W[expert(p)]^T for every routed row p
 *   gnf4_combine        out[t] = sum_j w[t,j] * Y[inv[t*k+j]]
 * (gnf4_route_grouped_gemm runs the first two as one call, one launch for a
 * single token) and a whole FFN layer adds the steps either side of the GEMM:
 *   gnf4_route_logits   router logits -> top-k ids and weights, then route
 *   gnf4_grouped_gemm_swiglu   gate_up projection (gathered token rows)
 *                       with H = silu(gate) * up, bf16, as its epilogue
 *                       (or gnf4_grouped_gemm, then gnf4_swiglu)
 *   gnf4_grouped_gemm   down projection (rows of H, routed order)
 *   gnf4_combine        (gnf4_grouped_gemm_combine: the last two as one call,
 *                       one launch for a single token)
 * and the backward pass through the frozen experts is, per projection:
 *   gnf4_grouped_gemm_dx   dA[p] = dY[p] . W'[e]    (one launch)
 *   gnf4_combine           with unit weights: dX[t] = sum_j dA[inv[t*k+j]]
 *                          for a projection whose rows were gathered
 * and a layer whose experts stay in host RAM streams them through an HBM
 * cache before the route: gnf4_expert_cache_stage, gnf4_expert_cache_fill.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never frees or retains them and allocates no device memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronize with the host.
 *  - Arguments are validated on the host before anything is launched; a
 *    failure returns a non-zero status, launches nothing and leaves the
 *    reason in gnf4_last_error() (per calling thread).
 *  - Two calls that write the same outputs race unless ordered by the
 *    caller's streams; the library keeps no state between calls apart from
 *    the per-thread error text.
 *
 * Weight layout. The experts of a layer are one fused [E, N, K] parameter
 * (Jordan Anderson, jordananderson.work, experts4bit-qlora entry, first
 * bullet) computing Y = X . W[e]^T (N output features, K input features):
 *   codes   uint8 [E][N][K/2], two 4-bit codes per byte along K.
 *           NF4 / NF4_DQ: element 2i in the HIGH nibble (bitsandbytes order).
 *           MXFP4:        element 2i in the LOW nibble (gpt-oss byte order).
 *   scales  NF4:    float32 absmax [E][N][K/64]
 *           NF4_DQ: int8 q8 [E][N][K/64]; absmax = fp32(q8 * scales2[b/256])
 *                   where b is the flat block index e*N*(K/64) + n*(K/64) + j
 *           MXFP4:  uint8 e8m0 [E][N][K/32]; scale 2^(s-127), s = 255 is NaN
 *   scales2 NF4_DQ only: float32 [ceil(E*N*(K/64)/256)]; else NULL.
 * NF4 codebook: the 16 NormalFloat-4 values (QLoRA construction) in float32,
 * readable with gnf4_nf4_codebook().
 */
#ifndef GNF4_H
#define GNF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *gnf4_stream_t; /* identical to hipStream_t */

typedef enum {
  GNF4_OK = 0,
  GNF4_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment */
  GNF4_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle */
  GNF4_ERR_WORKSPACE = 3,   /* the workspace given is smaller than the call needs */
  GNF4_ERR_DEVICE = 4       /* a HIP call or launch failed */
} gnf4_status;

typedef enum { GNF4_NF4 = 0, GNF4_NF4_DQ = 1, GNF4_MXFP4 = 2 } gnf4_format;

typedef struct {
  int32_t format;         /* gnf4_format */
  int32_t E, N, K;        /* experts, output features, input features */
  const uint8_t *codes;   /* [E][N][K/2], 16-byte aligned */
  const void *scales;     /* see the layout above */
  const float *scales2;   /* NF4_DQ only, else NULL */
} gnf4_weights;

/* Limits checked on the host. Besides these, one expert's packed codes
 * (N * K / 2 bytes) must stay below 4 GiB and all experts' below 1 TiB
 * (GNF4_ERR_UNSUPPORTED otherwise). */
#define GNF4_MAX_EXPERTS 1024
#define GNF4_MAX_K 65536
#define GNF4_MAX_N 262144

/* gnf4_route_workspace_bytes -- device bytes of workspace that gnf4_route
 * (and every call that routes: gnf4_route_logits, gnf4_route_grouped_gemm,
 * gnf4_route_logits_grouped_gemm) needs for T tokens with k ids each over E
 * experts: 0 up to T*k = 1024 (one workgroup routes them), else about
 * 4 * (E + 1) bytes per chunk of 1024 or more consecutive assignments (at
 * most about 256 chunks), rounded up to 256 bytes; 0 for invalid arguments.
 * 128 experts at T*k = 32768: 16,640 bytes. */
size_t gnf4_route_workspace_bytes(int32_t T, int32_t k, int32_t E);

/* gnf4_route -- group the flat top-k assignments f = t*k + j by expert.
 *
 * Computes a counting sort of topk_ids (int32 [T][k], row-major):
 *   counts[e]   number of assignments with id e                   int32 [E]
 *   offsets     exclusive prefix sum of counts, offsets[E] = total int32 [E+1]
 *   perm[p]     for p in [offsets[e], offsets[e+1]): the flat indices f with
 *               id e in ascending f (stable); -1 for p >= offsets[E]  int32 [T*k]
 *   inv[f]      the p with perm[p] = f; -1 for a dropped assignment int32 [T*k]
 *   active      ascending experts with counts > 0, then -1        int32 [E]
 *   n_active    number of active experts                          int32 [1]
 *   bad_id_flag set to 1 if any id lies outside [0, E) (such entries are
 *               dropped), else 0                                   int32 [1]
 * The result is deterministic (no order-dependent atomics). T = 0 is a valid
 * no-op apart from zeroing counts/offsets/n_active/bad_id_flag and filling
 * active with -1. Duplicate ids within a token are routed as separate rows.
 * workspace: caller-owned device memory of workspace_bytes >=
 * gnf4_route_workspace_bytes(T, k, E), 16-byte aligned (NULL when that is
 * 0); its contents on entry do not matter and on return are unspecified;
 * GNF4_ERR_WORKSPACE when workspace_bytes is smaller. Up to T*k = 1024 the
 * route is one launch; above, three (chunk histograms, one scan over them,
 * chunk scatters), each a multi-workgroup launch except the scan.
 * Limits: 1 <= E <= GNF4_MAX_EXPERTS, 1 <= k <= 64, 0 <= T, T*k < 2^31.
 * The pages describe the kernel running one launch for all active experts
 * behind a real router (section cited at the top); the grouping itself is
 * this library's reading. */
gnf4_status gnf4_route(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                       int32_t *active, int32_t *n_active, int32_t *bad_id_flag,
                       void *workspace, size_t workspace_bytes, gnf4_stream_t stream);

/* gnf4_route_noalloc -- gnf4_route for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results without the workspace
 * pair. The route's workspace is a file-scope 1 MiB device array, one per
 * GPU, held until the process ends; its address is looked up once per
 * device (hipGetSymbolAddress with that device current) on the first call
 * there, and nothing is allocated. That covers every route with
 * E <= 1023, and E = 1024 up to T*k = 261,120; a larger need returns
 * GNF4_ERR_WORKSPACE with the sizes in gnf4_last_error(). All calls on one GPU share the
 * array: two that overlap on that GPU (unordered streams) race and may give
 * wrong results; calls ordered on the caller's streams do not interfere.
 * Nothing in the array needs to start at any value. */
gnf4_status gnf4_route_noalloc(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                               int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv,
                               int32_t *active, int32_t *n_active, int32_t *bad_id_flag,
                               gnf4_stream_t stream);

/* gnf4_grouped_gemm -- one launch for all active experts.
 *
 * For every expert e and routed row p in [offsets[e], offsets[e+1]):
 *   Y[p][n] = sum_k A[p][k] * W'[e][n][k]       (float32 accumulate)
 * A[p] = X[perm[p] / k] when gather = 1 (X is bf16 [T][K], the token
 * activations) and A[p] = X[p] when gather = 0 (X is bf16 [T*k][K], already
 * in routed order, e.g. the second projection's input). Rows p >= offsets[E]
 * of Y are not written. W' is the packed weight decoded in registers: NF4 as
 * the bf16 operand values bf16(s * codebook) with fp32(absmax * (1/s))
 * applied to each 64-value partial sum (gnf4_nf4_codebook_bf16 gives the
 * values and s), MXFP4 exactly (e2m1 * 2^(e8m0 - 127)). The route outputs
 * (offsets, perm, active, n_active) must come from gnf4_route with the same
 * T, k, E.
 * X: uint16 bf16 bits, 16-byte aligned. Y: float32 [T*k][N], 16-byte aligned.
 * The path (wavefront GEMV for decode, LDS-staged bf16 MFMA for prefill) is
 * chosen from T*k on the host; nothing is read back from the device. */
gnf4_status gnf4_grouped_gemm(const gnf4_weights *w, const uint16_t *X, int32_t gather,
                              const int32_t *offsets, const int32_t *perm,
                              const int32_t *active, const int32_t *n_active,
                              int32_t T, int32_t k, float *Y, gnf4_stream_t stream);

/* gnf4_route_grouped_gemm -- gnf4_route followed by the first projection
 * (rows gathered from the token activations, gather = 1), as one call:
 *   gnf4_route(topk_ids, T, k, w->E, counts, ..., bad_id_flag)
 *   gnf4_grouped_gemm(w, X, 1, offsets, perm, active, n_active, T, k, Y)
 * or, with H given instead of Y, gnf4_grouped_gemm_swiglu. Every output
 * (the routing arrays and Y or H) is bit-identical to those two calls. For
 * a single token (T == 1, the decode step) it is one launch: each
 * workgroup of the one-token GEMV derives the routing from the k ids and
 * the first workgroup writes the routing outputs, which saves a launch and
 * a dependent round trip per layer step (the pages put per-token time at
 * bytes over bandwidth plus a fixed cost: Jordan Anderson,
 * jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
 * experts-4bit", demonstration paragraph of the first bullet). Otherwise
 * the two launches of the separate calls. Exactly one of Y, H is non-NULL
 * (for T > 0). Arguments (the workspace is gnf4_route's), limits and errors
 * as the two calls. */
gnf4_status gnf4_route_grouped_gemm(const int32_t *topk_ids, int32_t T, int32_t k,
                                    int32_t *counts, int32_t *offsets, int32_t *perm,
                                    int32_t *inv, int32_t *active, int32_t *n_active,
                                    int32_t *bad_id_flag, void *workspace,
                                    size_t workspace_bytes, const gnf4_weights *w,
                                    const uint16_t *X, float *Y, uint16_t *H,
                                    gnf4_stream_t stream);

/* gnf4_route_logits_grouped_gemm -- gnf4_route_logits followed by the first
 * projection (gather = 1), as one call: the router's top-k ids and softmax
 * weights, the routing arrays and Y (or H with the SwiGLU epilogue) are
 * bit-identical to gnf4_route_logits then gnf4_grouped_gemm (or
 * gnf4_grouped_gemm_swiglu). For a single token (T == 1) it is one launch:
 * every workgroup of the one-token GEMV forms the top-k from the logits
 * [1][E] and the routing from it; the first writes topk_ids, topk_w and the
 * routing outputs. Otherwise the separate launches. Exactly one of Y, H is
 * non-NULL (for T > 0). Arguments, limits and errors as the calls it
 * replaces (k <= E). */
gnf4_status gnf4_route_logits_grouped_gemm(const float *logits, int32_t T, int32_t k,
                                           int32_t *topk_ids, float *topk_w, int32_t *counts,
                                           int32_t *offsets, int32_t *perm, int32_t *inv,
                                           int32_t *active, int32_t *n_active,
                                           int32_t *bad_id_flag, void *workspace,
                                           size_t workspace_bytes, const gnf4_weights *w,
                                           const uint16_t *X, float *Y, uint16_t *H,
                                           gnf4_stream_t stream);

/* gnf4_grouped_gemm_swiglu -- the first projection with the SwiGLU step as
 * its epilogue: for every routed row p and i < N/2,
 *   H[p][i] = bf16(silu(Y[p][i]) * Y[p][N/2 + i])
 * where Y is what gnf4_grouped_gemm computes for the same arguments (same
 * kernels, same float32 values) and the rounding is gnf4_swiglu's, so the
 * result equals gnf4_grouped_gemm followed by gnf4_swiglu bit for bit,
 * without writing or reading the float32 Y. The weight's rows [0, N/2) are
 * the gate, [N/2, N) the up projection; N must be even. H uint16 bf16 bits
 * [T*k][N/2] (2-byte aligned), the down projection's input in routed order.
 * Other arguments, limits and errors as gnf4_grouped_gemm. Not described on
 * the pages (reading of gnf4_swiglu). */
gnf4_status gnf4_grouped_gemm_swiglu(const gnf4_weights *w, const uint16_t *X, int32_t gather,
                                     const int32_t *offsets, const int32_t *perm,
                                     const int32_t *active, const int32_t *n_active,
                                     int32_t T, int32_t k, uint16_t *H, gnf4_stream_t stream);

/* gnf4_grouped_gemm_dx -- input gradient of gnf4_grouped_gemm through the
 * frozen packed weights, one launch for all active experts, the codes and
 * scales read as stored (Jordan Anderson, jordananderson-pages.pages.dev,
 * section "grouped-nf4-gemm & experts-4bit", fourth bullet: a differentiable
 * kernel whose backward is one launch on the packed 4-bit weights). For
 * expert e and every routed row p in [offsets[e], offsets[e+1]),
 *   dA[p][j] = sum_{n<N} dY[p][n] * W'[e][n][j]         (j < K)
 * with W' the dequantized weights (exactly as gnf4_dequant decodes them).
 * dY uint16 bf16 bits [T*k][N] and dA float32 [T*k][K], both in the routed
 * order of gnf4_route (rows of Y in the forward call), both 16-byte aligned;
 * N % 8 == 0. The weights are read only (no weight gradient: the experts are
 * frozen). Rows p >= offsets[E] (dropped assignments) are not written.
 * Arithmetic: float32 accumulation of bf16 products; each dequantized NF4 /
 * NF4_DQ weight w (float32) enters as bf16(w) plus bf16(w - bf16(w)), which
 * leaves out less than 2^-16 of |w|; MXFP4 weights are exact in bf16.
 * For the gathered first projection the gradient of token t's activation row
 * is the sum over its k routed copies: gnf4_combine(dA, inv, ones, T, k, K).
 * Errors: INVALID_ARG for bad weights (as gnf4_grouped_gemm), k outside
 * [1, 64], T < 0, N % 8 != 0, NULL or misaligned pointers; UNSUPPORTED when
 * dY reaches 4 GiB (T*k*N*2 bytes, 32-bit buffer offsets); T = 0 is a
 * no-op. */
gnf4_status gnf4_grouped_gemm_dx(const gnf4_weights *w, const uint16_t *dY,
                                 const int32_t *offsets, int32_t T, int32_t k, float *dA,
                                 gnf4_stream_t stream);

/* gnf4_grouped_gemm_combine -- the second projection (rows already in
 * routed order, gather = 0) followed by the combine, as one call:
 *   gnf4_grouped_gemm(w, X, 0, offsets, perm, active, n_active, T, k, Y)
 *   gnf4_combine(Y, inv, topk_w, T, k, N, out)
 * out is bit-identical to those two calls. For a single token (T == 1) with
 * K <= 8192 it is one launch that never writes Y: each output row block
 * forms the products of every routed copy (the same float32 values as the
 * GEMM) and adds them with the combine's operations in its order
 * (j ascending, dropped copies skipped), which saves a launch and the Y
 * round trip per layer step (fixed per-token cost: Jordan Anderson,
 * jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
 * experts-4bit", demonstration paragraph of the first bullet). Otherwise
 * the two launches, with Y float32 [T*k][N] (16-byte aligned) as their
 * intermediate; Y may be NULL when the one-launch path applies. out float32
 * [T][N] (16-byte aligned); N % 4 == 0. Other arguments, limits and errors
 * as the two calls. */
gnf4_status gnf4_grouped_gemm_combine(const gnf4_weights *w, const uint16_t *X,
                                      const int32_t *offsets, const int32_t *perm,
                                      const int32_t *inv, const int32_t *active,
                                      const int32_t *n_active, const float *topk_w, int32_t T,
                                      int32_t k, float *Y, float *out, gnf4_stream_t stream);

/* gnf4_combine -- weighted top-k combine back to tokens.
 *   out[t][n] = sum_{j=0..k-1} topk_w[t][j] * Y[inv[t*k+j]][n]
 * float32, j ascending, an assignment with inv = -1 contributes nothing.
 * The pages run the grouped kernel inside a mixture-of-experts layer behind
 * a real router (section cited at the top, demonstration paragraph) but do
 * not describe the step back to tokens; this is this library's reading, the
 * weighted sum of a token's k expert outputs that defines such a layer, in
 * a fixed order so that the result is deterministic.
 * Y float32 [T*k][N] (16-byte aligned), inv int32 [T*k], topk_w float32
 * [T][k], out float32 [T][N] (16-byte aligned). N % 4 == 0. */
gnf4_status gnf4_combine(const float *Y, const int32_t *inv, const float *topk_w,
                         int32_t T, int32_t k, int32_t N, float *out, gnf4_stream_t stream);

/* gnf4_route_logits -- the router's choice, then gnf4_route.
 *
 * The pages put the fused kernel behind a real router (section cited at the
 * top, demonstration paragraph) without describing it; the definition used
 * is that of the public models the workloads are shaped after. For each
 * token t of logits float32 [T][E] (row-major):
 *   topk_ids[t][j], j < k   the k largest logits in descending order, ties
 *                           to the lower expert id; NaN ranks below every
 *                           number (chosen only when fewer than k numbers
 *                           remain, in ascending id)           int32 [T][k]
 *   topk_w[t][j]            float32 of the softmax of the k chosen logits,
 *                           computed in float64 with the largest chosen
 *                           logit subtracted and the exponentials summed in
 *                           rank order                         float32 [T][k]
 * then gnf4_route(topk_ids, T, k, E, ...) with the same outputs and
 * meaning. Limits: 1 <= k <= 64, k <= E <= GNF4_MAX_EXPERTS, 0 <= T,
 * T*k < 2^31. T = 0 behaves as gnf4_route with T = 0. */
gnf4_status gnf4_route_logits(const float *logits, int32_t T, int32_t k, int32_t E,
                              int32_t *topk_ids, float *topk_w, int32_t *counts,
                              int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *active,
                              int32_t *n_active, int32_t *bad_id_flag, void *workspace,
                              size_t workspace_bytes, gnf4_stream_t stream);

/* gnf4_swiglu -- the activation between the two projections.
 *   H[p][i] = bf16(silu(Y[p][i]) * Y[p][I + i]),  silu(x) = x / (1 + exp(-x))
 * for p < rows, i < I: Y float32 [rows][2I] is the gate_up output with the
 * gate in columns [0, I) and up in [I, 2I); H (uint16 bf16 bits [rows][I])
 * is the input of the down projection in the same routed order (gather = 0).
 * The product is formed in float64 and rounded once to bf16 (nearest, ties
 * to even; NaN gives 0x7FC0), so H does not depend on how the GPU orders
 * float32 operations. Rows of Y past the routed total (dropped ids) hold
 * unspecified values, and so do the matching rows of H.
 * I % 4 == 0, Y 16-byte and H 8-byte aligned. Not described on the pages
 * (same reading as gnf4_route_logits). */
gnf4_status gnf4_swiglu(const float *Y, int32_t rows, int32_t I, uint16_t *H,
                        gnf4_stream_t stream);

/* gnf4_dequant -- decode expert e of w to float32 out [N][K] (test aid).
 * NF4: fp32(c[q] * absmax); NF4_DQ: fp32(c[q] * fp32(q8 * scale2));
 * MXFP4: e2m1(q) * 2^(s-127), exact (s = 255 gives NaN). The pages name the
 * formats (NF4 on the bitsandbytes layout, MXFP4 as e2m1 codes with e8m0
 * scales: section cited at the top, first and third bullets) but print no
 * decode rule; this is the reading of the weight layout above (QLoRA
 * NormalFloat-4 table times the block absmax; OCP MX e2m1 times 2^(s-127)).
 * The GEMMs never write this decode anywhere: it lets tests check the
 * device's decode bit for bit against the CPU oracle. */
gnf4_status gnf4_dequant(const gnf4_weights *w, int32_t e, float *out, gnf4_stream_t stream);

/* gnf4_dequant_experts_bf16 -- the decode step of the dequantize-then-matmul
 * path the pages measure the fused kernel against (section cited at the
 * top: grouped decode faster than a dequant path; the comparison path is
 * this library's reading of it). For slot s < min(*count, max_experts)
 * with e = experts[s] in [0, E):
 *   out[s][n][k] = bf16(W'[e][n][k])   (nearest even; NaN -> 0x7FC0)
 * where W' is gnf4_dequant's float32 value. experts and count are device
 * int32 (e.g. gnf4_route's active and n_active, so nothing is read back);
 * slots at or past *count, or with an id outside [0, E), are left as they
 * are. out uint16 bf16 bits [max_experts][N][K], 16-byte aligned.
 * 0 <= max_experts <= E. */
gnf4_status gnf4_dequant_experts_bf16(const gnf4_weights *w, const int32_t *experts,
                                      const int32_t *count, int32_t max_experts,
                                      uint16_t *out, gnf4_stream_t stream);

/* gnf4_quantize -- pack float32 weights W [rows][K] (rows = E*N) into the
 * layout above: NF4 / NF4_DQ block 64 with nearest-code rounding (ties to
 * the lower code, decided in float64), NF4_DQ with linear int8 absmax and
 * one float32 scale per 256 blocks, MXFP4 by the OCP MX rule (shared
 * exponent floor(log2 amax) - 2, round to nearest even, saturate at 6).
 * W must be finite. codes uint8 [rows][K/2]; scales as the format says;
 * scales2 float32 [ceil(rows*(K/64)/256)] for NF4_DQ, else ignored. */
gnf4_status gnf4_quantize(int32_t format, const float *W, int32_t rows, int32_t K,
                          uint8_t *codes, void *scales, float *scales2, gnf4_stream_t stream);

/* Expert streaming from host RAM (Jordan Anderson,
 * jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit":
 * the demonstration paragraph of the first bullet streams the 4-bit experts
 * from pinned host memory over PCIe with the fused kernel as the only expert
 * compute, per-token time being streamed bytes over link speed plus a fixed
 * per-host cost; the experts4bit-qlora bullets keep hot experts resident and
 * stream the cold tail). A layer's packed experts stay in pinned host memory
 * (host_w, E experts) and S of them at a time in an HBM cache laid out as an
 * ordinary weight tensor with E = S (cache_w). A decode step is:
 *   gnf4_expert_cache_stage   ids -> slot ids, residency update, copy list
 *   gnf4_expert_cache_fill    copy the listed experts host -> slots
 *   gnf4_route / gnf4_route_grouped_gemm ... on the slot ids over S "experts"
 *   (and the grouped GEMM on cache_w), exactly as on the resident layer: the
 *   outputs equal those of the resident layer bit for bit, since every routed
 *   row meets the same expert bytes and the combine sums in the same order.
 * The residency state is a caller-owned device int32 array of
 * gnf4_expert_cache_state_words(E, S) words:
 *   [0] steps staged since the reset
 *   [1, 1+E)          slot of expert e, -1 if not resident
 *   [1+E, 1+E+S)      expert in slot s, -1 if empty
 *   [1+E+S, 1+E+2S)   last step that used slot s, 0 if never
 * Limits: 1 <= S <= E <= GNF4_MAX_EXPERTS. Calls that share one state must be
 * ordered on the caller's streams. */

/* Words of the state array (0 for invalid E, S). */
size_t gnf4_expert_cache_state_words(int32_t E, int32_t S);

/* Words of a copy list for T tokens with k ids each: 1 + 2 * min(T*k, E, S)
 * (0 for invalid arguments). */
size_t gnf4_expert_cache_copies_words(int32_t T, int32_t k, int32_t E, int32_t S);

/* gnf4_expert_cache_reset -- empty cache: step 0, no expert resident. One
 * small fill kernel (no memset node, so it may be graph-captured). */
gnf4_status gnf4_expert_cache_reset(int32_t *state, int32_t E, int32_t S, gnf4_stream_t stream);

/* gnf4_expert_cache_stage -- one step's residency decision, on the GPU.
 * The experts the step needs are the distinct ids of topk_ids [T][k] in
 * [0, E). A needed expert already in a slot is a hit and keeps its slot. The
 * misses, taken in ascending expert order, go to the slots no hit uses:
 * empty slots first, then least recently used (oldest last use), ties to the
 * lower slot; an evicted expert stops being resident. Every used slot is
 * stamped with the step. Outputs (device int32):
 *   slot_ids [T][k]   the slot of each id's expert; -1 for ids outside
 *                     [0, E), which gnf4_route then drops and flags;
 *   copies            [0] = number of misses m, then m pairs (expert, slot)
 *                     in ascending expert order; gnf4_expert_cache_copies_words
 *                     words.
 * UNSUPPORTED when S < min(E, T*k) (the step's distinct experts might not
 * fit). T = 0 still advances the step. */
gnf4_status gnf4_expert_cache_stage(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                    int32_t S, int32_t *state, int32_t *slot_ids, int32_t *copies,
                                    gnf4_stream_t stream);

/* gnf4_expert_cache_fill -- copy the packed bytes of every (expert, slot)
 * pair of copies from host_w into cache_w: codes, scales and, for NF4_DQ,
 * the expert's second-level scales (its N*K/64 blocks must be whole groups
 * of 256). The GPU reads host_w over the host link; its arrays must be
 * pinned host memory (hipHostMalloc, or torch pin_memory) or device memory,
 * anything else is INVALID_ARG. Same format, N and K on both sides,
 * cache_w->E = S <= host_w->E, every per-expert segment a multiple of 16
 * bytes and every array 16-byte aligned. The launch covers max_copies pairs
 * (pass 1 + 2*max_copies words of copies; usually min(T*k, E, S)); pairs past
 * copies[0], or with an expert or slot out of range, copy nothing. */
gnf4_status gnf4_expert_cache_fill(const gnf4_weights *host_w, const gnf4_weights *cache_w,
                                   const int32_t *copies, int32_t max_copies,
                                   gnf4_stream_t stream);

/* gnf4_read_probe -- the achievable HBM read rate of the device, the
 * ceiling the decode GEMV's packed-weight bandwidth is compared with (the
 * pages measure the ceilings they report against rather than assume them:
 * GitHub profile pjordanandrsn, NVMe-tier bullets; Jordan Anderson,
 * jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
 * demonstration paragraph). Reads bytes [0, nbytes) of the device buffer src
 * once with 16-byte non-temporal loads, eight in flight per thread, in
 * `workgroups` workgroups of 256 threads (0: eight per compute unit; fewer
 * if the buffer is small), and computes nothing from them but an XOR fold;
 * sink (one device word) is written only if the fold equals one fixed
 * constant. Over a buffer larger than the 256 MB Infinity Cache the call also
 * evicts that cache. src 16-byte aligned, nbytes % 16 == 0 (0 is a no-op);
 * INVALID_ARG otherwise. */
gnf4_status gnf4_read_probe(const void *src, size_t nbytes, int32_t workgroups, uint32_t *sink,
                            gnf4_stream_t stream);

/* The 16 NF4 codebook values used by every kernel (host copy, float32). */
void gnf4_nf4_codebook(float out[16]);

/* The bf16 operand values of the NF4 contractions (forward GEMV and MFMA
 * paths): out[q] = bf16 bits of fp32(s * c[q]) (nearest even), and *scale =
 * s, the float32 in [1, 2) minimizing the mean over q of
 * (bf16(s * c[q]) / s - c[q])^2; the kernels scale each 64-value partial
 * sum by fp32(absmax * fp32(1/s)). Reading of the pages' in-register
 * codebook decode (section cited at the top): a bf16 operand of the
 * codebook scaled so that its rounding error is smallest. Either pointer
 * may be NULL. */
void gnf4_nf4_codebook_bf16(uint16_t out[16], float *scale);

/* Thread-local text describing the last non-OK status ("" if none). */
const char *gnf4_last_error(void);

/* Source revision and target of the compiled library, e.g. "gnf4 1a2b3c4 gfx950". */
const char *gnf4_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* GNF4_H */
