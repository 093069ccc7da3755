/*
 * nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 block-scaled linear and
 * Mixture-of-Experts grouped GEMM library (libnvfp4.so).
 *
 * What is computed.  The block-scaled GEMM
 *     y = (x * scale_a * gsa) @ (w * scale_b * gsb)^T
 * as stated on page "nvfp4-megamoe-kernel, commit 1121cd7 -
 * single_shot_inference.py" (the note on the weight-dequant global scale):
 * every operand element is an E2M1 value times its FP8-E4M3 block scale times
 * one fp32 global scale per tensor.  For weights the global scale is
 * weight_scale_2 (page "commit efe63ca - single_shot_inference.py", notes on
 * weight_scale_2 and on input_scale).  For NVFP4 activations it is the
 * activation global scale gs = amax / (6 * 448), used as it is, never
 * inverted (page "commit 4c6464e - vllm", note on the activation global
 * scale).  The product of the two global scales is applied exactly once.
 *
 * Formats (all entry points):
 *   E2M1 ("fp4"): 2 codes per byte, element 2j in bits 0-3, 2j+1 in bits 4-7;
 *                 values {0, .5, 1, 1.5, 2, 3, 4, 6} with sign bit 3.
 *   E4M3FN block scale: one byte per 16 consecutive K elements of a row.
 *   Weights [N, K/2] bytes + scales [N, K/16] bytes, K contiguous ("N-major",
 *   page "commit efe63ca", note on the checkpoint layout; scales are not
 *   transposed, same page, note on scale assembly).
 *   bf16 tensors are row-major with the last dimension contiguous.
 *   K is always the logical element count, not the packed byte count
 *   (page "commit 4c6464e", note on K being the hidden size).
 *
 * Pointers are DEVICE pointers unless marked "host".  `stream` is a
 * hipStream_t (NULL = the default stream).  Every call only enqueues work on
 * `stream` and returns; it never synchronises, never allocates or frees device
 * memory, and keeps no state between calls (calls on different streams may
 * run concurrently as long as their buffers do not overlap; a call can be
 * captured into a HIP graph).  The caller owns every buffer.
 *
 * Constraints (checked on the host before any launch):
 *   K and every reduction length % 256 == 0; output widths % 16 == 0;
 *   device pointers 16-byte aligned (scale and gs pointers 4-byte aligned);
 *   sizes positive and below 2^31 elements per dimension, except the row or
 *   token count (M, T), which may be 0: the other sizes are still checked,
 *   nothing is written (but the gs of a quantizer with compute_gs) and NULL
 *   pointers are accepted.
 * Errors: a negative NVFP4_ERR_* code is returned and nothing is launched
 * when a check fails; NVFP4_ERR_LAUNCH reports a HIP launch error.  Values
 * inside device buffers (expert ids, NaN scales) are not checked on the host:
 * an expert id outside [0, E) makes that (token, expert) pair contribute
 * zero; it can never cause an out-of-bounds access.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = -2,     /* a size is out of range or not a required multiple */
  NVFP4_ERR_ALIGN = -3,     /* a pointer is not aligned as required */
  NVFP4_ERR_WORKSPACE = -4, /* workspace missing or smaller than the size function says */
  NVFP4_ERR_LAUNCH = -5,    /* a kernel launch failed (hipGetLastError) */
  NVFP4_ERR_ARG = -6,       /* an incompatible combination of optional arguments */
  NVFP4_ERR_SCRATCH = -7    /* nvfp4_moe_grouped_noalloc: the call needs more scratch than it holds */
};

/* Host: a static, human-readable description of a status code. */
const char* nvfp4_status_string(int status);

/* Host: ABI version of this header (incremented on incompatible changes). */
int nvfp4_abi_version(void);
#define NVFP4_ABI_VERSION 2

/*
 * nvfp4_quantize_act - quantize bf16 activations to NVFP4.
 * Page "commit 4c6464e - vllm": the activation quantizer
 * (quantize_activation_nvfp4, named in the note on the custom-op GEMM) and
 * the activation global scale gs = amax / (6 * 448) (note on the activation
 * global scale).  Per 16-element block of a row:
 *     scale byte = RNE_E4M3(amax_blk / (6 * gs)), saturating at 448;
 *     code       = RNE_E2M1(x * (1 / (E4M3(byte) * gs))), saturating at 6;
 * each step one IEEE fp32 operation in that order (so the result is
 * reproducible bit for bit); gs == 0 gives all-zero codes and scales.
 *   x_bf16     [M, K] bf16 input.
 *   gs         device fp32 scalar: output when compute_gs != 0 (written with
 *              max|x| / 2688 computed on the device), input otherwise.
 *   x_fp4      [M, K/2] output codes; x_sf [M, K/16] output scale bytes.
 *   workspace  device scratch of nvfp4_quantize_act_workspace_size(M, K)
 *              bytes, 16-byte aligned, when compute_gs != 0 (per-workgroup
 *              maxima of |x|; undefined after the call); may be NULL otherwise.
 * M == 0 writes nothing but gs, which compute_gs sets to 0 (no elements);
 * x_bf16, x_fp4, x_sf and workspace may then be NULL.
 * Requires K % 16 == 0 (K % 256 == 0 if the result feeds nvfp4_linear or
 * nvfp4_moe_grouped).
 */
size_t nvfp4_quantize_act_workspace_size(int64_t M, int64_t K);
int nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, float* gs, int compute_gs,
                       uint8_t* x_fp4, uint8_t* x_sf, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_rmsnorm_quantize - RMSNorm fused with nvfp4_quantize_act (page
 * "commit 1121cd7 - single_shot_inference.py", the notes on the A/B
 * comparison of the fused "P4" RMSNorm + quantization against the unfused
 * path): the result is exactly that of RMSNorm followed by the quantizer.
 *   RMSNorm of each row of x_bf16 [T, K] with weight w_bf16 [K]:
 *     r = fp32(1 / sqrt(sum_k x^2 / K + eps))   (sum, root and quotient in fp64)
 *     y = bf16_RNE(fp32(fp32(x * r) * w))
 *   y_bf16 [T, K]: optional output of y (NULL: not written).
 *   gs, compute_gs, x_fp4 [T, K/2], x_sf [T, K/16]: as nvfp4_quantize_act,
 *   applied to y.
 *   workspace: nvfp4_rmsnorm_quantize_workspace_size(T) bytes (r per row and
 *   the per-workgroup maxima of |y|; scratch, undefined after the call).
 * T == 0 writes nothing but gs, which compute_gs sets to 0 (no elements);
 * every other pointer may then be NULL.
 * Requires K % 16 == 0 (K % 256 == 0 to feed nvfp4_linear), eps > 0 and
 * finite (NVFP4_ERR_ARG otherwise), 16-byte aligned tensors.
 */
size_t nvfp4_rmsnorm_quantize_workspace_size(int64_t T);
int nvfp4_rmsnorm_quantize(const void* x_bf16, const void* w_bf16, float eps, int64_t T, int64_t K, void* y_bf16,
                           float* gs, int compute_gs, uint8_t* x_fp4, uint8_t* x_sf, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * nvfp4_linear - dense NVFP4 linear, y[M, N] = x[M, K] @ W[N, K]^T, bf16 out,
 * fp32 accumulation (page "commit 1121cd7", the GEMM statement in the note on
 * the weight-dequant global scale; the NVFP4 linear layer of page
 * "commit efe63ca", note on weight_scale_2).
 *   Activations, one of:
 *     x_bf16 [M, K] bf16 (then x_fp4, x_sf, gsa must be NULL; scale_a = gsa = 1), or
 *     x_fp4 [M, K/2] + x_sf [M, K/16] + gsa (device fp32 scalar) from nvfp4_quantize_act.
 *   w_fp4 [N, K/2], w_sf [N, K/16]; gsb = device fp32 scalar weight_scale_2.
 *   y_bf16 [M, N] bf16 output, fully overwritten.
 *   workspace: device scratch of nvfp4_linear_workspace_size(M, N, K) bytes
 *   (may be NULL when that size is 0).  Its contents are undefined after the
 *   call; it must not be shared with a concurrently running call.
 */
size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K);
int nvfp4_linear(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa,
                 const uint8_t* w_fp4, const uint8_t* w_sf, const float* gsb,
                 int64_t M, int64_t N, int64_t K, void* y_bf16,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_grouped_linear - NVFP4 grouped linear of the attention output
 * projection wo_a: G groups, y[t, g, :] = x[t, g, :] @ W[g]^T, bf16 out, fp32
 * accumulation (page "commit 4c6464e - vllm": the notes on the BF16 wo_a
 * path, a batched matmul over n_local_groups groups of in_features 4096, and
 * on replacing it with an NVFP4 grouped linear over those groups).
 *   Activations [T, G, K] (token-major, as the [T, G*K] attention output is
 *   laid out), one of:
 *     x_bf16 [T, G, K] bf16 (then x_fp4, x_sf, gsa must be NULL), or
 *     x_fp4 [T, G, K/2] + x_sf [T, G, K/16] + gsa (device fp32 scalar), from
 *     nvfp4_quantize_act on the [T * G, K] view (one global scale).
 *   w_fp4 [G, N, K/2], w_sf [G, N, K/16]; ws2 [G] device fp32, each group's
 *   weight_scale_2.
 *   y_bf16 [T, G, N] bf16 output, fully overwritten.
 *   workspace: device scratch of nvfp4_grouped_linear_workspace_size(T, G, N, K)
 *   bytes, 256-byte aligned (the fp16 copy of bf16 activations, and fp32
 *   partial sums when the call splits K: with few tokens the work is split
 *   along K and the partial sums are added in a fixed order); contents
 *   undefined after the call, not shared with a concurrent call.
 *   Requires K % 256 == 0, N % 16 == 0, 16-byte aligned tensors.
 * Errors: as nvfp4_linear.
 */
size_t nvfp4_grouped_linear_workspace_size(int64_t T, int64_t G, int64_t N, int64_t K);
int nvfp4_grouped_linear(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa,
                         const uint8_t* w_fp4, const uint8_t* w_sf, const float* ws2,
                         int64_t T, int64_t G, int64_t N, int64_t K, void* y_bf16,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_moe_grouped - one Mixture-of-Experts layer with NVFP4 experts.
 * Routed experts (stacked (E, N, K), page "commit efe63ca", note on stacking
 * experts; one weight_scale_2 per expert and layer, same page, note on
 * weight_scale_2) and an optional shared expert (Nvfp4SharedExpert, same
 * note).  For every token t and routed slot j, with e = topk_ids[t, j]:
 *     gate|up = x_t @ W1_e^T          (W1 rows [0, I) = gate, [I, 2I) = up)
 *     h       = silu(gate) * up        (silu(z) = z / (1 + e^-z))
 *     o       = h @ W2_e^T
 *     y_t     = sum_{j=0..topk-1} topk_w[t, j] * o(t, j)  +  o_shared(t)
 * computed as: a stable token->expert permutation with int32 segment offsets
 * (page "commit 4c6464e", note on the custom-op GEMM: int32 expert offsets),
 * a grouped gate/up GEMM with a fused SwiGLU epilogue, a grouped down GEMM
 * that scatters each pair's output row, and a weighted combine in the fixed
 * order j = 0..topk-1 then the shared expert.
 *
 * Activations, one of:
 *   x [T, H] bf16                          (x_fp4, x_sf, a1_gs NULL), or
 *   x_fp4 [T, H/2] + x_sf [T, H/16] + a1_gs (from nvfp4_quantize_act).
 * Hidden activations h:
 *   a2_gs != NULL: h is quantized to NVFP4 with global scale *a2_gs (the
 *                  nvfp4_quantize_act rule with a supplied gs) and the down
 *                  GEMM runs on NVFP4 activations (fully-FP4 path);
 *   a2_gs == NULL: h stays fp32.  If a2_gs_out != NULL it receives
 *                  max|h| / 2688, the calibrated global scale of h for later
 *                  calls (the warm-up calibration of page "commit 4c6464e").
 * Weights: w1 [E, 2I, H/2], w1_sf [E, 2I, H/16], w1_ws2 [E] fp32;
 *          w2 [E, H, I/2],  w2_sf [E, H, I/16],  w2_ws2 [E] fp32;
 *          shared expert s1/s1_sf/s1_ws2[1], s2/s2_sf/s2_ws2[1], all NULL if absent.
 * Routing: topk_ids [T, topk] int32 (distinct ids per token expected),
 *          topk_w [T, topk] fp32 combine weights (applied after the down GEMM).
 * Optional outputs: offsets_out [E + 2] int32 (group starts; offsets_out[E] =
 *          number of routed rows, offsets_out[E+1] = that + T if shared),
 *          perm_out [T*topk + T] int32 (sorted row -> pair id t*topk + j;
 *          shared rows hold T*topk + t).
 * y [T, H] bf16 output, fully overwritten.
 * workspace: nvfp4_moe_workspace_size(...) bytes of device scratch; h_fp4 = 1
 * sizes it for calls with a2_gs != NULL (smaller), 0 for a2_gs == NULL.
 * stage_events: optional host array of NVFP4_MOE_STAGE_EVENTS hipEvent_t
 * (instrumentation for timing single kernels), recorded on `stream`:
 *   [0] permute [1] gate/up GEMM, groups of > 4 rows [2] gate/up GEMM, the
 *   other groups [3] calibration and conversion of h (fp32 h only) [4] down
 *   GEMM, groups of > 4 rows [5] down GEMM, the other groups [6] combine
 *   [7] end (when the groups average more than 16 rows, [1] and [4] cover
 *   every group and [2] and [5] are empty); event i is recorded before the
 *   work it names, so stage i lasts
 *   from event i to event i + 1.  NULL entries are skipped (each recorded
 *   event costs a few microseconds between two kernels).
 */
#define NVFP4_MOE_STAGE_EVENTS 8
typedef struct nvfp4_moe_args {
  int64_t T, H, I, E, topk;
  const void* x;
  const uint8_t* x_fp4;
  const uint8_t* x_sf;
  const float* a1_gs;
  const float* a2_gs;
  float* a2_gs_out;
  const int32_t* topk_ids;
  const float* topk_w;
  const uint8_t* w1;
  const uint8_t* w1_sf;
  const float* w1_ws2;
  const uint8_t* w2;
  const uint8_t* w2_sf;
  const float* w2_ws2;
  const uint8_t* s1;
  const uint8_t* s1_sf;
  const float* s1_ws2;
  const uint8_t* s2;
  const uint8_t* s2_sf;
  const float* s2_ws2;
  void* workspace;
  size_t workspace_bytes;
  int32_t* offsets_out;
  int32_t* perm_out;
  void* y;
  void** stage_events;
} nvfp4_moe_args;

size_t nvfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                                int has_shared, int h_fp4);
int nvfp4_moe_grouped(const nvfp4_moe_args* args, void* stream);

/*
 * nvfp4_moe_grouped_noalloc - nvfp4_moe_grouped for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, same kernels and the
 * same results, but args->workspace must be NULL and args->workspace_bytes 0
 * (NVFP4_ERR_ARG otherwise): the scratch memory comes from a static device
 * array of NVFP4_MOE_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  Nothing is allocated or freed.
 *   Capacity: a call whose nvfp4_moe_workspace_size(...) exceeds
 *   NVFP4_MOE_NOALLOC_SCRATCH_BYTES returns NVFP4_ERR_SCRATCH before any
 *   launch.  At hidden 7168, intermediate 2048, 384 experts, top-8 that is
 *   any batch of at most 297 tokens with a shared expert and bf16 h, or 545
 *   tokens with NVFP4 h and no shared expert (the 64-token decode step
 *   needs 51.6 MiB, the 128-token prefill chunk 31 MiB).
 *   Device: the array of the current device is used (its address is looked
 *   up on the first call on each device); `stream` must belong to it.
 *   Concurrency: every call on one GPU shares that GPU's array, which keeps
 *   the last call's contents (every call initialises what it reads).  Calls
 *   that overlap in time on one GPU (on different streams, or from
 *   different threads without ordering) race on it: order them on one
 *   stream.  The caller still owns and passes all inputs and outputs.
 */
#define NVFP4_MOE_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int nvfp4_moe_grouped_noalloc(const nvfp4_moe_args* args, void* stream);

/*
 * Router gate (page "commit 1121cd7 - single_shot_inference.py", note on the
 * router gate): the router weight goes through an FP8-E4M3 round trip with one
 * per-tensor scale amax/448 and back to bf16; the router is a plain linear of
 * the activations with it, followed by top-k softmax routing.  Its outputs
 * topk_ids / topk_w are exactly the routing inputs of nvfp4_moe_grouped.
 *
 * nvfp4_router_prepare - the weight preparation (done once per weight):
 *   w_bf16     [E, H] bf16 router weight (already dequantized to bf16).
 *   scale      device fp32 scalar, output: amax / 448.
 *   w_rt_bf16  [E, H] bf16 output: bf16(E4M3(RNE(w / scale)) * scale), each
 *              step one IEEE fp32 operation, E4M3 saturating at 448 with the
 *              sign of w; scale == 0 gives zeros.
 *   Requires H % 256 == 0.
 *
 * nvfp4_router_topk - logits and selection for T tokens:
 *   x_bf16     [T, H] bf16 activations; w_rt_bf16 [E, H] from nvfp4_router_prepare.
 *   logits     [T, E] fp32 output: sum_k x[t,k] * w_rt[e,k] (exact products,
 *              fp32 accumulation in a fixed order for given T, H, E).
 *   topk_ids   [T, topk] int32 output: experts by descending logit, ties to
 *              the lower id.
 *   topk_w     [T, topk] fp32 output: softmax of the topk selected logits.
 *   workspace  device scratch of nvfp4_router_workspace_size(T, H, E) bytes
 *              (partial sums of the K splits); contents undefined afterwards.
 *   Requires H % 256 == 0, E <= 512, topk <= min(E, 64).  NaN logits are not
 *   handled.
 */
int nvfp4_router_prepare(const void* w_bf16, int64_t E, int64_t H, float* scale, void* w_rt_bf16, void* stream);
size_t nvfp4_router_workspace_size(int64_t T, int64_t H, int64_t E);
int nvfp4_router_topk(const void* x_bf16, const void* w_rt_bf16, int64_t T, int64_t H, int64_t E, int64_t topk,
                      float* logits, int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
