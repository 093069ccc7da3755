// NVFP4 activation quantization (gfx950).
//
// Page "nvfp4-megamoe-kernel, commit 4c6464e - vllm", note on the activation
// global scale: gs = amax / (6 * 448), used as a multiplier (never inverted).
// Per 16-element block of a row (the unstated steps, read plainly):
//   scale byte = RNE_E4M3(amax_blk / (6 * gs)), saturating at 448;
//   code       = RNE_E2M1(x * (1 / (E4M3(byte) * gs))), saturating at 6.
// Each step is one correctly rounded fp32 operation in this order, so codes
// and scale bytes are reproducible bit for bit.  gs == 0 gives zeros.
//
// compute_gs: 1) zero the amax word, 2) grid-wide max |x| with an integer
// atomicMax on the non-negative fp32 bit patterns (exact and order-free),
// 3) quantize with gs = amax / 2688 computed by every thread from the amax
// word, 4) overwrite the word with gs.
#include "device_util.h"

namespace nvfp4 {

__global__ void nvfp4_quant_zero(float* gs) { gs[0] = 0.0f; }

// Grid-wide max |x|: every thread folds 8 independent 16-byte loads per
// iteration, the block reduces through LDS, and one atomic per block (not per
// wave: thousands of atomics on one word serialise) merges the blocks.
__global__ __launch_bounds__(256) void nvfp4_quant_amax(const uint16_t* x, int64_t n8, float* amax_word) {
  const uint4* v4 = reinterpret_cast<const uint4*>(x);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t mx = 0;
  auto fold = [&](const uint4 v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = max(mx, u[e] & 0x7FFFu);
      mx = max(mx, (u[e] >> 16) & 0x7FFFu);
    }
  };
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n8; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = v4[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) fold(v[u]);
  }
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 a = v4[i], b = v4[i + stride], c = v4[i + 2 * stride], d = v4[i + 3 * stride];
    fold(a);
    fold(b);
    fold(c);
    fold(d);
  }
  for (; i < n8; i += stride) fold(v4[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned*>(amax_word), max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])) << 16);
}

// one thread per 16-element block
__global__ __launch_bounds__(256) void nvfp4_quant_blocks(const uint16_t* x, int64_t nblk, const float* gs_word,
                                                          int word_is_amax, uint8_t* q, uint8_t* sf) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const float gs = word_is_amax ? gs_word[0] / 2688.0f : gs_word[0];
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 16);
  const uint4 v0 = src[0], v1 = src[1];
  const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float xv[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    xv[2 * e] = bf16_bits_to_float(u[e] & 0xFFFFu);
    xv[2 * e + 1] = bf16_bits_to_float(u[e] >> 16);
  }
  uint2 packed;
  const uint32_t sbyte = quant_block16(xv, gs, packed);
  reinterpret_cast<uint2*>(q)[b] = packed;
  sf[b] = (uint8_t)sbyte;
}

__global__ void nvfp4_quant_finish(float* gs) { gs[0] = gs[0] / 2688.0f; }

hipError_t launch_bf16_amax(const uint16_t* x, int64_t n, float* word, hipStream_t s) {
  hipLaunchKernelGGL(nvfp4_quant_zero, dim3(1), dim3(1), 0, s, word);
  const int64_t n8 = n / 8;
  if (n8 > 0) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (n8 + 255) / 256));
    hipLaunchKernelGGL(nvfp4_quant_amax, dim3(grid), dim3(256), 0, s, x, n8, word);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, float* gs, int compute_gs, uint8_t* q,
                               uint8_t* sf, hipStream_t s) {
  const int64_t n = M * K;
  const int64_t nblk = n / 16;
  if (compute_gs) {
    hipLaunchKernelGGL(nvfp4_quant_zero, dim3(1), dim3(1), 0, s, gs);
    const int64_t n8 = n / 8;
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (n8 + 255) / 256));
    hipLaunchKernelGGL(nvfp4_quant_amax, dim3(grid), dim3(256), 0, s, x, n8, gs);
  }
  if (nblk > 0) {
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(nvfp4_quant_blocks, dim3((unsigned)grid), dim3(256), 0, s, x, nblk, gs, compute_gs, q, sf);
  }
  if (compute_gs) hipLaunchKernelGGL(nvfp4_quant_finish, dim3(1), dim3(1), 0, s, gs);
  return hipGetLastError();
}

}  // namespace nvfp4
