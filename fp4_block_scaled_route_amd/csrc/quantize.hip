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
// compute_gs: two launches.  1) every workgroup folds max |x| over its part
// (integer max of the non-negative fp32 bit patterns: exact and order-free)
// and writes it to its own slot; 2) every quantizing workgroup reduces the
// slots to amax, gs = amax / 2688, and quantizes its blocks; workgroup 0
// writes gs.  No word needs clearing first.
#include <algorithm>

#include "device_util.h"

namespace nvfp4 {

namespace {
constexpr int kAmaxSlots = 256;       // max-pass workgroups, at most
constexpr int kAmaxThreads = 512;
constexpr int kBlockThreads = 256;
constexpr int kBlockGroups = 2048;    // quantizing workgroups, at most (grid-strided)
}  // namespace

__global__ void nvfp4_quant_zero(float* gs) { gs[0] = 0.0f; }

// Max |x| over a workgroup's part of the n8 16-byte pieces: every thread
// folds 8 independent loads per step.  Result: to slots[blockIdx.x] (bits of
// the fp32 max), or merged into *amax_word with one atomic per workgroup.
__device__ __forceinline__ uint32_t fold_amax(const uint16_t* x, int64_t n8) {
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
  __shared__ uint32_t wmax[16];
  const int nwv = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  uint32_t m = 0;
  for (int w = 0; w < nwv; ++w) m = max(m, wmax[w]);
  return m << 16;   // fp32 bits of the workgroup's max |x|
}

__global__ __launch_bounds__(kAmaxThreads) void nvfp4_quant_amax_slots(const uint16_t* x, int64_t n8,
                                                                       unsigned* slots) {
  const uint32_t m = fold_amax(x, n8);
  if (threadIdx.x == 0) slots[blockIdx.x] = m;
}

__global__ __launch_bounds__(kAmaxThreads) void nvfp4_quant_amax(const uint16_t* x, int64_t n8, float* amax_word) {
  const uint32_t m = fold_amax(x, n8);
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned*>(amax_word), m);
}

// Blocks of 16 elements, grid-strided; gs from the slots (slots != nullptr)
// or the word.
__global__ __launch_bounds__(kBlockThreads) void nvfp4_quant_blocks(const uint16_t* x, int64_t nblk,
                                                                    const unsigned* slots, int nslots, float* gs_word,
                                                                    uint8_t* q, uint8_t* sf) {
  __shared__ float s_gs;
  if (threadIdx.x < 64) {
    float g;
    if (slots) {
      uint32_t m = 0;
      for (int i = threadIdx.x; i < nslots; i += 64) m = max(m, slots[i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
      g = __uint_as_float(m) / 2688.0f;
      if (blockIdx.x == 0 && threadIdx.x == 0) gs_word[0] = g;
    } else {
      g = gs_word[0];
    }
    if (threadIdx.x == 0) s_gs = g;
  }
  __syncthreads();
  const float gs = s_gs;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
    const uint4* src = reinterpret_cast<const uint4*>(x + b * 16);
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float xv[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xv[2 * e] = __uint_as_float(u[e] << 16);
      xv[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
    }
    uint2 packed;
    const uint32_t sbyte = quant_block16(xv, gs, packed);
    reinterpret_cast<uint2*>(q)[b] = packed;
    sf[b] = (uint8_t)sbyte;
  }
}

size_t quantize_workspace_bytes() { return kAmaxSlots * sizeof(unsigned); }

hipError_t launch_bf16_amax(const uint16_t* x, int64_t n, float* word, hipStream_t s) {
  hipLaunchKernelGGL(nvfp4_quant_zero, dim3(1), dim3(1), 0, s, word);
  const int64_t n8 = n / 8;
  if (n8 > 0) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxSlots, (n8 + kAmaxThreads - 1) / kAmaxThreads));
    hipLaunchKernelGGL(nvfp4_quant_amax, dim3(grid), dim3(kAmaxThreads), 0, s, x, n8, word);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, float* gs, int compute_gs, uint8_t* q,
                               uint8_t* sf, unsigned* slots, hipStream_t s) {
  const int64_t n = M * K;
  const int64_t nblk = n / 16;
  if (nblk <= 0) {
    if (compute_gs) hipLaunchKernelGGL(nvfp4_quant_zero, dim3(1), dim3(1), 0, s, gs);   // no elements: gs = 0
    return hipGetLastError();
  }
  int nslots = 0;
  if (compute_gs) {
    const int64_t n8 = n / 8;
    nslots = (int)std::max<int64_t>(1, std::min<int64_t>(kAmaxSlots, (n8 + kAmaxThreads * 2 - 1) / (kAmaxThreads * 2)));
    hipLaunchKernelGGL(nvfp4_quant_amax_slots, dim3(nslots), dim3(kAmaxThreads), 0, s, x, n8, slots);
  }
  const int64_t grid = std::min<int64_t>(kBlockGroups, (nblk + kBlockThreads - 1) / kBlockThreads);
  hipLaunchKernelGGL(nvfp4_quant_blocks, dim3((unsigned)grid), dim3(kBlockThreads), 0, s, x, nblk,
                     compute_gs ? slots : nullptr, nslots, gs, q, sf);
  return hipGetLastError();
}

}  // namespace nvfp4
