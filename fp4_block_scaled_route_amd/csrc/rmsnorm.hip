// RMSNorm fused with the NVFP4 activation quantization (gfx950).
//
// Page "nvfp4-megamoe-kernel, commit 1121cd7 - single_shot_inference.py",
// notes on the A/B comparison of the fused ("P4") and unfused paths: the
// fused kernel must give the global scale and FP4 data of RMSNorm followed by
// the activation quantizer.  So this is that composition, each rounding as in
// the unfused path (RMSNorm's output is bf16 before it is quantized):
//   ss  = sum_k x[k]^2 in fp64 (every square of a bf16 value is exact);
//   r   = fp32(1 / sqrt(ss / K + eps)), the root and quotient in fp64;
//   y_k = bf16_RNE(fp32(fp32(x_k * r) * w_k));
//   then the quantizer of quantize.hip on y (gs = amax|y| / 2688, or given).
// Two passes over x instead of four over x and y: pass 1 (one wave per row)
// computes r, the row's max |y| (merged with one atomic per workgroup) and
// optionally writes y; pass 2 (one thread per 16-element block) recomputes
// its 16 values of y from x, w and r, bit for bit, and quantizes them.
#include "device_util.h"

namespace nvfp4 {

namespace {

constexpr int kRowCache = 16;   // rows of up to 16 * 512 elements stay in registers

__device__ __forceinline__ float norm_value(float x, float r, float w) {
  const float xr = __fmul_rn(x, r);
  return bf16_bits_to_float(float_to_bf16_bits(__fmul_rn(xr, w)));
}

__global__ __launch_bounds__(256) void nvfp4_rmsnorm_stats(const uint16_t* x, const uint16_t* w, int T, int K,
                                                           float eps, float* rrow, uint16_t* y, float* amax_word) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  uint32_t mx = 0;   // max |y| bits of this wave's row (bf16 magnitude << 16)
  if (t < T) {
    const uint16_t* row = x + (int64_t)t * K;
    const bool cached = K <= kRowCache * 512;
    uint4 v[kRowCache];
    double ss = 0.0;
    auto add_sq = [&](const uint4 p) {
      const uint32_t u[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = bf16_bits_to_float(u[e] & 0xFFFFu), b = bf16_bits_to_float(u[e] >> 16);
        ss += a * a;
        ss += b * b;
      }
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < kRowCache; ++i) {
        const int c = lane * 8 + 512 * i;
        v[i] = c < K ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kRowCache; ++i) add_sq(v[i]);
    } else {
      for (int c = lane * 8; c < K; c += 512) add_sq(*reinterpret_cast<const uint4*>(row + c));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = (float)(1.0 / __builtin_sqrt(ss / (double)K + (double)eps));
    if (lane == 0) rrow[t] = r;
    auto norm_piece = [&](const uint4 p, int c) {
      const uint4 wp = *reinterpret_cast<const uint4*>(w + c);
      const uint32_t u[4] = {p.x, p.y, p.z, p.w};
      const uint32_t wu[4] = {wp.x, wp.y, wp.z, wp.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = norm_value(bf16_bits_to_float(u[e] & 0xFFFFu), r, bf16_bits_to_float(wu[e] & 0xFFFFu));
        const float hi = norm_value(bf16_bits_to_float(u[e] >> 16), r, bf16_bits_to_float(wu[e] >> 16));
        const uint32_t lb = float_to_bf16_bits(lo), hb = float_to_bf16_bits(hi);
        mx = max(mx, max(lb & 0x7FFFu, hb & 0x7FFFu));
        o[e] = lb | (hb << 16);
      }
      if (y) *reinterpret_cast<uint4*>(y + (int64_t)t * K + c) = make_uint4(o[0], o[1], o[2], o[3]);
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < kRowCache; ++i) {
        const int c = lane * 8 + 512 * i;
        if (c < K) norm_piece(v[i], c);
      }
    } else {
      for (int c = lane * 8; c < K; c += 512) norm_piece(*reinterpret_cast<const uint4*>(row + c), c);
    }
  }
  if (!amax_word) return;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  __shared__ uint32_t wmax[4];
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned*>(amax_word), max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])) << 16);
}

// one thread per 16-element block of y
__global__ __launch_bounds__(256) void nvfp4_rmsnorm_quant(const uint16_t* x, const uint16_t* w, const float* rrow,
                                                           int K, int64_t nblk, const float* gs_word,
                                                           int word_is_amax, uint8_t* q, uint8_t* sf) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  const int kb = K / 16;
  const int64_t t = b / kb;
  const int c = (int)(b - t * kb) * 16;
  const float gs = word_is_amax ? gs_word[0] / 2688.0f : gs_word[0];
  const float r = rrow[t];
  const uint4* src = reinterpret_cast<const uint4*>(x + t * K + c);
  const uint4* wsrc = reinterpret_cast<const uint4*>(w + c);
  const uint4 v0 = src[0], v1 = src[1], w0 = wsrc[0], w1 = wsrc[1];
  const uint32_t u[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  const uint32_t wu[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float yv[16];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    yv[2 * e] = norm_value(bf16_bits_to_float(u[e] & 0xFFFFu), r, bf16_bits_to_float(wu[e] & 0xFFFFu));
    yv[2 * e + 1] = norm_value(bf16_bits_to_float(u[e] >> 16), r, bf16_bits_to_float(wu[e] >> 16));
  }
  uint2 packed;
  const uint32_t sbyte = quant_block16(yv, gs, packed);
  reinterpret_cast<uint2*>(q)[b] = packed;
  sf[b] = (uint8_t)sbyte;
}

__global__ void nvfp4_rmsnorm_gs_zero(float* gs) { gs[0] = 0.0f; }
__global__ void nvfp4_rmsnorm_gs_finish(float* gs) { gs[0] = gs[0] / 2688.0f; }

}  // namespace

hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* w, float eps, int T, int K, uint16_t* y,
                                   float* gs, int compute_gs, uint8_t* q, uint8_t* sf, float* rrow, hipStream_t s) {
  if (compute_gs) hipLaunchKernelGGL(nvfp4_rmsnorm_gs_zero, dim3(1), dim3(1), 0, s, gs);
  if (T <= 0) return hipGetLastError();
  hipLaunchKernelGGL(nvfp4_rmsnorm_stats, dim3((T + 3) / 4), dim3(256), 0, s, x, w, T, K, eps, rrow, y,
                     compute_gs ? gs : nullptr);
  const int64_t nblk = (int64_t)T * (K / 16);
  hipLaunchKernelGGL(nvfp4_rmsnorm_quant, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, x, w, rrow, K, nblk,
                     gs, compute_gs, q, sf);
  if (compute_gs) hipLaunchKernelGGL(nvfp4_rmsnorm_gs_finish, dim3(1), dim3(1), 0, s, gs);
  return hipGetLastError();
}

}  // namespace nvfp4
