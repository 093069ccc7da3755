// RMSNorm fused with the NVFP4 activation quantization (gfx950).
//
// Page "nvfp4-megamoe-kernel, commit 1121cd7 - single_shot_inference.py",
// notes on the A/B comparison of the fused ("P4") and unfused paths: the
// fused kernel must give the global scale and FP4 data of RMSNorm followed by
// the activation quantizer.  So this is that composition, each rounding as in
// the unfused path (RMSNorm's output is bf16 before it is quantized):
//   ss  = sum_k x[k]^2 in fp64 (every square of a bf16 value is exact, a
//         16-bit significand; the additions are exact while the row's squares
//         fit one 53-bit fixed point with the carries of K terms, i.e. their
//         exponents span at most 53 - 16 - ceil(log2 K) bits: 24 for K = 7168,
//         x within about 12 binades of the row's largest |x|; otherwise they
//         round, in this kernel's order);
//   r   = fp32(1 / sqrt(ss / K + eps)), the root and quotient in fp64;
//   y_k = bf16_RNE(fp32(fp32(x_k * r) * w_k));
//   then the quantizer of quantize.hip on y (gs = amax|y| / 2688, or given).
// Two launches, two passes over x:
//  pass 1 (a wave per row, the row held in registers, w staged in LDS once per
//    workgroup): r of the row, the row's max |y|, y if asked for; each
//    workgroup writes the max over its rows to its own slot (no atomics, so
//    nothing needs clearing first);
//  pass 2 (a thread per 16-element block, grid-strided; w again in LDS):
//    every workgroup reduces the slots to amax (integer max of the bit
//    patterns: exact and order-free) and gs = amax / 2688, recomputes its 16
//    values of y from x, w and r bit for bit and quantizes them; workgroup 0
//    writes gs.
#include <algorithm>

#include "device_util.h"

namespace nvfp4 {

namespace {

constexpr int kStatsWaves = 8;     // waves per pass-1 workgroup, at most
constexpr int kMaxSlots = 512;     // pass-1 workgroups, at most (one max slot each)
constexpr int kQuantThreads = 256;
constexpr int kLdsW = 32768;       // bf16 weights staged in LDS (K up to this; longer K reads w from memory)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// y of two adjacent elements, packed bf16 (element 2j in the low half):
// bf16_RNE(fp32(fp32(x * r) * w)); one packed conversion (NaN preserving).
__device__ __forceinline__ uint32_t norm_pair(uint32_t xp, uint32_t wp, float r) {
  const float lo = __fmul_rn(__fmul_rn(__uint_as_float(xp << 16), r), __uint_as_float(wp << 16));
  const float hi = __fmul_rn(__fmul_rn(__uint_as_float(xp & 0xFFFF0000u), r), __uint_as_float(wp & 0xFFFF0000u));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// w [K] into LDS (K <= kLdsW), by all threads of the workgroup, eight
// 16-byte loads in flight per thread
__device__ __forceinline__ void stage_w(const uint16_t* w, int K, uint16_t* wl) {
  const int nv = K / 8;
  for (int base = threadIdx.x; base < nv; base += blockDim.x * 8) {
    u32x4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = min(base + j * (int)blockDim.x, nv - 1);   // (repeats the last vector past the end)
      t[j] = *reinterpret_cast<const u32x4*>(w + i * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + j * (int)blockDim.x;
      if (i < nv) *reinterpret_cast<u32x4*>(wl + i * 8) = t[j];
    }
  }
  __syncthreads();
}

// Pass 1: piece i of a lane covers columns 8 * lane + 512 * i (rows of up to
// RC * 512 elements stay in registers; longer rows are read twice).
template <int RC>
__global__ __launch_bounds__(kStatsWaves * 64, 4) void nvfp4_rmsnorm_stats(const uint16_t* x, const uint16_t* w,
                                                                          int T, int K, float eps, float* rrow,
                                                                          uint16_t* y, unsigned* slots) {
  extern __shared__ __attribute__((aligned(16))) uint16_t wl[];   // K bf16 when K <= kLdsW
  __shared__ uint32_t wmax[kStatsWaves];
  const bool wlds = K <= kLdsW;
  const uint16_t* wsrc = wlds ? wl : w;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwv = blockDim.x >> 6;
  const bool cached = K <= RC * 512;
  u16x2_t mx2 = {0, 0};   // max |y| bits (bf16 magnitudes) of this wave's rows, per half
  bool staged = !wlds;
  for (int t = blockIdx.x * nwv + wave; t < T || !staged; t += gridDim.x * nwv) {
    // the row's loads go out before the workgroup stages w (first row)
    const bool has_row = t < T;
    const uint16_t* row = x + (int64_t)(has_row ? t : 0) * K;
    u32x4 v[RC];
    if (cached) {
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        const int c = lane * 8 + 512 * i;
        v[i] = has_row && c < K ? *reinterpret_cast<const u32x4*>(row + c) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
    if (!staged) {
      stage_w(w, K, wl);   // (every wave of the workgroup takes this branch on its first row)
      staged = true;
    }
    if (!has_row) break;
    // sum of squares: four fp64 partial sums per lane (pair e of each 16-byte
    // piece into sum e, pieces in column order), added pairwise, then across
    // lanes in a butterfly
    double ss4[4] = {0.0, 0.0, 0.0, 0.0};
    auto add_sq = [&](const u32x4 p) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double a = __uint_as_float(p[e] << 16), b = __uint_as_float(p[e] & 0xFFFF0000u);
        ss4[e] += a * a;
        ss4[e] += b * b;
      }
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < RC; ++i) add_sq(v[i]);
    } else {
      for (int c = lane * 8; c < K; c += 512) add_sq(*reinterpret_cast<const u32x4*>(row + c));
    }
    double ss = (ss4[0] + ss4[1]) + (ss4[2] + ss4[3]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = (float)(1.0 / __builtin_sqrt(ss / (double)K + (double)eps));
    if (lane == 0) rrow[t] = r;
    auto norm_piece = [&](const u32x4 p, int c) {
      const u32x4 wp = *reinterpret_cast<const u32x4*>(wsrc + c);
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = norm_pair(p[e], wp[e], r);
        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2_t, o[e] & 0x7FFF7FFFu));
      }
      if (y) *reinterpret_cast<u32x4*>(y + (int64_t)t * K + c) = o;
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        const int c = lane * 8 + 512 * i;
        if (c < K) norm_piece(v[i], c);
        __builtin_amdgcn_sched_barrier(0);   // one piece at a time: the row stays the only large live set
      }
    } else {
      for (int c = lane * 8; c < K; c += 512) norm_piece(*reinterpret_cast<const u32x4*>(row + c), c);
    }
  }
  if (!slots) return;
  uint32_t mx = max((uint32_t)mx2[0], (uint32_t)mx2[1]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
  if (lane == 0) wmax[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < nwv; ++i) m = max(m, wmax[i]);
    slots[blockIdx.x] = m << 16;   // fp32 bits of the workgroup's max |y|
  }
}

// Pass 2: blocks of 16 elements of y, grid-strided; gs from the slots
// (compute_gs) or the word.
__global__ __launch_bounds__(kQuantThreads) void nvfp4_rmsnorm_quant(const uint16_t* x, const uint16_t* w,
                                                                     const float* rrow, int K, int64_t nblk,
                                                                     const unsigned* slots, int nslots, float* gs_word,
                                                                     uint8_t* q, uint8_t* sf) {
  extern __shared__ __attribute__((aligned(16))) uint16_t wl[];   // K bf16 when K <= kLdsW
  __shared__ float s_gs;
  const bool wlds = K <= kLdsW;
  if (wlds) stage_w(w, K, wl);
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
  const uint16_t* wsrc = wlds ? wl : w;
  const int kb = K / 16;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = b / kb;
    const int c = (int)(b - t * kb) * 16;
    const float r = rrow[t];
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * K + c);
    const u32x4* wp = reinterpret_cast<const u32x4*>(wsrc + c);
    const u32x4 v0 = src[0], v1 = src[1], w0 = wp[0], w1 = wp[1];
    float yv[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ya = norm_pair(v0[e], w0[e], r), yb = norm_pair(v1[e], w1[e], r);
      yv[2 * e] = __uint_as_float(ya << 16);
      yv[2 * e + 1] = __uint_as_float(ya & 0xFFFF0000u);
      yv[8 + 2 * e] = __uint_as_float(yb << 16);
      yv[8 + 2 * e + 1] = __uint_as_float(yb & 0xFFFF0000u);
    }
    uint2 packed;
    const uint32_t sbyte = quant_block16(yv, gs, packed);
    reinterpret_cast<uint2*>(q)[b] = packed;
    sf[b] = (uint8_t)sbyte;
  }
}

__global__ void nvfp4_rmsnorm_gs_empty(float* gs) { gs[0] = 0.0f; }

}  // namespace

size_t rmsnorm_workspace_bytes(int T) {
  return (((size_t)T * sizeof(float) + 255) / 256) * 256 + kMaxSlots * sizeof(unsigned);
}

hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* w, float eps, int T, int K, uint16_t* y,
                                   float* gs, int compute_gs, uint8_t* q, uint8_t* sf, void* workspace,
                                   hipStream_t s) {
  if (T <= 0) {
    // no elements: amax = 0
    if (compute_gs) hipLaunchKernelGGL(nvfp4_rmsnorm_gs_empty, dim3(1), dim3(1), 0, s, gs);
    return hipGetLastError();
  }
  float* rrow = static_cast<float*>(workspace);
  unsigned* slots = reinterpret_cast<unsigned*>(static_cast<uint8_t*>(workspace) +
                                                (((size_t)T * sizeof(float) + 255) / 256) * 256);
  // a wave per row, spread over up to kMaxSlots workgroups of up to 8 waves
  const int wpg = std::min(kStatsWaves, std::max(1, (T + kMaxSlots - 1) / kMaxSlots));
  const int g1 = std::min(kMaxSlots, (T + wpg - 1) / wpg);
  const size_t lds = K <= kLdsW ? (size_t)K * 2 : 0;
  const dim3 grid1(g1), block1(wpg * 64);
  unsigned* sl = compute_gs ? slots : nullptr;
  // the row cache sized to K (rows of up to 8192 elements stay in registers)
  const int pieces = (K + 511) / 512;
  if (pieces <= 2)
    hipLaunchKernelGGL(nvfp4_rmsnorm_stats<2>, grid1, block1, lds, s, x, w, T, K, eps, rrow, y, sl);
  else if (pieces <= 4)
    hipLaunchKernelGGL(nvfp4_rmsnorm_stats<4>, grid1, block1, lds, s, x, w, T, K, eps, rrow, y, sl);
  else if (pieces <= 8)
    hipLaunchKernelGGL(nvfp4_rmsnorm_stats<8>, grid1, block1, lds, s, x, w, T, K, eps, rrow, y, sl);
  else if (pieces <= 14)
    hipLaunchKernelGGL(nvfp4_rmsnorm_stats<14>, grid1, block1, lds, s, x, w, T, K, eps, rrow, y, sl);
  else
    hipLaunchKernelGGL(nvfp4_rmsnorm_stats<16>, grid1, block1, lds, s, x, w, T, K, eps, rrow, y, sl);
  const int64_t nblk = (int64_t)T * (K / 16);
  const int64_t g2 = std::max<int64_t>(1, std::min<int64_t>(2048, (nblk + kQuantThreads - 1) / kQuantThreads));
  hipLaunchKernelGGL(nvfp4_rmsnorm_quant, dim3((unsigned)g2), dim3(kQuantThreads), lds, s, x, w, rrow, K, nblk, sl,
                     g1, gs, q, sf);
  return hipGetLastError();
}

}  // namespace nvfp4
