// Router gate of the MoE layer (gfx950): FP8-E4M3 round trip of the router
// weight, logits, top-k softmax.
//
// Page "nvfp4-megamoe-kernel, commit 1121cd7 - single_shot_inference.py",
// note on the router gate: the router weight (bf16) is quantized to FP8-E4M3
// with one per-tensor scale amax/448 and dequantized back to bf16, and the
// router is a plain linear of the activations with that weight.  The
// selection is top-k softmax routing.  Readings where the page is silent:
//   scale = amax / 448;  byte = RNE_E4M3(w / scale) with the sign of w
//   (saturating at 448);  w_rt = bf16_RNE(E4M3(byte) * scale), each step one
//   IEEE fp32 operation (the weight preparation, done once);
//   logits = x . w_rt^T with exact bf16 products and fp32 accumulation;
//   top-k by descending logit, ties to the lower expert id; the k weights are
//   the softmax of the k selected logits.
#include <algorithm>

#include "device_util.h"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(256) void nvfp4_router_roundtrip(const uint16_t* w, int64_t n8, const float* amax,
                                                              uint16_t* w_rt) {
  const float scale = amax[0] / 448.0f;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(w)[i];
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t pair = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float x = bf16_bits_to_float((u[e] >> (16 * h)) & 0xFFFFu);
      uint32_t r = 0;
      if (scale != 0.0f) {
        const float q = x / scale;
        const uint32_t byte = (__float_as_uint(q) >> 31 << 7) | e4m3_encode_nonneg(__builtin_fabsf(q));
        const float dq = e4m3_to_float(byte) * scale;
        r = float_to_bf16_bits(dq);
      }
      pair |= r << (16 * h);
    }
    o[e] = pair;
  }
  reinterpret_cast<uint4*>(w_rt)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ void nvfp4_router_scale_finish(float* scale) { scale[0] = scale[0] / 448.0f; }

// Logits: a workgroup computes the partial sums of 64 tokens x 128 experts
// over one K split.  Wave w owns experts e0 + 32w .. e0 + 32w + 31 (two MFMA A
// operands of 16) and the four 16-token chunks (B operands): 8 MFMAs per
// 32-wide K step, three steps in flight.  Lane (r, g) loads 16 bytes (8 bf16)
// at K offset 8g of each step for its row r; rows past T or E re-read the last
// row (in bounds, results not written).  Partial tiles go to part[ks][t][e];
// the selection adds the splits in a fixed order.
constexpr int kRT = 64;    // tokens per workgroup
constexpr int kRE = 128;   // experts per workgroup

__global__ __launch_bounds__(256) void nvfp4_router_logits(const uint16_t* x, const uint16_t* w_rt, int T, int H,
                                                           int E, int ksplit, float* part) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int t0 = blockIdx.x * kRT;
  const int e0 = blockIdx.y * kRE + 32 * wave;
  const int ks = blockIdx.z;
  const int kw = H / ksplit;                 // multiple of 64
  const int kbeg = ks * kw;
  const int nsteps = kw / 32;
  const rsrc_t rw = make_rsrc(w_rt, (uint32_t)((int64_t)E * H * 2));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((int64_t)T * H * 2));
  uint32_t we[2], xt[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) we[f] = (uint32_t)min(e0 + 16 * f + lr, E - 1) * H * 2 + lg * 16 + kbeg * 2;
#pragma unroll
  for (int c = 0; c < 4; ++c) xt[c] = (uint32_t)min(t0 + 16 * c + lr, T - 1) * H * 2 + lg * 16 + kbeg * 2;

  f32x4 acc[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[f][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  struct Step {
    u32x4 a[2], b[4];
  };
  // steps past the end keep their place in the pipeline but carry an offset
  // outside the buffer resources: zeros, no memory access (results unused)
  auto load = [&](int step, Step& st) {
    const uint32_t past = step >= nsteps ? 0x80000000u : 0u;
    const uint32_t off = (uint32_t)min(step, nsteps - 1) * 64;
#pragma unroll
    for (int f = 0; f < 2; ++f) st.a[f] = buf_load16(rw, we[f] | past, off);
#pragma unroll
    for (int c = 0; c < 4; ++c) st.b[c] = buf_load16(rx, xt[c] | past, off);
  };
  auto mma = [&](const Step& st) {
    typedef short bf16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[f][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.a[f]),
                                                            __builtin_bit_cast(bf16x8, st.b[c]), acc[f][c], 0, 0, 0);
  };
  Step s0, s1, s2;
  load(0, s0);
  load(1, s1);
  load(2, s2);
  for (int st = 0; st < nsteps; st += 3) {
    mma(s0);
    load(st + 3, s0);
    if (st + 1 >= nsteps) break;
    mma(s1);
    load(st + 4, s1);
    if (st + 2 >= nsteps) break;
    mma(s2);
    load(st + 5, s2);
  }
  // lane (lr, lg) of fragment f, chunk c holds experts e0 + 16f + 4lg + i, token t0 + 16c + lr
  float* pk = part + (int64_t)ks * T * E;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int t = t0 + 16 * c + lr;
    if (t >= T) continue;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + 16 * f + 4 * lg + i;
        if (e < E) pk[(int64_t)t * E + e] = acc[f][c][i];
      }
  }
}

// Largest (value, -index) pair of the wave, in every lane: rotations within
// each 16-lane row (DPP row_ror 8, 4, 2, 1), then the partner row and the
// partner half through the lane-swap instructions (no LDS round trips; the
// comparison is the same in every step, so the order of the steps does not
// change the result).
__device__ __forceinline__ void take_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}
template <int R>
__device__ __forceinline__ void row_ror_step(float& bv, int& bi) {
  // DPP row_ror:R: every lane reads the lane R places away, rotating within its
  // 16-lane row (after rotations by 8, 4, 2 and 1 each lane has seen its whole row)
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bv), 0x120 + R, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, 0x120 + R, 0xF, 0xF, false);
  take_better(bv, bi, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float& bv, int& bi, int lane) {
  row_ror_step<8>(bv, bi);
  row_ror_step<4>(bv, bi);
  row_ror_step<2>(bv, bi);
  row_ror_step<1>(bv, bi);
  {
    // rows 0<->1, 2<->3: vdst gets rows (0, 0, 2, 2), vsrc rows (1, 1, 3, 3) of the value
    const auto v = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, bv), __builtin_bit_cast(unsigned, bv), false, false);
    const auto i = __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    const bool odd = (lane >> 4) & 1;
    take_better(bv, bi, __builtin_bit_cast(float, odd ? v[0] : v[1]), (int)(odd ? i[0] : i[1]));
  }
  {
    // halves: vdst gets (low, low), vsrc (high, high)
    const auto v = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, bv), __builtin_bit_cast(unsigned, bv), false, false);
    const auto i = __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false);
    const bool high = lane >= 32;
    take_better(bv, bi, __builtin_bit_cast(float, high ? v[0] : v[1]), (int)(high ? i[0] : i[1]));
  }
}

// Top-k softmax: one workgroup of 4 waves per token.  Wave w adds the
// K-split partials s = w, w + 4, w + 8, ... in increasing s (4 splits per
// batch of loads); wave 0 then adds the four wave sums in wave order (a fixed
// order, so the logits do not depend on timing), writes them, and selects:
// lane l holds logits l, l + 64, ...
constexpr int kMaxPerLane = 8;   // E <= 512
constexpr int kSelWaves = 4;

__global__ __launch_bounds__(256) void nvfp4_router_select(const float* part, int ksplit, int T, int E, int topk,
                                                           float* logits, int32_t* ids, float* wts) {
  __shared__ float wsum[kSelWaves][kMaxPerLane * 64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x;
  const int64_t sstride = (int64_t)T * E;
  bool valid[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) valid[j] = lane + 64 * j < E;
  float v[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) v[j] = 0.0f;
  const float* p = part + (int64_t)t * E + lane;
  for (int s0 = wave; s0 < ksplit; s0 += 4 * kSelWaves) {
    float q[4][kMaxPerLane];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = s0 + kSelWaves * u;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) q[u][j] = (sp < ksplit && valid[j]) ? p[(int64_t)sp * sstride + 64 * j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j)
        if (s0 + kSelWaves * u < ksplit) v[j] = (s0 + kSelWaves * u == wave) ? q[u][j] : v[j] + q[u][j];
  }
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) wsum[wave][lane + 64 * j] = v[j];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    float a = wsum[0][lane + 64 * j];
    for (int w = 1; w < kSelWaves && w < ksplit; ++w) a += wsum[w][lane + 64 * j];
    v[j] = a;
  }
  bool taken[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    taken[j] = !valid[j];
    if (valid[j]) logits[(int64_t)t * E + lane + 64 * j] = v[j];
  }
  float top = 0.0f, zsum = 0.0f;
  float sel_v = 0.0f;   // lane s keeps the s-th selected value
  int sel_i = 0;
  for (int s = 0; s < topk; ++s) {
    // best of this lane: largest value, then smallest index
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      if (!taken[j] && (v[j] > bv || (v[j] == bv && e < bi))) {
        bv = v[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi, lane);
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j)
        if (j == (bi >> 6)) taken[j] = true;
    }
    if (s == 0) top = bv;
    const float z = expf(bv - top);
    zsum += z;
    if (lane == s) {
      sel_v = z;
      sel_i = bi;
    }
  }
  if (lane < topk) {
    ids[(int64_t)t * topk + lane] = sel_i;
    wts[(int64_t)t * topk + lane] = sel_v / zsum;
  }
}

}  // namespace

hipError_t launch_router_prepare(const uint16_t* w, int64_t n, float* scale, uint16_t* w_rt, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 > 0)
    hipLaunchKernelGGL(nvfp4_router_roundtrip, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, w, n8, scale,
                       w_rt);
  hipLaunchKernelGGL(nvfp4_router_scale_finish, dim3(1), dim3(1), 0, s, scale);
  return hipGetLastError();
}

int router_ksplit(int T, int H, int E) {
  // enough workgroups to cover the GPU twice, K splits of at least 256
  const int blocks = ((T + kRT - 1) / kRT) * ((E + kRE - 1) / kRE);
  int ks = std::max(1, (512 + blocks - 1) / blocks);
  ks = std::min(ks, H / 256);
  while (H % (ks * 64) != 0) --ks;       // K split = a multiple of 64
  return std::max(ks, 1);
}

hipError_t launch_router_topk(const uint16_t* x, const uint16_t* w_rt, int T, int H, int E, int topk, float* logits,
                              int32_t* ids, float* wts, float* part, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int ks = router_ksplit(T, H, E);
  hipLaunchKernelGGL(nvfp4_router_logits, dim3((T + kRT - 1) / kRT, (E + kRE - 1) / kRE, ks), dim3(256), 0, s, x,
                     w_rt, T, H, E, ks, part);
  hipLaunchKernelGGL(nvfp4_router_select, dim3(T), dim3(64 * kSelWaves), 0, s, part, ks, T, E, topk, logits, ids,
                     wts);
  return hipGetLastError();
}

}  // namespace nvfp4
