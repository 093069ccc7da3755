// Weighted combine of the routed experts' output rows and the shared expert
// (gfx950).  For token t: y_t = sum_{j=0..topk-1} w[t, j] * o(t, j) + o_shared(t),
// accumulated in fp32 in that fixed order, then rounded to bf16.  o(t, j) is
// the down-projection row of pair t*topk + j, already scaled by the pair's
// weight_scale_2 and stored in bf16 (the layer's output precision); routing
// weights are applied here, after the down GEMM (the "weighted combine" of the
// MoE layer; summation order is a reading).  A pair whose expert id is outside
// [0, E) contributes nothing.
#include "device_util.h"

namespace nvfp4 {

// Each slot row is read once, here, so its loads carry the non-temporal hint
// (measured on MI355X: the 4096-token combine 0.098-0.101 -> 0.090 ms).
__device__ __forceinline__ uint4 load_slot(const uint16_t* p) {
  const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(q[0], q[1], q[2], q[3]);
}

// KMAX > 0 (topk <= KMAX): all row loads of the token are issued before the
// first use, so a wave has topk + 1 requests in flight instead of one; the
// sum still runs in the order j = 0..topk-1, then the shared row.  KMAX == 0:
// any topk, one row at a time.
template <int KMAX>
__global__ __launch_bounds__(256) void nvfp4_moe_combine(const CombineArgs a) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (n >= a.H) return;
  const int P = a.T * a.topk;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4 v, float w) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * bf16_bits_to_float(u[i] & 0xffffu);
      acc[2 * i + 1] += w * bf16_bits_to_float(u[i] >> 16);
    }
  };
  auto add_shared = [&](const uint4 v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_bits_to_float(u[i] & 0xffffu);
      acc[2 * i + 1] += bf16_bits_to_float(u[i] >> 16);
    }
  };
  if constexpr (KMAX > 0) {
    uint4 v[KMAX];
    bool ok[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int id = j < a.topk ? a.ids[t * a.topk + j] : -1;
      ok[j] = id >= 0 && id < a.E;
      v[j] = ok[j] ? load_slot(a.slot + (int64_t)(t * a.topk + j) * a.H + n) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 vs = make_uint4(0u, 0u, 0u, 0u);
    if (a.shared) vs = load_slot(a.slot + (int64_t)(P + t) * a.H + n);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (ok[j]) add(v[j], a.w[t * a.topk + j]);
    if (a.shared) add_shared(vs);
  } else {
    for (int j = 0; j < a.topk; ++j) {
      const int id = a.ids[t * a.topk + j];
      if (id < 0 || id >= a.E) continue;
      add(load_slot(a.slot + (int64_t)(t * a.topk + j) * a.H + n), a.w[t * a.topk + j]);
    }
    if (a.shared) add_shared(load_slot(a.slot + (int64_t)(P + t) * a.H + n));
  }
  uint4 o;
  o.x = float_to_bf16_bits(acc[0]) | (float_to_bf16_bits(acc[1]) << 16);
  o.y = float_to_bf16_bits(acc[2]) | (float_to_bf16_bits(acc[3]) << 16);
  o.z = float_to_bf16_bits(acc[4]) | (float_to_bf16_bits(acc[5]) << 16);
  o.w = float_to_bf16_bits(acc[6]) | (float_to_bf16_bits(acc[7]) << 16);
  *reinterpret_cast<uint4*>(a.y + (int64_t)t * a.H + n) = o;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  dim3 grid((a.H / 8 + 255) / 256, a.T);
  if (a.topk <= 8)
    hipLaunchKernelGGL(nvfp4_moe_combine<8>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(nvfp4_moe_combine<0>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nvfp4
