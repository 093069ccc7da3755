// Grouped NVFP4 GEMM for gfx950: weight-stationary streaming of packed E2M1
// weights + E4M3 block scales, exact decode to fp16, fp16 MFMA, fused
// epilogues (dense bf16 output, SwiGLU with fp32 or NVFP4 hidden output,
// scatter of per-pair output rows).
//
// Computes, per group g and weight row n, acc[row, n] = sum_k A[row, k] * E2M1(W[n,k]) * E4M3(S[n,k/16])
// and applies the product of the two global scales (weight_scale_2 of the
// group and the activation global scale) once, in the epilogue: the block-
// scaled GEMM y = (x*scale_a*gsa) @ (w*scale_b*gsb)^T of page
// "nvfp4-megamoe-kernel, commit 1121cd7 - single_shot_inference.py" (note on
// the weight-dequant global scale).
//
// Mapping (one workgroup = NW waves):
//  * a work item is (group, block of weight rows); groups come in the order of
//    a device-side list (largest first), so no host synchronisation is needed;
//  * every wave owns R fragments of 16 weight rows and streams them over the
//    whole K range once per pass of up to 16*MAXC activation rows: weights are
//    read from HBM once per pass (once in total unless a group has more rows);
//  * K is walked in chunks of 256.  Lane (r, g) of a fragment (r = lane%16,
//    g = lane/16) loads bytes [32g, 32g+32) of the chunk of row r (64 codes)
//    and the 4 scale bytes of those 4 blocks, with two 16-byte loads and one
//    4-byte load.  MFMA step q (0..7) of the chunk then covers K positions
//    {64g' + 8q + e}: the MFMA's K index is a permutation of the real K, the
//    same for both operands, so the sum is unchanged;
//  * the workgroup stages the activation chunk [16*MAXC rows, 256] into LDS as
//    fp16 (double buffered), converted exactly: NVFP4 rows decode exactly;
//    bf16 / fp32 rows are scaled by a per-row power of two into [2^14, 2^15)
//    so fp16 holds them (the shift is undone in the epilogue);
//  * weights are the MFMA A operand (16 weight rows), activations the B
//    operand (16 tokens): D[weight row][token], so decode-sized groups waste
//    MFMA lanes but never HBM bandwidth.
#include "device_util.h"

namespace nvfp4 {

namespace {

template <int R>
struct WBuf {
  u32x4 c0[R];
  u32x4 c1[R];
  uint32_t s[R];
};

__device__ __forceinline__ uint32_t word_of(const u32x4& a, const u32x4& b, int q) {
  return q < 4 ? a[q & 3] : b[q & 3];
}

template <int EP>
constexpr bool is_swiglu() { return EP == EPI_SWIGLU_F32 || EP == EPI_SWIGLU_FP4; }

// Rows (output columns) covered by one workgroup.
template <int R, int NW, int EP>
constexpr int block_rows() { return is_swiglu<EP>() ? NW * (R / 2) * 16 : NW * R * 16; }

}  // namespace

template <int MAXC, int R, int NW, int AM, int EP>
__global__ __launch_bounds__(NW * 64) void nvfp4_grouped_gemm(const GemmArgs a) {
  static_assert(!is_swiglu<EP>() || (R % 2 == 0), "SwiGLU needs gate/up fragment pairs");
  constexpr int PR = 16 * MAXC;          // activation rows per pass
  constexpr int TPR = 32;                // threads per staged row (8 elements each)
  constexpr int RSTEP = NW * 64 / TPR;   // rows staged per thread sweep
  constexpr int SROWS = (PR + RSTEP - 1) / RSTEP;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][PR * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  // ---- work item: (group, block of weight rows)
  const int gi = blockIdx.x / a.nb;
  const int nbk = blockIdx.x - gi * a.nb;
  int g, row0, m;
  if (a.offsets) {
    if (gi >= *a.gcount) return;
    g = a.glist[gi];
    row0 = a.offsets[g];
    m = a.offsets[g + 1] - row0;
  } else {
    g = 0;
    row0 = 0;
    m = a.M;
  }
  if (m <= 0) return;
  const bool shared = g >= a.n_routed;
  const uint8_t* W = shared ? a.sw : a.w + (int64_t)g * a.w_gstride;
  const uint8_t* WS = shared ? a.sw_sf : a.w_sf + (int64_t)g * a.sf_gstride;
  float alpha = shared ? a.sw_ws2[0] : a.w_ws2[g];
  if (a.gsa) alpha *= a.gsa[0];

  const int K = a.K;
  const int64_t KB = K / 2, KS = K / 16;
  const int nkc = K / kChunk;

  // ---- this wave's weight fragments
  int fbase[R];       // first weight row of the fragment (gate row for SwiGLU pairs)
  bool fvalid[R];
  const uint8_t* wp[R];
  const uint8_t* sp[R];
#pragma unroll
  for (int f = 0; f < R; ++f) {
    int row;
    if constexpr (is_swiglu<EP>()) {
      const int gate = nbk * block_rows<R, NW, EP>() + (wave * (R / 2) + (f >> 1)) * 16;
      fbase[f] = gate;
      fvalid[f] = gate < a.I;
      row = (f & 1 ? a.I : 0) + gate + lr;
    } else {
      const int base = nbk * block_rows<R, NW, EP>() + (wave * R + f) * 16;
      fbase[f] = base;
      fvalid[f] = base < a.N;
      row = base + lr;
    }
    if (!fvalid[f]) row = lr;  // keep addresses inside the group; results are discarded
    wp[f] = W + (int64_t)row * KB + lg * 32;
    sp[f] = WS + (int64_t)row * KS + lg * 4;
  }

  auto wload = [&](WBuf<R>& wb, int kc) {
#pragma unroll
    for (int f = 0; f < R; ++f) {
      const u32x4* p = reinterpret_cast<const u32x4*>(wp[f] + (int64_t)kc * 128);
      wb.c0[f] = __builtin_nontemporal_load(p);
      wb.c1[f] = __builtin_nontemporal_load(p + 1);
      wb.s[f] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sp[f] + (int64_t)kc * 16));
    }
  };

  // A row (in the activation tensor) of sorted row r, and its staging shift.
  auto a_row_of = [&](int r) -> int {
    if (!a.a_by_token || !a.offsets) return r;
    const int pid = a.perm[r];
    return pid < a.P ? pid / a.topk : pid - a.P;
  };
  auto shift_of = [&](int arow) -> int {
    if constexpr (AM == A_BF16) return a.rowshift[arow];
    else if constexpr (AM == A_F32) return shift_from_maxbits(a.rowmax[arow]);
    else return 0;
  };

  const int seg = tid % TPR;       // 8-element segment of the 256-element chunk
  const int rsub = tid / TPR;

  const int npass = (m + PR - 1) / PR;
  for (int pass = 0; pass < npass; ++pass) {
    const int pbase = pass * PR;
    const int prow = min(PR, m - pbase);
    const int nc = (prow + 15) >> 4;

    // staging rows of this thread
    int srow[SROWS];
    int sshift[SROWS];
    bool sval[SROWS];
#pragma unroll
    for (int i = 0; i < SROWS; ++i) {
      const int rr = rsub + RSTEP * i;
      sval[i] = rr < prow;
      const int arow = sval[i] ? a_row_of(row0 + pbase + rr) : 0;
      srow[i] = arow;
      sshift[i] = sval[i] ? shift_of(arow) : 0;
    }

    // staging registers
    uint4 st0[SROWS];
    uint4 st1[SROWS];  // A_F32 second half
    uint32_t stc[SROWS], sts[SROWS];

    auto stage_load = [&](int kc) {
#pragma unroll
      for (int i = 0; i < SROWS; ++i) {
        if (!sval[i]) continue;
        if constexpr (AM == A_BF16) {
          const uint16_t* src = reinterpret_cast<const uint16_t*>(a.a) + (int64_t)srow[i] * K + kc * kChunk + seg * 8;
          st0[i] = *reinterpret_cast<const uint4*>(src);
        } else if constexpr (AM == A_F32) {
          const float* src = reinterpret_cast<const float*>(a.a) + (int64_t)srow[i] * K + kc * kChunk + seg * 8;
          st0[i] = *reinterpret_cast<const uint4*>(src);
          st1[i] = *reinterpret_cast<const uint4*>(src + 4);
        } else {
          const uint8_t* src = reinterpret_cast<const uint8_t*>(a.a) + (int64_t)srow[i] * KB + kc * 128 + seg * 4;
          stc[i] = *reinterpret_cast<const uint32_t*>(src);
          sts[i] = a.a_sf[(int64_t)srow[i] * KS + kc * 16 + (seg >> 1)];
        }
      }
    };
    auto stage_write = [&](int buf) {
#pragma unroll
      for (int i = 0; i < SROWS; ++i) {
        if (!sval[i]) continue;
        const int rr = rsub + RSTEP * i;
        f16x8 v;
        if constexpr (AM == A_BF16) {
          const uint32_t u[4] = {st0[i].x, st0[i].y, st0[i].z, st0[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] & 0xFFFFu), sshift[i]);
            v[2 * e + 1] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] >> 16), sshift[i]);
          }
        } else if constexpr (AM == A_F32) {
          const uint32_t u[8] = {st0[i].x, st0[i].y, st0[i].z, st0[i].w, st1[i].x, st1[i].y, st1[i].z, st1[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (f16)__builtin_ldexpf(__uint_as_float(u[e]), sshift[i]);
        } else {
          v = decode8(stc[i], (f16)e4m3_to_float(sts[i]));
        }
        *reinterpret_cast<f16x8*>(&lds[buf][rr * kLdsRow + seg * 16]) = v;
      }
    };

    f32x4 acc[R][MAXC];
#pragma unroll
    for (int f = 0; f < R; ++f)
#pragma unroll
      for (int c = 0; c < MAXC; ++c) acc[f][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const WBuf<R>& wb, int buf) {
      f16 sc[R][4];
#pragma unroll
      for (int f = 0; f < R; ++f) scales4(wb.s[f], sc[f]);
      const uint8_t* B = &lds[buf][0];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f16x8 af[R];
#pragma unroll
        for (int f = 0; f < R; ++f) af[f] = decode8(word_of(wb.c0[f], wb.c1[f], q), sc[f][q >> 1]);
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          if (c < nc) {
            const f16x8 b = *reinterpret_cast<const f16x8*>(B + (16 * c + lr) * kLdsRow + (64 * lg + 8 * q) * 2);
#pragma unroll
            for (int f = 0; f < R; ++f)
              acc[f][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[f], b, acc[f][c], 0, 0, 0);
          }
        }
      }
    };

    WBuf<R> wb0, wb1;
    wload(wb0, 0);
    if (nkc > 1) wload(wb1, 1);
    stage_load(0);
    stage_write(0);
    __syncthreads();
    for (int kc = 0; kc < nkc; kc += 2) {
      // chunk kc: weights in wb0, activations in LDS buffer 0
      if (kc + 1 < nkc) stage_load(kc + 1);
      compute(wb0, 0);
      if (kc + 2 < nkc) wload(wb0, kc + 2);
      if (kc + 1 < nkc) stage_write(1);
      __syncthreads();
      if (kc + 1 >= nkc) break;
      // chunk kc+1: weights in wb1, activations in LDS buffer 1
      if (kc + 2 < nkc) stage_load(kc + 2);
      compute(wb1, 1);
      if (kc + 3 < nkc) wload(wb1, kc + 3);
      if (kc + 2 < nkc) stage_write(0);
      __syncthreads();
    }

    // ---- epilogue
    if constexpr (EP == EPI_Y_BF16 || EP == EPI_SLOT) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int tr = pbase + 16 * c + lr;
        if (c >= nc || tr >= m) continue;
        const int r = row0 + tr;
        const int sh = shift_of(a_row_of(r));
#pragma unroll
        for (int f = 0; f < R; ++f) {
          if (!fvalid[f]) continue;
          const int n0 = fbase[f] + 4 * lg;
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = __builtin_ldexpf(acc[f][c][i], -sh) * alpha;
          if constexpr (EP == EPI_Y_BF16) {
            uint2 o;
            o.x = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
            o.y = float_to_bf16_bits(v[2]) | (float_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(a.y + (int64_t)r * a.N + n0) = o;
          } else {
            const int pid = a.perm[r];
            *reinterpret_cast<float4*>(a.slot + (int64_t)pid * a.N + n0) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    } else {
      // SwiGLU: fragments 2p (gate rows) and 2p+1 (up rows) share the layout
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        if (c >= nc) continue;   // uniform across the wave
        const int tr = pbase + 16 * c + lr;
        const bool tv = tr < m;
        const int r = row0 + (tv ? tr : 0);
        const int sh = tv ? shift_of(a_row_of(r)) : 0;
        float hmx = 0.f;
#pragma unroll
        for (int p = 0; p < R / 2; ++p) {
          if (!fvalid[2 * p]) continue;  // uniform across the wave
          const int n0 = fbase[2 * p] + 4 * lg;
          float hv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gv = __builtin_ldexpf(acc[2 * p][c][i], -sh) * alpha;
            const float uv = __builtin_ldexpf(acc[2 * p + 1][c][i], -sh) * alpha;
            hv[i] = gv / (1.0f + __expf(-gv)) * uv;
          }
          if constexpr (EP == EPI_SWIGLU_F32) {
            if (tv) *reinterpret_cast<float4*>(a.h + (int64_t)r * a.I + n0) = make_float4(hv[0], hv[1], hv[2], hv[3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) hmx = fmaxf(hmx, __builtin_fabsf(hv[i]));
          } else {
            // NVFP4 quantization of h: the fragment's 16 gate rows are one
            // 16-element block of row r; its 4 lanes hold 4 values each.
            float ab = fmaxf(fmaxf(__builtin_fabsf(hv[0]), __builtin_fabsf(hv[1])),
                             fmaxf(__builtin_fabsf(hv[2]), __builtin_fabsf(hv[3])));
            ab = fmaxf(ab, __shfl_xor(ab, 16));
            ab = fmaxf(ab, __shfl_xor(ab, 32));
            const float gs = a.h_gs[0];
            uint32_t sbyte = 0, packed = 0;
            if (gs != 0.0f) {
              sbyte = e4m3_encode_nonneg(ab / (6.0f * gs));
              const float scale = e4m3_to_float(sbyte) * gs;
              if (scale != 0.0f) {
                const float rcp = 1.0f / scale;
#pragma unroll
                for (int i = 0; i < 4; ++i) packed |= e2m1_encode(hv[i] * rcp) << (4 * i);
              }
            }
            if (tv) {
              *reinterpret_cast<uint16_t*>(a.hq + (int64_t)r * (a.I / 2) + n0 / 2) = (uint16_t)packed;
              if (lg == 0) a.hq_sf[(int64_t)r * (a.I / 16) + fbase[2 * p] / 16] = (uint8_t)sbyte;
            }
          }
        }
        if constexpr (EP == EPI_SWIGLU_F32) {
          hmx = fmaxf(hmx, __shfl_xor(hmx, 16));
          hmx = fmaxf(hmx, __shfl_xor(hmx, 32));
          if (tv && lg == 0) atomicMax(a.hmax + r, __float_as_uint(hmx));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

namespace {
constexpr int kNW = 4;

template <int MAXC, int R, int AM, int EP>
hipError_t launch_one(const GemmArgs& a, int n_groups, hipStream_t s) {
  const int grid = n_groups * a.nb;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((nvfp4_grouped_gemm<MAXC, R, kNW, AM, EP>), dim3(grid), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

template <int AM, int EP, int R>
hipError_t by_maxc(const GemmArgs& a, int maxc, int n_groups, hipStream_t s) {
  switch (maxc) {
    case 1: return launch_one<1, R, AM, EP>(a, n_groups, s);
    case 2: return launch_one<2, R, AM, EP>(a, n_groups, s);
    case 4: return launch_one<4, R, AM, EP>(a, n_groups, s);
    case 8: return launch_one<8, R, AM, EP>(a, n_groups, s);
    default: return hipErrorInvalidValue;
  }
}

template <int AM, int EP>
hipError_t by_r(const GemmArgs& a, GemmShape sh, int n_groups, hipStream_t s) {
  switch (sh.r) {
    case 2: return by_maxc<AM, EP, 2>(a, sh.maxc, n_groups, s);
    case 4: return by_maxc<AM, EP, 4>(a, sh.maxc, n_groups, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

int gemm_rows_per_block(int epi, GemmShape sh) {
  const bool sw = epi == EPI_SWIGLU_F32 || epi == EPI_SWIGLU_FP4;
  return sw ? kNW * (sh.r / 2) * 16 : kNW * sh.r * 16;
}

hipError_t launch_gemm(const GemmArgs& a, int amode, int epi, GemmShape sh, int n_groups, hipStream_t s) {
  // valid (activation, epilogue) pairs
  if (amode == A_BF16 && epi == EPI_Y_BF16) return by_r<A_BF16, EPI_Y_BF16>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_Y_BF16) return by_r<A_FP4, EPI_Y_BF16>(a, sh, n_groups, s);
  if (amode == A_BF16 && epi == EPI_SWIGLU_F32) return by_r<A_BF16, EPI_SWIGLU_F32>(a, sh, n_groups, s);
  if (amode == A_BF16 && epi == EPI_SWIGLU_FP4) return by_r<A_BF16, EPI_SWIGLU_FP4>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SWIGLU_F32) return by_r<A_FP4, EPI_SWIGLU_F32>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SWIGLU_FP4) return by_r<A_FP4, EPI_SWIGLU_FP4>(a, sh, n_groups, s);
  if (amode == A_F32 && epi == EPI_SLOT) return by_r<A_F32, EPI_SLOT>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SLOT) return by_r<A_FP4, EPI_SLOT>(a, sh, n_groups, s);
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
