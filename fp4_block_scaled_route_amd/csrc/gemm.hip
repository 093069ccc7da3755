// Grouped NVFP4 GEMM for gfx950: weight-stationary streaming of packed E2M1
// weights + E4M3 block scales, exact decode to fp16, fp16 MFMA with fp32
// accumulation, fused epilogues (dense bf16 output, SwiGLU with fp32 or NVFP4
// hidden output, scatter of per-pair output rows).
//
// Per group g and weight row n: acc[row, n] = sum_k A[row, k] * E2M1(W[n,k]) * E4M3(S[n,k/16]);
// the product of the two global scales (weight_scale_2 of the group and the
// activation global scale) is applied once, in the epilogue: the block-scaled
// GEMM y = (x*scale_a*gsa) @ (w*scale_b*gsb)^T of page "nvfp4-megamoe-kernel,
// commit 1121cd7 - single_shot_inference.py" (note on the weight-dequant
// global scale).
//
// Common mapping:
//  * a work item is (group, block of weight rows); MoE groups come from a
//    device-side list sorted by size, so no host synchronisation is needed:
//    groups of more than 4 rows go to the LDS kernel, the others to the
//    barrier-free kernels (two launches over the two parts of the list; at
//    large batches, averaging more than 16 rows per group, one launch of the
//    LDS kernel over the whole list).  The
//    dense and grouped linear have fixed groups; their work items also carry
//    a pass of rows and, when they are few, a part of a split K range;
//  * every wave owns R fragments of 16 weight rows and streams them over its
//    K range once per pass of activation rows;
//  * K is walked in chunks of 256.  Lane (r, g) of a fragment (r = lane%16,
//    g = lane/16) holds bytes [32g, 32g+32) of the chunk of row r (64 codes)
//    and the 4 scale bytes of those 4 blocks.  MFMA step q (0..7) covers K
//    positions {64g' + 8q + e}: the MFMA's K index is a permutation of the
//    real K, the same for both operands, so the sum is unchanged;
//  * weights are the MFMA A operand (16 weight rows), activations the B
//    operand (16 rows of tokens): D[weight row][token row];
//  * activations arrive as fp16 rows (bf16 / fp32 values scaled by a per-row
//    power of two into [2^14, 2^15), undone in the epilogue: exact) or as
//    NVFP4 rows (decoded exactly; global scale in the epilogue).
//
// Compact kernel (groups of at most 4 rows, fp16 activations: the decode
// case) and direct kernel (the same with NVFP4 activations): no barriers;
// every wave streams its weights independently, two chunks ahead.
//
// LDS kernel (bigger groups): the workgroup stages the activation chunk
// [16*MAXC rows, 256] into LDS (double buffered) and every wave reads its B
// fragments from there, so the activation rows are fetched once per
// workgroup instead of once per wave.
#include <algorithm>

#include "device_util.h"

namespace nvfp4 {

namespace {

template <int R>
struct WBuf {
  u32x4 c0[R];
  u32x4 c1[R];
  uint32_t s[R];
};

// B fragment of one lane for one chunk: 8 x 8 fp16 (A_F16) or 64 codes + 4 scales (A_FP4)
template <int AM>
struct BBuf;
template <>
struct BBuf<A_F16> {
  u32x4 v[8];
};
template <>
struct BBuf<A_FP4> {
  u32x4 c0, c1;
  uint32_t s;
};

__device__ __forceinline__ uint32_t word_of(const u32x4& a, const u32x4& b, int q) {
  return q < 4 ? a[q & 3] : b[q & 3];
}

template <int EP>
constexpr bool is_swiglu() { return EP == EPI_SWIGLU_F32 || EP == EPI_SWIGLU_FP4; }

template <int R, int NW, int EP>
constexpr int block_rows() { return is_swiglu<EP>() ? NW * (R / 2) * 16 : NW * R * 16; }

constexpr int kNW = 4;  // waves per workgroup
// s_waitcnt operand (gfx9 encoding) waiting for all vector memory loads only
constexpr int kVmcnt0 = 0x0F70;
// Requests for chunks past the end of a work item (the prefetches of its last
// steps) keep their place in the code, so the pipeline has no branches, but
// with this bit in their lane offset they fall outside the buffer resource:
// the hardware returns zeros without touching memory (re-reading the last
// chunk instead cost 2 of every 8 chunks' traffic on short-K items: the
// non-temporal code loads go back to HBM).  The results are never used.
constexpr uint32_t kPast = 0x80000000u;

// Resolved work item.
struct Item {
  int g, row0, m;
  int gl;              // MoE: position in this launch's part of the group list
  int ks;              // K split (grouped linear), else 0
  const uint8_t* W;
  const uint8_t* WS;
  float alpha;
};

__device__ __forceinline__ bool resolve_item(const GemmArgs& a, int gi, Item& it) {
  it.ks = 0;
  if (a.offsets) {
    if (a.mks > 1) {
      const int gi2 = gi / a.mks;
      it.ks = gi - gi2 * a.mks;
      gi = gi2;
    }
    const int lo = a.list_part == 1 ? a.gcount[1] : 0;
    const int hi = a.list_part == 0 ? a.gcount[1] : a.gcount[0];
    it.gl = gi;
    gi += lo;
    if (gi >= hi) return false;
    it.g = a.glist[gi];
    it.row0 = a.offsets[it.g];
    it.m = a.offsets[it.g + 1] - it.row0;
  } else if (a.gl_G) {
    if (a.ksplit > 1) {
      const int gi2 = gi / a.ksplit;
      it.ks = gi - gi2 * a.ksplit;
      gi = gi2;
    }
    const int g = gi / a.gl_npass, p = gi - g * a.gl_npass;
    if (g >= a.gl_G) return false;
    it.g = g;
    it.row0 = g * a.gl_T + p * a.gl_pr;
    it.m = min(a.gl_pr, a.gl_T - p * a.gl_pr);
  } else {
    if (gi > 0) return false;
    it.g = 0;
    it.row0 = 0;
    it.m = a.M;
  }
  if (it.m <= 0) return false;
  const bool shared = it.g >= a.n_routed;
  it.W = shared ? a.sw : a.w + (int64_t)it.g * a.w_gstride;
  it.WS = shared ? a.sw_sf : a.w_sf + (int64_t)it.g * a.sf_gstride;
  it.alpha = shared ? a.sw_ws2[0] : a.w_ws2[it.g];
  if (a.gsa) it.alpha *= a.gsa[0];
  return true;
}

// Activation row (in the A tensor) of sorted row r.
__device__ __forceinline__ int a_row_of(const GemmArgs& a, int r) {
  if (a.gl_G) {
    const int g = r / a.gl_T;
    return (r - g * a.gl_T) * a.gl_G + g;
  }
  if (!a.a_by_token || !a.offsets) return r;
  const int pid = a.perm[r];
  return pid < a.P ? pid / a.topk : pid - a.P;
}

__device__ __forceinline__ int shift_of(const GemmArgs& a, int arow) {
  return a.rowshift ? a.rowshift[arow] : 0;
}

// Weight fragments of this wave, read with buffer loads: one resource per
// group (codes and scales), one 32-bit lane offset shared by all fragments,
// and wave-uniform fragment offsets (scalar registers).
template <int R, int EP, int NW = kNW>
struct Frags {
  int fbase[R];
  bool fvalid[R];
  rsrc_t rw, rs;       // codes [N, K/2], scales [N, K/16] of the group
  uint32_t vw, vs;     // lane offsets: row lr, byte 32*lg (codes) / 4*lg (scales)
  uint32_t sw[R], ss[R];  // fragment offsets (first row of the fragment)
  uint32_t KB, KS;

  __device__ __forceinline__ void init(const GemmArgs& a, const Item& it, int nbk, int wave, int lr, int lg) {
    KB = a.K / 2;
    KS = a.K / 16;
    rw = make_rsrc(it.W, (uint32_t)a.N * KB);
    rs = make_rsrc(it.WS, (uint32_t)a.N * KS);
    vw = lr * KB + lg * 32;
    vs = lr * KS + lg * 4;
#pragma unroll
    for (int f = 0; f < R; ++f) {
      int row0;
      if constexpr (is_swiglu<EP>()) {
        const int gate = nbk * block_rows<R, NW, EP>() + (wave * (R / 2) + (f >> 1)) * 16;
        fbase[f] = gate;
        fvalid[f] = gate < a.I;
        row0 = (f & 1 ? a.I : 0) + gate;
      } else {
        const int base = nbk * block_rows<R, NW, EP>() + (wave * R + f) * 16;
        fbase[f] = base;
        fvalid[f] = base < a.N;
        row0 = base;
      }
      if (!fvalid[f]) row0 = 0;  // stay inside the group; results are discarded
      sw[f] = (uint32_t)row0 * KB;
      ss[f] = (uint32_t)row0 * KS;
    }
  }

  // Codes of a chunk, loaded by whole rows: instruction h reads rows
  // 8h..8h+7 of each fragment, lane l the 16 bytes at 16*(l/8) of row
  // 8h + l%8 (every instruction reads 8 full 128-byte rows; with the
  // non-temporal hint this streams faster than 16 rows read in 16-byte
  // pieces: measured on MI355X, 5% on the decode gate/up GEMM, while the
  // hint alone on the 16-byte pieces is slower); unshuffle_rows then
  // gives every lane the 32 bytes the MFMA layout wants (row l%16, bytes
  // 32*(l/16) .. +32) in c0 (first 16) and c1 (second 16).
  __device__ __forceinline__ void load_codes_rows(u32x4 (&h0)[R], u32x4 (&h1)[R], uint32_t vrow, int kc) const {
#pragma unroll
    for (int f = 0; f < R; ++f) {
      h0[f] = buf_load16_nt(rw, vrow, sw[f] + kc * 128);
      h1[f] = buf_load16_nt(rw, vrow, sw[f] + kc * 128 + 8 * KB);
    }
  }

  // Codes only (scales come from load_scales8).
  __device__ __forceinline__ void load_codes(u32x4 (&c0)[R], u32x4 (&c1)[R], int kc) const {
#pragma unroll
    for (int f = 0; f < R; ++f) {
      c0[f] = buf_load16(rw, vw, sw[f] + kc * 128);
      c1[f] = buf_load16(rw, vw + 16, sw[f] + kc * 128);
    }
  }

  // Scale words of 8 consecutive chunks [8*sc, 8*sc+8): lane group G loads
  // the 16 scale bytes of chunks 8*sc+G and 8*sc+4+G of its row (clamped to
  // the last chunk), both at once, so the row's 128 scale bytes of the group
  // are requested together; transpose4 of raw[f][h] then gives every lane its
  // word of chunks 8*sc+4h .. 8*sc+4h+3.
  __device__ __forceinline__ void load_scales8(u32x4 (&raw)[R][2], int sc, int nkc, int lg, int kbase = 0,
                                               uint32_t past = 0) const {
    const int k0 = kbase + min(8 * sc + lg, nkc - 1);
    const int k1 = kbase + min(8 * sc + 4 + lg, nkc - 1);
#pragma unroll
    for (int f = 0; f < R; ++f) {
      // (down GEMM: with the non-temporal hint, measured 3% faster on MI355X;
      // gate/up: 8% slower with it)
      if constexpr (EP == EPI_SLOT) {
        raw[f][0] = buf_load16_nt(rs, (vs - lg * 4 + k0 * 16) | past, ss[f]);
        raw[f][1] = buf_load16_nt(rs, (vs - lg * 4 + k1 * 16) | past, ss[f]);
      } else {
        raw[f][0] = buf_load16(rs, (vs - lg * 4 + k0 * 16) | past, ss[f]);
        raw[f][1] = buf_load16(rs, (vs - lg * 4 + k1 * 16) | past, ss[f]);
      }
    }
  }

  __device__ __forceinline__ void load(WBuf<R>& wb, int kc, uint32_t past = 0) const {
#pragma unroll
    for (int f = 0; f < R; ++f) {
      wb.c0[f] = buf_load16(rw, vw | past, sw[f] + kc * 128);
      wb.c1[f] = buf_load16(rw, (vw + 16) | past, sw[f] + kc * 128);
      wb.s[f] = buf_load4(rs, vs | past, ss[f] + kc * 16);
    }
  }
};

// From the whole-row code loads (h0: rows 0-7, h1: rows 8-15 of a
// fragment; lane l holds bytes 16*(l/8) .. +16 of row l%8 of each) to the
// MFMA layout (c0, c1: bytes 32*(l/16) .. +16 and +16 .. +32 of row l%16).
// Lanes l and l^8 (bit 3 of l: odd) swap one of their two vectors: the even
// lane keeps its h0 (first half of the segment of row l%8 = l%16) and takes
// the odd lane's h0 (the second half); the odd lane keeps its h1 (second half
// of row 8 + l%8 = l%16) and takes the even lane's h1 (the first half).
__device__ __forceinline__ void unshuffle_rows(u32x4& h0, u32x4& h1, bool odd) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t send = odd ? h0[i] : h1[i];
    // row_ror:8 within each 16-lane row: lane l receives lane l ^ 8
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0x128, 0xF, 0xF, false);
    const uint32_t c0 = odd ? recv : h0[i];
    const uint32_t c1 = odd ? h1[i] : recv;
    h0[i] = c0;
    h1[i] = c1;
  }
}

// 4x4 transpose of dwords across the four 16-lane groups: on entry lane group
// G holds v[j] = X[G][j]; on exit it holds v[c] = X[c][G].
__device__ __forceinline__ void transpose4(u32x4& v) {
  auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// Epilogue for one pass.  acc[f][c]: fragment f, token chunk c; lane holds
// D rows 4*lg..4*lg+3 of the fragment for token row pbase + 16c + lr.
// Rows at or past `mlim` (end of this pass) are not written.
// hgs: the global scale of the NVFP4 h (EPI_SWIGLU_FP4), read by the caller
// before its first store: read here, between the stores, it would have to
// wait for them (the compiler cannot rule out that they alias it).
template <int R, int MAXC, int EP, int NW>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const Item& it, const Frags<R, EP, NW>& fr,
                                         f32x4 (&acc)[R][MAXC], int nc, int pbase, int mlim, int lr, int lg,
                                         float hgs) {
  // Per token chunk c, for this lane's row of the pass: its activation row,
  // power-of-two shift and (EPI_SLOT) pair id, all read before the first
  // store for the reason given for hgs.
  int arow[MAXC], sh[MAXC], pid[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int tr = pbase + 16 * c + lr;
    const bool ok = c < nc && tr < mlim;
    arow[c] = ok ? a_row_of(a, it.row0 + tr) : 0;
    sh[c] = ok ? shift_of(a, arow[c]) : 0;
    pid[c] = EP == EPI_SLOT && ok ? a.perm[it.row0 + tr] : 0;
  }
  // (one wait for them here, while no store is in flight: the compiler
  // would otherwise wait at each use after a branch, with stores pending)
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  if constexpr (EP == EPI_PART_F32) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int tr = pbase + 16 * c + lr;
      if (c >= nc || tr >= mlim) continue;
#pragma unroll
      for (int f = 0; f < R; ++f) {
        if (!fr.fvalid[f]) continue;
        const int n0 = fr.fbase[f] + 4 * lg;
        float4 v;
        v.x = __builtin_ldexpf(acc[f][c][0], -sh[c]) * it.alpha;
        v.y = __builtin_ldexpf(acc[f][c][1], -sh[c]) * it.alpha;
        v.z = __builtin_ldexpf(acc[f][c][2], -sh[c]) * it.alpha;
        v.w = __builtin_ldexpf(acc[f][c][3], -sh[c]) * it.alpha;
        *reinterpret_cast<float4*>(a.part + ((int64_t)it.ks * a.a_rows + arow[c]) * a.N + n0) = v;
      }
    }
  } else if constexpr (EP == EPI_Y_BF16 || EP == EPI_SLOT) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int tr = pbase + 16 * c + lr;
      if (c >= nc || tr >= mlim) continue;
      // The row's values of every fragment first, then its stores back to
      // back, so that no register of a store is rewritten before the next
      // one (output row = activation row for the dense and grouped linear,
      // t * G + g for the latter; the pair's slot row for the MoE).
      uint16_t* const yrow = EP == EPI_Y_BF16 ? a.y + (int64_t)arow[c] * a.N : a.slot + (int64_t)pid[c] * a.N;
      uint2 o[R];
#pragma unroll
      for (int f = 0; f < R; ++f) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_ldexpf(acc[f][c][i], -sh[c]) * it.alpha;
        o[f].x = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
        o[f].y = float_to_bf16_bits(v[2]) | (float_to_bf16_bits(v[3]) << 16);
      }
#pragma unroll
      for (int f = 0; f < R; ++f)
        if (fr.fvalid[f]) *reinterpret_cast<uint2*>(yrow + fr.fbase[f] + 4 * lg) = o[f];
    }
  } else {
    // SwiGLU: fragments 2p (gate rows) and 2p+1 (up rows) share the layout
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c >= nc) continue;  // uniform across the workgroup
      const int tr = pbase + 16 * c + lr;
      const bool tv = tr < mlim;
      const int r = it.row0 + (tv ? tr : 0);
      float hmx = 0.f;
#pragma unroll
      for (int p = 0; p < R / 2; ++p) {
        if (!fr.fvalid[2 * p]) continue;  // uniform across the wave
        const int n0 = fr.fbase[2 * p] + 4 * lg;
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gv = __builtin_ldexpf(acc[2 * p][c][i], -sh[c]) * it.alpha;
          const float uv = __builtin_ldexpf(acc[2 * p + 1][c][i], -sh[c]) * it.alpha;
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
          const float gs = hgs;
          // Scale byte and codes on the hardware converters, which give the
          // software encoders' bytes for every input but a NaN (see
          // quant_block16): a lane whose values or reciprocal scale are not
          // finite takes the software encoders.
          uint32_t sbyte = 0, packed = 0;
          if (gs != 0.0f) {
            sbyte = e4m3_encode_hw(ab / (6.0f * gs));
            const float scale = e4m3_to_float(sbyte) * gs;
            if (scale != 0.0f) {
              const float rcp = 1.0f / scale;
              uint32_t im = 0;
#pragma unroll
              for (int i = 0; i < 4; ++i) im = max(im, __float_as_uint(hv[i]) & 0x7FFFFFFFu);
              if (im < 0x7F800000u && rcp <= 3.402823466e38f) {
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, hv[0] * rcp, hv[1] * rcp, 1.0f, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, hv[2] * rcp, hv[3] * rcp, 1.0f, 1) & 0xFFFFu;
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) packed |= e2m1_encode(hv[i] * rcp) << (4 * i);
              }
            }
          }
          if (tv) {
            *reinterpret_cast<uint16_t*>(a.hq + (int64_t)r * (a.I / 2) + n0 / 2) = (uint16_t)packed;
            if (lg == 0) a.hq_sf[(int64_t)r * (a.I / 16) + fr.fbase[2 * p] / 16] = (uint8_t)sbyte;
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

}  // namespace

// ---------------------------------------------------------------------------
// compact kernel: fp16 activations, at most kSmallRows rows per pass
// ---------------------------------------------------------------------------
//
// Per 256-K chunk a wave issues 2 code loads per fragment (8 whole rows each,
// non-temporal, then a lane-pair swap into the MFMA layout), 1/4 scale load per
// fragment (the scales of 8 chunks come with two loads per fragment issued
// together, so each weight row's 128 scale bytes of the group are fetched
// once; transposed across lane groups) and ceil(rows/2) activation loads:
// lanes 0-31 load 512 bytes of one row, lanes 32-63 of the next.  The
// activation rows go through a wave-private LDS slot (LDS operations of one
// wave complete in order, so no barrier is needed) and are read back in the
// MFMA layout; lanes of absent rows read row 0 (their columns are
// discarded).  Activations are loaded three chunks ahead, weights two chunks
// ahead, scales one 8-chunk group ahead.

constexpr int kSmallRows = 4;
constexpr int kSlotPitch = kChunk * 2 + 64;           // bytes per staged row (bank-shifted)
constexpr int kSlotBytes = kSmallRows * kSlotPitch;   // one chunk of up to 4 rows

template <int R, int EP>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void nvfp4_gemm_compact(const GemmArgs a) {
  static_assert(!is_swiglu<EP>() || (R % 2 == 0), "SwiGLU needs gate/up fragment pairs");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kNW][2][kSlotBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  Item it;
  int gi0, nbk;
  if (a.xcd_order) {
    // workgroup b runs on XCD b % 8; XCD x takes groups x, x + 8, ... with
    // all nb row blocks of a group in a row, so one L2 holds its activations
    const int j = blockIdx.x >> 3;
    gi0 = (j / a.nb) * 8 + (blockIdx.x & 7);
    nbk = j % a.nb;
  } else {
    gi0 = blockIdx.x / a.nb;
    nbk = blockIdx.x % a.nb;
  }
  if (!resolve_item(a, gi0, it)) return;
  Frags<R, EP> fr;
  fr.init(a, it, nbk, wave, lr, lg);
  const float hgs = EP == EPI_SWIGLU_FP4 ? a.h_gs[0] : 0.0f;
  const int K = a.K;
  // chunks of this item: [kbase, kbase + nkc) (all of K unless K is split)
  const int nkc = K / kChunk / (a.ksplit > 1 ? a.ksplit : 1);
  const int kbase = it.ks * nkc;
  const int last = nkc - 1;
  const rsrc_t rb = make_rsrc(a.a, (uint32_t)a.a_rows * K * 2);
  const uint32_t vrow = (lane & 7) * fr.KB + (lane >> 3) * 16;   // whole-row code loads
  uint8_t* slot0 = &lds[wave][0][0];
  uint8_t* slot1 = &lds[wave][1][0];

  const int npass = (it.m + kSmallRows - 1) / kSmallRows;
  for (int pass = 0; pass < npass; ++pass) {
    const int pbase = pass * kSmallRows;
    const int prow = min(kSmallRows, it.m - pbase);
    const bool two = prow > 2;                     // second compact load needed
    // compact load lanes: row (lane/32) and (lane/32)+2 of this pass, 16 bytes at (lane%32)*16
    const int cr0 = lane >> 5, cr1 = cr0 + 2;
    const uint32_t vb0 = cr0 < prow ? (uint32_t)a_row_of(a, it.row0 + pbase + cr0) * K * 2 + (lane & 31) * 16
                                    : 0x80000000u;
    const uint32_t vb1 = cr1 < prow ? (uint32_t)a_row_of(a, it.row0 + pbase + cr1) * K * 2 + (lane & 31) * 16
                                    : 0x80000000u;
    const int wr0 = cr0 * kSlotPitch + (lane & 31) * 16;
    const int wr1 = cr1 * kSlotPitch + (lane & 31) * 16;
    // MFMA-layout read: row lr of the pass (row 0 for absent rows), step-major column
    const int rd = (lr < prow ? lr : 0) * kSlotPitch + lg * 16;

    f32x4 acc[R][1];
#pragma unroll
    for (int f = 0; f < R; ++f) acc[f][0] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 bq0a, bq0b, bq1a, bq1b;   // compact activation loads, two chunks in flight
    // kc past the end: no memory access (kPast)
    auto bload = [&](u32x4& x, u32x4& y, int kc) {
      const uint32_t past = kc > last ? kPast : 0u;
      kc = min(kc, last);
      x = buf_load16(rb, vb0 | past, (kbase + kc) * kChunk * 2);
      if (two) y = buf_load16(rb, vb1 | past, (kbase + kc) * kChunk * 2);
    };
    auto codes = [&](u32x4 (&h0)[R], u32x4 (&h1)[R], int kc) {
      fr.load_codes_rows(h0, h1, kc > last ? vrow | kPast : vrow, kbase + min(kc, last));
    };
    auto bstore = [&](uint8_t* slot, const u32x4& x, const u32x4& y) {
      *reinterpret_cast<u32x4*>(slot + wr0) = x;
      if (two) *reinterpret_cast<u32x4*>(slot + wr1) = y;
    };

    u32x4 wc0a[R], wc1a[R], wc0b[R], wc1b[R];   // codes of two chunks in flight
    u32x4 sraw[R][2];                           // scales of the next 8-chunk group
    u32x4 scur[R][2];                           // this lane's scale word of each chunk of the group

    auto compute = [&](u32x4 (&c0)[R], u32x4 (&c1)[R], const uint8_t* slot, int c8) {
#pragma unroll
      for (int f = 0; f < R; ++f) unshuffle_rows(c0[f], c1[f], (lane >> 3) & 1);
      f16 sc[R][4];
#pragma unroll
      for (int f = 0; f < R; ++f) scales4(scur[f][c8 >> 2][c8 & 3], sc[f]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f16x8 bf = *reinterpret_cast<const f16x8*>(slot + rd + q * 64);
#pragma unroll
        for (int f = 0; f < R; ++f) {
          const f16x8 af = decode8(word_of(c0[f], c1[f], q), sc[f][q >> 1]);
          acc[f][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[f][0], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // prologue
    fr.load_scales8(sraw, 0, nkc, lg, kbase);
    bload(bq0a, bq0b, 0);
    bload(bq1a, bq1b, 1);
    codes(wc0a, wc1a, 0);
    codes(wc0b, wc1b, 1);
    bstore(slot0, bq0a, bq0b);
    bload(bq0a, bq0b, 2);

    // one iteration = one group of 8 chunks; chunk kc uses codes set (kc%2),
    // activation slot (kc%2); at its end the activations of chunk kc+1 are
    // stored to slot ((kc+1)%2) and chunk kc+3 is requested
    for (int kc = 0; kc < nkc; kc += 8) {
#pragma unroll
      for (int f = 0; f < R; ++f) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          scur[f][h] = sraw[f][h];
          transpose4(scur[f][h]);
        }
      }
      fr.load_scales8(sraw, kc / 8 + 1, nkc, lg, kbase, kc + 8 >= nkc ? kPast : 0u);
#pragma unroll
      for (int c8 = 0; c8 < 8; ++c8) {
        const int k = kc + c8;
        if (k >= nkc) break;
        if ((c8 & 1) == 0) {
          compute(wc0a, wc1a, slot0, c8);
          codes(wc0a, wc1a, k + 2);
          bstore(slot1, bq1a, bq1b);
          bload(bq1a, bq1b, k + 3);
        } else {
          compute(wc0b, wc1b, slot1, c8);
          codes(wc0b, wc1b, k + 2);
          bstore(slot0, bq0a, bq0b);
          bload(bq0a, bq0b, k + 3);
        }
      }
    }
    epilogue<R, 1, EP, kNW>(a, it, fr, acc, 1, pbase, pbase + prow, lr, lg, hgs);
  }
}

// ---------------------------------------------------------------------------
// direct kernel: one 16-row activation chunk per pass, no LDS, no barriers
// ---------------------------------------------------------------------------

template <int R, int AM, int EP>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void nvfp4_gemm_direct(const GemmArgs a) {
  static_assert(!is_swiglu<EP>() || (R % 2 == 0), "SwiGLU needs gate/up fragment pairs");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  Item it;
  int gi0, nbk;
  if (a.xcd_order) {
    // workgroup b runs on XCD b % 8; XCD x takes groups x, x + 8, ... with
    // all nb row blocks of a group in a row, so one L2 holds its activations
    const int j = blockIdx.x >> 3;
    gi0 = (j / a.nb) * 8 + (blockIdx.x & 7);
    nbk = j % a.nb;
  } else {
    gi0 = blockIdx.x / a.nb;
    nbk = blockIdx.x % a.nb;
  }
  if (!resolve_item(a, gi0, it)) return;
  Frags<R, EP> fr;
  fr.init(a, it, nbk, wave, lr, lg);
  const float hgs = EP == EPI_SWIGLU_FP4 ? a.h_gs[0] : 0.0f;
  const int K = a.K;
  const int nkc = K / kChunk;

  const int npass = (it.m + 15) >> 4;
  for (int pass = 0; pass < npass; ++pass) {
    const int pbase = pass * 16;
    const int tr = pbase + lr;
    const bool bv = tr < it.m;
    const int arow = bv ? a_row_of(a, it.row0 + tr) : 0;
    // this lane's B fragment source.  Lanes past the group's rows get an
    // offset beyond the buffer: their loads return zeros without touching
    // memory (their MFMA columns are discarded anyway).
    constexpr uint32_t kOut = 0x80000000u;
    rsrc_t rb, rbs;
    uint32_t vb, vbs = 0;
    if constexpr (AM == A_F16) {
      rb = make_rsrc(a.a, (uint32_t)a.a_rows * K * 2);
      vb = bv ? (uint32_t)arow * K * 2 + lg * 16 : kOut;   // step-major rows
    } else {
      rb = make_rsrc(a.a, (uint32_t)a.a_rows * (K / 2));
      rbs = make_rsrc(a.a_sf, (uint32_t)a.a_rows * (K / 16));
      vb = bv ? (uint32_t)arow * (K / 2) + lg * 32 : kOut;
      vbs = bv ? (uint32_t)arow * (K / 16) + lg * 4 : kOut;
    }

    f32x4 acc[R][1];
#pragma unroll
    for (int f = 0; f < R; ++f) acc[f][0] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // B fragments: fp16 rows use a rolling prefetch (the register of step q
    // is refilled with the next chunk's step q right after use); NVFP4 rows
    // are double buffered like the weights.
    BBuf<AM> bb0, bb1;
    auto bload = [&](BBuf<AM>& b, int kc, uint32_t past = 0) {
      if constexpr (AM == A_F16) {
#pragma unroll
        for (int q = 0; q < 8; ++q) b.v[q] = buf_load16(rb, vb | past, kc * kChunk * 2 + q * 64);
      } else {
        b.c0 = buf_load16(rb, vb | past, kc * 128);
        b.c1 = buf_load16(rb, (vb + 16) | past, kc * 128);
        b.s = buf_load4(rbs, vbs | past, kc * 16);
      }
    };

    // next_kc: chunk whose B fragments refill the registers (rolling prefetch
    // for fp16 rows); always a valid chunk, so every load is unconditional
    auto compute = [&](const WBuf<R>& wb, BBuf<AM>& b, int next_kc) {
      f16 sc[R][4];
#pragma unroll
      for (int f = 0; f < R; ++f) scales4(wb.s[f], sc[f]);
      f16 bsc[4];
      if constexpr (AM == A_FP4) scales4(b.s, bsc);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f16x8 bf;
        if constexpr (AM == A_F16) {
          bf = __builtin_bit_cast(f16x8, b.v[q]);
          b.v[q] = buf_load16(rb, vb, next_kc * kChunk * 2 + q * 64);
        } else {
          bf = decode8(word_of(b.c0, b.c1, q), bsc[q >> 1]);
        }
#pragma unroll
        for (int f = 0; f < R; ++f) {
          const f16x8 af = decode8(word_of(wb.c0[f], wb.c1[f], q), sc[f][q >> 1]);
          acc[f][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[f][0], 0, 0, 0);
        }
        // keep each step's decode next to its MFMAs (bounds register pressure;
        // the MFMAs still overlap the next step's VALU decode)
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Prefetch: weights two chunks ahead (wb0 / wb1), B one chunk ahead.
    // Requests past the end keep their place (no branch) but carry kPast:
    // no memory access, results unused.
    const int last = nkc - 1;
    WBuf<R> wb0, wb1;
    auto past = [&](int kc) { return kc > last ? kPast : 0u; };
    fr.load(wb0, 0);
    bload(bb0, 0);
    fr.load(wb1, min(1, last), past(1));
    if constexpr (AM == A_FP4) bload(bb1, min(1, last), past(1));
    for (int kc = 0; kc < nkc; kc += 2) {
      if constexpr (AM == A_F16) {
        compute(wb0, bb0, min(kc + 1, last));
      } else {
        compute(wb0, bb0, 0);
        bload(bb0, min(kc + 2, last), past(kc + 2));
      }
      fr.load(wb0, min(kc + 2, last), past(kc + 2));
      if (kc + 1 >= nkc) break;
      if constexpr (AM == A_F16) {
        compute(wb1, bb0, min(kc + 2, last));
      } else {
        compute(wb1, bb1, 0);
        bload(bb1, min(kc + 3, last), past(kc + 3));
      }
      fr.load(wb1, min(kc + 3, last), past(kc + 3));
    }
    epilogue<R, 1, EP, kNW>(a, it, fr, acc, 1, pbase, min(it.m, pbase + 16), lr, lg, hgs);
  }
}

// ---------------------------------------------------------------------------
// LDS kernel: activation chunks staged per workgroup
// ---------------------------------------------------------------------------

template <int MAXC, int R, int NW, int AM, int EP>
__global__ __launch_bounds__(NW * 64) void nvfp4_gemm_lds(const GemmArgs a) {
  static_assert(!is_swiglu<EP>() || (R % 2 == 0), "SwiGLU needs gate/up fragment pairs");
  constexpr int PR = 16 * MAXC;         // activation rows per pass
  // Staging of the activation chunk, branch-free (rows of the pass past its
  // last row read through an offset beyond the buffer and are not used).
  //  fp16 rows: 32 threads per row, 16 bytes each; lanes 0-31 and 32-63 of a
  //    wave take two rows.
  //  NVFP4 rows: 4 threads per row, each 64 codes (32 bytes) and their 4 scale
  //    bytes, decoded to 128 bytes of fp16; lane l of wave w takes row
  //    16w + l%16, quarter l/16, so 8 consecutive lanes write 8 rows (distinct
  //    LDS banks).
  constexpr int TPR = AM == A_F16 ? 32 : 4;   // threads per staged row
  constexpr int RSTEP = NW * 64 / TPR;        // rows staged per sweep of the workgroup
  constexpr int SROWS = (PR + RSTEP - 1) / RSTEP;
  // four-wave configuration: the weights of two chunks in registers
  constexpr bool DB = NW == 4;
  // B fragments of a whole step read at once (see compute)
  constexpr bool BQ = !(NW == 8 && AM == A_F16);
  // every thread writes its rows (the rows past PR hold zeros nobody reads),
  // so no wave-dependent branch separates the loads from their uses
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][SROWS * RSTEP * kLdsRow];
  // Down GEMM, eight waves: pair ids of the pass's rows (see the epilogue)
  constexpr bool SLOT_TILE = EP == EPI_SLOT && NW == 8 && R == 4;
  __shared__ int s_pid[SLOT_TILE ? PR : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  // Eight-wave configuration: workgroups go to the 8 XCDs in turn (workgroup
  // b to XCD b % 8); XCD x takes groups x, x + 8, ... with all nb row blocks
  // of a group one after another, so the workgroups that read one group's
  // activation rows run together on one XCD and share its L2.  (The grid is
  // a multiple of 8 * nb.)  Four-wave configuration (a few groups): item =
  // b / nb, spread over all XCDs.
  int gi, nbk;
  if constexpr (NW == 8) {
    const int j = blockIdx.x >> 3;
    gi = (j / a.nb) * 8 + (blockIdx.x & 7);
    nbk = j % a.nb;
  } else {
    gi = blockIdx.x / a.nb;
    nbk = blockIdx.x % a.nb;
  }
  Item it;
  if (!resolve_item(a, gi, it)) return;
  Frags<R, EP, NW> fr;
  fr.init(a, it, nbk, wave, lr, lg);
  const float hgs = EP == EPI_SWIGLU_FP4 ? a.h_gs[0] : 0.0f;
  const int K = a.K;
  // chunks of this item: [kbase, kbase + nkc) (all of K unless K is split)
  const int nkc = K / kChunk / (a.ksplit > 1 ? a.ksplit : a.mks > 1 ? a.mks : 1);
  const int kbase = it.ks * nkc;
  const int last = nkc - 1;
  const int seg = AM == A_F16 ? lane & 31 : lg;
  const int rsub = AM == A_F16 ? 2 * wave + (lane >> 5) : 16 * wave + lr;
  const rsrc_t ra = make_rsrc(a.a, AM == A_F16 ? (uint32_t)a.a_rows * K * 2 : (uint32_t)a.a_rows * (K / 2));
  const rsrc_t ras = make_rsrc(a.a_sf, AM == A_F16 ? 0u : (uint32_t)a.a_rows * (K / 16));
  constexpr uint32_t kOut = 0x80000000u;

  const int npass = (it.m + PR - 1) / PR;
  for (int pass = 0; pass < npass; ++pass) {
    const int pbase = pass * PR;
    const int prow = min(PR, it.m - pbase);
    const int nc = __builtin_amdgcn_readfirstlane((prow + 15) >> 4);

    uint32_t so[SROWS], sso[SROWS];   // per-row offsets of codes (or fp16) and scales
#pragma unroll
    for (int i = 0; i < SROWS; ++i) {
      const int rr = rsub + RSTEP * i;
      const bool ok = rr < prow;   // (prow <= PR, so rows of the workgroup past PR load nothing)
      const uint32_t arow = ok ? (uint32_t)a_row_of(a, it.row0 + pbase + rr) : 0u;
      if constexpr (AM == A_F16) {
        so[i] = ok ? arow * (uint32_t)K * 2 + seg * 16 : kOut;
        sso[i] = 0;
      } else {
        so[i] = ok ? arow * (uint32_t)(K / 2) + seg * 32 : kOut;
        sso[i] = ok ? arow * (uint32_t)(K / 16) + seg * 4 : kOut;
      }
    }
    u32x4 st0[SROWS], st1[SROWS];
    uint32_t sts[SROWS];
    // Only the sweeps holding rows of the pass (workgroup-uniform count) are
    // written.  Four-wave configuration: only they load, too.  Eight-wave
    // configuration (one sweep): every lane loads (absent rows read zeros
    // without a memory access).
    const int nsw = __builtin_amdgcn_readfirstlane((prow + RSTEP - 1) / RSTEP);

    // kc past the end: no memory access (kPast)
    auto stage_load = [&](int kc) {
      const uint32_t past = kc > last ? kPast : 0u;
      kc = min(kc, last) + kbase;
#pragma unroll
      for (int i = 0; i < SROWS; ++i) {
        if (DB && i >= nsw) break;
        if constexpr (AM == A_F16) {
          st0[i] = buf_load16(ra, so[i] | past, kc * kChunk * 2);
        } else {
          st0[i] = buf_load16(ra, so[i] | past, kc * 128);
          st1[i] = buf_load16(ra, so[i] | past, kc * 128 + 16);
          sts[i] = buf_load4(ras, sso[i] | past, kc * 16);
        }
      }
    };
    auto stage_write = [&](int buf) {
#pragma unroll
      for (int i = 0; i < SROWS; ++i) {
        if (i >= nsw) break;
        const int rr = rsub + RSTEP * i;
        if constexpr (AM == A_F16) {
          *reinterpret_cast<u32x4*>(&lds[buf][rr * kLdsRow + seg * 16]) = st0[i];
        } else {
          const f16x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sts[i], 1.0f, false);
          const f16x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sts[i], 1.0f, true);
          uint8_t* dst = &lds[buf][rr * kLdsRow + seg * 128];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t w = j < 4 ? st0[i][j] : st1[i][j - 4];
            const f16 sc = j < 2 ? s01[0] : j < 4 ? s01[1] : j < 6 ? s23[0] : s23[1];
            *reinterpret_cast<f16x8*>(dst + j * 16) = decode8(w, sc);
          }
        }
      }
    };

    f32x4 acc[R][MAXC];
#pragma unroll
    for (int f = 0; f < R; ++f)
#pragma unroll
      for (int c = 0; c < MAXC; ++c) acc[f][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Weights.  Four-wave configuration (DB): the codes and scale words of
    // two chunks in registers (wb, wb1), requested a whole chunk ahead.
    // Eight-wave configuration (QUAD, no registers for that): one rolling
    // buffer of codes, whose first 16 bytes per lane (steps 0-3) are refilled
    // with the next chunk's once step 3 has decoded them and the second 16
    // bytes after step 7; scale words by quads of chunks: lane group G loads
    // the 16 scale bytes of chunk 4j + G of its row (all four groups' words of
    // that chunk), and a 4x4 transpose across the lane groups gives every lane
    // its word of the quad's four chunks.  A row's 64 scale bytes of a quad
    // thus come with one request: requests per chunk or per pair of chunks,
    // a few microseconds apart, fetched the 128-byte line again each time
    // under this kernel's streaming load (measured on MI355X: 1.9x and 1.55x
    // the algorithmic bytes of the fully-FP4 gate/up GEMM).
    constexpr bool QUAD = NW == 8;
    WBuf<R> wb, wb1;
    u32x4 sq[R];        // QUAD: scale words of the quad (raw, then transposed)
    uint32_t s3[R];     // QUAD: word of the quad's last chunk, while sq receives the next quad
    auto load_quad = [&](int j, uint32_t past) {   // raw scale bytes of quad j (chunks clamped to the last one)
      const int k = min(4 * j + lg, last);
#pragma unroll
      for (int f = 0; f < R; ++f) sq[f] = buf_load16(fr.rs, (fr.vs - lg * 4 + k * 16) | past, fr.ss[f]);
    };
    const int lane_off = lr * kLdsRow + (AM == A_F16 ? lg * 16 : lg * 128);
    auto item_off = [&](int q, int c) {
      return c * 16 * kLdsRow + (AM == A_F16 ? q * 64 : q * 16);
    };
    // buf: LDS buffer = parity of the chunk; w: its weights; next_kc: chunk
    // whose codes are requested into w while it is consumed (QUAD; past the
    // end: no memory access); j: position of the chunk in its quad (QUAD)
    auto compute = [&](int buf, WBuf<R>& w, int next_kc, int j) {
      const uint32_t npast = next_kc > last ? kPast : 0u;
      next_kc = min(next_kc, last);
      if constexpr (QUAD) {
        if (j == 0) {
#pragma unroll
          for (int f = 0; f < R; ++f) transpose4(sq[f]);
        } else if (j == 3) {
          // the next quad's raw words go to sq, a chunk before they are needed
#pragma unroll
          for (int f = 0; f < R; ++f) s3[f] = sq[f][3];
          load_quad(next_kc / 4, npast);
          __builtin_amdgcn_sched_barrier(0);   // keep the requests here, a chunk ahead
        }
      }
      auto sword = [&](int f) -> uint32_t {
        if constexpr (QUAD) return j == 3 ? s3[f] : sq[f][j & 3];
        else return w.s[f];
      };
      // scale bytes 0-1 (steps 0-3) are converted now, bytes 2-3 at step 4
      f16x2 sc[R];
#pragma unroll
      for (int f = 0; f < R; ++f) sc[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sword(f), 1.0f, false);
      const uint8_t* B = &lds[buf][0] + lane_off;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q == 4) {
#pragma unroll
          for (int f = 0; f < R; ++f) sc[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sword(f), 1.0f, true);
        }
        // B fragments of every token chunk of the step, read before the
        // decode so that the LDS latency hides behind it (chunks past the
        // pass hold rows nobody uses; reading them keeps the number of LDS
        // reads in flight the same on every path).  The eight-wave
        // configuration with fp16 activations has no registers to spare and
        // reads each fragment just before its MFMAs.
        f16x8 bq[MAXC];
        if constexpr (BQ) {
#pragma unroll
          for (int c = 0; c < MAXC; ++c) bq[c] = *reinterpret_cast<const f16x8*>(B + item_off(q, c));
          __builtin_amdgcn_sched_barrier(0);
        }
        f16x8 af[R];
#pragma unroll
        for (int f = 0; f < R; ++f) af[f] = decode8(word_of(w.c0[f], w.c1[f], q), sc[f][(q >> 1) & 1]);
        if (QUAD && q == 3) {
#pragma unroll
          for (int f = 0; f < R; ++f) w.c0[f] = buf_load16(fr.rw, fr.vw | npast, fr.sw[f] + next_kc * 128);
        }
        if (QUAD && q == 7) {
#pragma unroll
          for (int f = 0; f < R; ++f) w.c1[f] = buf_load16(fr.rw, (fr.vw + 16) | npast, fr.sw[f] + next_kc * 128);
        }
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          if (c < nc) {
            const f16x8 b = BQ ? bq[c] : *reinterpret_cast<const f16x8*>(B + item_off(q, c));
#pragma unroll
            for (int f = 0; f < R; ++f)
              acc[f][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[f], b, acc[f][c], 0, 0, 0);
          }
        }
      }
    };

    // Down GEMM, eight waves: the pair id of each row of the pass, requested
    // first and parked in LDS with the first chunk, for the epilogue's
    // stores (a read there would wait for the stores before it).
    int pidv = 0;
    if constexpr (SLOT_TILE) {
      if (tid < prow) pidv = a.perm[it.row0 + pbase + tid];
    }
    // requests for chunks past the end carry kPast (no memory access, unused)
    if constexpr (QUAD) {
      fr.load_codes(wb.c0, wb.c1, 0);
      load_quad(0, 0u);
    } else {
      fr.load(wb, kbase);
    }
    stage_load(0);
    stage_write(0);
    if constexpr (SLOT_TILE) {
      if (tid < prow) s_pid[tid] = pidv;
    }
    __syncthreads();
    // Even chunks in LDS buffer 0, odd ones in buffer 1; every chunk stages
    // the next one (past the end: zeros, into the buffer no wave reads any
    // more).
    if constexpr (QUAD) {
      // quads of chunks (the host uses this configuration when 4 divides
      // the chunk count)
      for (int kc = 0; kc < nkc; kc += 4) {
        stage_load(kc + 1);
        compute(0, wb, kc + 1, 0);
        stage_write(1);
        __syncthreads();
        stage_load(kc + 2);
        compute(1, wb, kc + 2, 1);
        stage_write(0);
        __syncthreads();
        stage_load(kc + 3);
        compute(0, wb, kc + 3, 2);
        stage_write(1);
        __syncthreads();
        stage_load(kc + 4);
        compute(1, wb, kc + 4, 3);
        stage_write(0);
        __syncthreads();
      }
    } else {
      // pairs of chunks; an odd last chunk runs after the loop.  Each half
      // starts by waiting for every load in flight (its own weights,
      // requested a chunk earlier), then requests the next chunk's
      // activations and weights, so the compiler's waits never cover loads
      // that were just issued.
      int kc = 0;
      for (; kc + 1 < nkc; kc += 2) {
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        stage_load(kc + 1);
        fr.load(wb1, kbase + kc + 1);
        compute(0, wb, kc + 1, 0);
        stage_write(1);
        __syncthreads();
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        stage_load(kc + 2);
        fr.load(wb, kbase + min(kc + 2, last), kc + 2 > last ? kPast : 0u);
        compute(1, wb1, kc + 2, 0);
        stage_write(0);
        __syncthreads();
      }
      if (kc < nkc) compute(0, wb, last, 0);
    }
    if constexpr (NW == kNW) {
      if (a.mks > 1) {
        // K split of a MoE item: this split's sums go to mpart; the split
        // that counts itself last adds all of them in split order and runs
        // the epilogue (no split waits for another).  The sums are written
        // and read past the caches and complete (vmcnt(0)) before the count,
        // which is a device-scope atomic.
        __shared__ int s_last;
        const rsrc_t rp = make_rsrc(a.mpart, (uint32_t)((int64_t)a.mks * a.mrows * a.mcols * 4));
        auto mcol = [&](int f) {
          return (is_swiglu<EP>() && (f & 1) ? a.I : 0) + fr.fbase[f] + 4 * lg;
        };
        const uint32_t sstride = (uint32_t)a.mrows * a.mcols * 4;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          const int tr = pbase + 16 * c + lr;
          if (c >= nc || tr >= pbase + prow) continue;
          const uint32_t base = (uint32_t)it.ks * sstride + (uint32_t)(it.row0 + tr) * a.mcols * 4;
#pragma unroll
          for (int f = 0; f < R; ++f)
            if (fr.fvalid[f]) buf_store16_coherent(__builtin_bit_cast(u32x4, acc[f][c]), rp, base + mcol(f) * 4);
        }
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        if (threadIdx.x == 0) {
          const int tile = (it.gl * a.nb + nbk) * a.mpass + pass;
          const bool last_split =
              __hip_atomic_fetch_add(a.mcnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.mks - 1);
          if (last_split) a.mcnt[tile] = 0u;   // every split has counted: ready for the next launch
          s_last = last_split;
        }
        __syncthreads();
        if (!s_last) continue;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          const int tr = pbase + 16 * c + lr;
          if (c >= nc || tr >= pbase + prow) continue;
          const uint32_t base = (uint32_t)(it.row0 + tr) * a.mcols * 4;
#pragma unroll
          for (int f = 0; f < R; ++f) {
            if (!fr.fvalid[f]) continue;
            f32x4 s = __builtin_bit_cast(f32x4, buf_load16_coherent(rp, base + mcol(f) * 4));
            for (int k = 1; k < a.mks; ++k) {
              const f32x4 v = __builtin_bit_cast(f32x4, buf_load16_coherent(rp, k * sstride + base + mcol(f) * 4));
              s[0] += v[0];
              s[1] += v[1];
              s[2] += v[2];
              s[3] += v[3];
            }
            acc[f][c] = s;
          }
        }
      }
    }
    if constexpr (EP == EPI_SLOT && NW == 8 && R == 4) {
      // Down GEMM, eight waves: the workgroup's outputs (the pass's token
      // rows x its 512 weight rows, bf16) go through LDS, so that each row's
      // 1 KB leaves in one store instruction of 16 bytes per lane instead of
      // 16-row x 32-byte pieces (every LDS buffer is free: the last barrier
      // of the K loop has passed).
      constexpr int kTilePitch = 512 * 2 + 16;
      static_assert(PR * kTilePitch <= 2 * SROWS * RSTEP * kLdsRow, "output tile fits the staging buffers");
      static_assert(NW * R * 16 == 512, "512 weight rows per workgroup");
      uint8_t* tile = &lds[0][0];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int tr = 16 * c + lr;   // token row of the pass
        if (c >= nc || pbase + tr >= it.m) continue;
        const int sh = shift_of(a, a_row_of(a, it.row0 + pbase + tr));
#pragma unroll
        for (int f = 0; f < R; ++f) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = __builtin_ldexpf(acc[f][c][i], -sh) * it.alpha;
          uint2 o;
          o.x = float_to_bf16_bits(v[0]) | (float_to_bf16_bits(v[1]) << 16);
          o.y = float_to_bf16_bits(v[2]) | (float_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(tile + tr * kTilePitch + ((wave * R + f) * 16 + 4 * lg) * 2) = o;
        }
      }
      __syncthreads();
      const int n0 = nbk * 512 + lane * 8;
      for (int tr = wave; tr < prow; tr += NW) {
        const int pid = s_pid[tr];
        const u32x4 o = *reinterpret_cast<const u32x4*>(tile + tr * kTilePitch + lane * 16);
        if (n0 < a.N) *reinterpret_cast<u32x4*>(a.slot + (int64_t)pid * a.N + n0) = o;
      }
      if (pass + 1 < npass) __syncthreads();   // the next pass stages into these buffers
    } else {
      epilogue<R, MAXC, EP, NW>(a, it, fr, acc, nc, pbase, pbase + prow, lr, lg, hgs);
    }
  }
}

// ---------------------------------------------------------------------------
// skinny kernel: at most 4 activation rows per group, one launch per call
// ---------------------------------------------------------------------------
//
// The dense and grouped linear at decode sizes read a few MB to tens of MB of
// weights once, so a call is one pass of the memory system plus launch
// costs.  A compute unit keeps only so many loads in flight and a memory
// round trip under load takes microseconds, so every wave requests its
// whole share at once and computes chunk by chunk as the data arrives.
//  * Work item (workgroup) = (group, R fragments of 16 weight rows); its
//    sk_kp <= 16 waves split K into ranges of U <= 4 chunks (the last may
//    be shorter), as short as the waves and the LDS allow.
//  * Each activation chunk of the group's T <= 4 rows is converted in the
//    wave's own LDS slots, so no wave waits for another until the end: bf16
//    rows are scaled by the power of two that takes the row's maximum over
//    the chunk into [2^14, 2^15) (exact for values within 29 binades of it);
//    the chunk's MFMA sums start from zero and are added to the fp32 total
//    with that power of two undone (exact scaling, one fp32 addition per
//    chunk).  NVFP4 rows are decoded exactly (no shift).
//  * The range totals of a fragment meet in LDS and are added in range
//    order; the global scales multiply the sum.
constexpr int kSkinnyRows = 4;
constexpr int kSkinnyMaxWaves = 16;
constexpr int kSkinnyLds = 64 * 1024;
constexpr int kSkinnyPitch = kChunk * 2 + 64;   // LDS bytes per staged row of a chunk (rows 16 banks apart)

// Max over each 16-lane row of the wave; every lane gets its row's max.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror:8
  return v;
}

template <int R>
struct SkW {
  u32x4 h0[R], h1[R];   // codes of a chunk, whole rows (rows 0-7, 8-15 of the fragment)
  uint32_t s[R];        // this lane's scale word of the chunk
};

template <int R, int U, int AM>
__global__ __launch_bounds__(kSkinnyMaxWaves * 64) void nvfp4_gemm_skinny(const GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sk[];
  const int lane = threadIdx.x & 63;
  const int kp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // this wave's range
  const int lr = lane & 15, lg = lane >> 4;
  const int KP = a.sk_kp;
  const int g = blockIdx.x / a.nb, nbk = blockIdx.x - g * a.nb;
  const int G = a.gl_G, T = a.gl_T;   // activation and output row of token t: t * G + g
  const int K = a.K, nkc = K / kChunk;
  const int c0 = kp * U;
  const int cnt = min(U, nkc - c0);   // >= 1 by the plan

  // weights
  const uint32_t KB = K / 2, KS = K / 16;
  const rsrc_t rw = make_rsrc(a.w + (int64_t)g * a.w_gstride, (uint32_t)a.N * KB);
  const rsrc_t rs = make_rsrc(a.w_sf + (int64_t)g * a.sf_gstride, (uint32_t)a.N * KS);
  const uint32_t vrow = (lane & 7) * KB + (lane >> 3) * 16;   // whole-row code loads
  const uint32_t vs = lr * KS + lg * 4;
  int fbase[R];
  bool fvalid[R];
  uint32_t sw[R], ss[R];
#pragma unroll
  for (int f = 0; f < R; ++f) {
    fbase[f] = (nbk * R + f) * 16;
    fvalid[f] = fbase[f] < a.N;
    const uint32_t row0 = fvalid[f] ? (uint32_t)fbase[f] : 0u;
    sw[f] = row0 * KB;
    ss[f] = row0 * KS;
  }

  // activations: bf16 x0 = rows 0, 1 (lanes 0-31, 32-63; 8 values at column
  // 8 * (lane % 32)), x1 = rows 2, 3 (requested only when T > 2).  NVFP4:
  // x0 = codes (lanes 0-31: row lane / 8, 32 codes at 32 * (lane % 8)), x1[0]
  // = scales (lanes 32-47: row (lane - 32) / 4, blocks 4 * (lane % 4) ..).
  // Rows past T: no memory access, zeros.
  const uint32_t rowb = AM == A_F16 ? K * 2 : K / 2;
  const rsrc_t rx = make_rsrc(a.a, (uint32_t)a.a_rows * rowb);
  const rsrc_t rxs = make_rsrc(a.a_sf, AM == A_F16 ? 0u : (uint32_t)a.a_rows * KS);
  uint32_t vx0, vx1;
  if constexpr (AM == A_F16) {
    const int r0 = lane >> 5, r1 = r0 + 2;
    vx0 = r0 < T ? (uint32_t)(r0 * G + g) * rowb + (lane & 31) * 16 : kPast;
    vx1 = r1 < T ? (uint32_t)(r1 * G + g) * rowb + (lane & 31) * 16 : kPast;
  } else {
    const int rq = lane >> 3, rsr = (lane - 32) >> 2;
    vx0 = lane < 32 && rq < T ? (uint32_t)(rq * G + g) * rowb + (lane & 7) * 16 : kPast;
    vx1 = lane >= 32 && lane < 48 && rsr < T ? (uint32_t)(rsr * G + g) * KS + (lane & 3) * 4 : kPast;
  }

  // every load of the range at once, chunk by chunk, activations first
  SkW<R> w[U];
  u32x4 x0[U], x1[U];
#pragma unroll
  for (int c = 0; c < U; ++c) {
    const uint32_t past = c < cnt ? 0u : kPast;
    const int kc = c0 + min(c, cnt - 1);
    if constexpr (AM == A_F16) {
      x0[c] = buf_load16(rx, vx0 | past, kc * (kChunk * 2));
      if (T > 2) x1[c] = buf_load16(rx, vx1 | past, kc * (kChunk * 2));
    } else {
      x0[c] = buf_load16(rx, vx0 | past, kc * (kChunk / 2));
      x1[c][0] = buf_load4(rxs, vx1 | past, kc * 16);
    }
#pragma unroll
    for (int f = 0; f < R; ++f) {
      w[c].h0[f] = buf_load16_nt(rw, vrow | past, sw[f] + kc * 128);
      w[c].h1[f] = buf_load16_nt(rw, vrow | past, sw[f] + kc * 128 + 8 * KB);
      w[c].s[f] = buf_load4(rs, vs | past, ss[f] + kc * 16);
    }
  }

  // the wave's two slots of T staged rows
  uint8_t* slots[2] = {sk + kp * (2 * T * kSkinnyPitch), sk + kp * (2 * T * kSkinnyPitch) + T * kSkinnyPitch};
  // stage one chunk; sh[r] = shift of row r (bf16)
  auto stage = [&](uint8_t* slot, const u32x4& v0, const u32x4& v1, int (&sh)[kSkinnyRows]) {
    if constexpr (AM == A_F16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 1 && T <= 2) {
          sh[2] = sh[3] = 0;
          break;
        }
        const u32x4& v = h == 0 ? v0 : v1;
        uint32_t mx = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(v[e] & 0x7FFFu, (v[e] >> 16) & 0x7FFFu));
        mx = row16_max(mx);
        const uint32_t m0 = max((uint32_t)__builtin_amdgcn_readlane((int)mx, 0), (uint32_t)__builtin_amdgcn_readlane((int)mx, 16));
        const uint32_t m1 = max((uint32_t)__builtin_amdgcn_readlane((int)mx, 32), (uint32_t)__builtin_amdgcn_readlane((int)mx, 48));
        sh[2 * h] = shift_from_maxbits(m0 << 16);
        sh[2 * h + 1] = shift_from_maxbits(m1 << 16);
        const int row = 2 * h + (lane >> 5);
        const int s = lane < 32 ? sh[2 * h] : sh[2 * h + 1];
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = (f16)__builtin_ldexpf(bf16_bits_to_float(v[e] & 0xFFFFu), s);
          o[2 * e + 1] = (f16)__builtin_ldexpf(bf16_bits_to_float(v[e] >> 16), s);
        }
        if (row < T) *reinterpret_cast<f16x8*>(slot + row * kSkinnyPitch + step_major_pos((lane & 31) * 8) * 2) = o;
      }
    } else {
      // lane l < 32 decodes 32 codes of row l / 8 (blocks 2p, 2p+1, p = l % 8);
      // their scale bytes sit in lane 32 + 4 * row + p / 2, half p % 2
      const int rq = lane >> 3, p = lane & 7;
      const uint32_t sw4 = (uint32_t)__shfl((int)v1[0], 32 + 4 * (rq & 3) + (p >> 1));
      const uint32_t sb = (p & 1) ? sw4 >> 16 : sw4 & 0xFFFFu;
      const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
      if (lane < 32 && rq < T) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f16x8*>(slot + rq * kSkinnyPitch + step_major_pos(p * 32 + 8 * j) * 2) =
              decode8(v0[j], s2[j >> 1]);
      }
#pragma unroll
      for (int r = 0; r < kSkinnyRows; ++r) sh[r] = 0;
    }
  };

  f32x4 acc[R];
#pragma unroll
  for (int f = 0; f < R; ++f) acc[f] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int rd = (lr < T ? lr : 0) * kSkinnyPitch + lg * 16;   // token columns past T read row 0 (discarded)
  auto compute = [&](SkW<R>& wc, const uint8_t* slot, const int (&sh)[kSkinnyRows]) {
#pragma unroll
    for (int f = 0; f < R; ++f) unshuffle_rows(wc.h0[f], wc.h1[f], (lane >> 3) & 1);
    f16 sc[R][4];
#pragma unroll
    for (int f = 0; f < R; ++f) scales4(wc.s[f], sc[f]);
    f32x4 c[R];
#pragma unroll
    for (int f = 0; f < R; ++f) c[f] = AM == A_F16 ? (f32x4){0.f, 0.f, 0.f, 0.f} : acc[f];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f16x8 bf = *reinterpret_cast<const f16x8*>(slot + rd + q * 64);
#pragma unroll
      for (int f = 0; f < R; ++f) {
        const f16x8 af = decode8(word_of(wc.h0[f], wc.h1[f], q), sc[f][q >> 1]);
        c[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, c[f], 0, 0, 0);
      }
    }
    if constexpr (AM == A_F16) {
      const int s = lr == 0 ? sh[0] : lr == 1 ? sh[1] : lr == 2 ? sh[2] : sh[3];
#pragma unroll
      for (int f = 0; f < R; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][i] += __builtin_ldexpf(c[f][i], -s);
    } else {
#pragma unroll
      for (int f = 0; f < R; ++f) acc[f] = c[f];
    }
  };

  // chunk c in slot c % 2; chunk c + 1 is staged before chunk c is computed
  int sh[2][kSkinnyRows];
  stage(slots[0], x0[0], x1[0], sh[0]);
#pragma unroll
  for (int c = 0; c < U; ++c) {
    if (c >= cnt) break;
    if (c + 1 < U && c + 1 < cnt) stage(slots[(c + 1) & 1], x0[c + 1], x1[c + 1], sh[(c + 1) & 1]);
    compute(w[c], slots[c & 1], sh[c & 1]);
  }

  float alpha = a.w_ws2[g];
  if (a.gsa) alpha *= a.gsa[0];
  auto store = [&](int f, const f32x4& v) {
    uint2 o;
    o.x = float_to_bf16_bits(v[0] * alpha) | (float_to_bf16_bits(v[1] * alpha) << 16);
    o.y = float_to_bf16_bits(v[2] * alpha) | (float_to_bf16_bits(v[3] * alpha) << 16);
    *reinterpret_cast<uint2*>(a.y + (int64_t)(lr * G + g) * a.N + fbase[f] + 4 * lg) = o;
  };
  if (KP == 1) {
    if (lr < T) {
#pragma unroll
      for (int f = 0; f < R; ++f)
        if (fvalid[f]) store(f, acc[f]);
    }
    return;
  }
  // the range totals of each fragment, added in range order
  __syncthreads();   // every wave is done with its slots
  f32x4* red = reinterpret_cast<f32x4*>(sk);
#pragma unroll
  for (int f = 0; f < R; ++f) red[(f * KP + kp) * 64 + lane] = acc[f];
  __syncthreads();
  if (kp != 0 || lr >= T) return;
#pragma unroll
  for (int f = 0; f < R; ++f) {
    if (!fvalid[f]) continue;
    f32x4 v = red[f * KP * 64 + lane];
    for (int j = 1; j < KP; ++j) {
      const f32x4 q = red[(f * KP + j) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += q[i];
    }
    store(f, v);
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

namespace {

template <int AM, int EP, int R>
hipError_t launch_direct(const GemmArgs& a, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (a.xcd_order) n_items = (n_items / a.nb + 7) / 8 * 8 * a.nb;   // whole rounds of 8 groups
  if constexpr (AM == A_F16)
    hipLaunchKernelGGL((nvfp4_gemm_compact<R, EP>), dim3(n_items), dim3(kNW * 64), 0, s, a);
  else
    hipLaunchKernelGGL((nvfp4_gemm_direct<R, AM, EP>), dim3(n_items), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

template <int AM, int EP, int R>
hipError_t launch_lds(const GemmArgs& a, int maxc, int nw, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (nw == 8 && maxc == 7 && R == 4) {
    if (a.K % (4 * kChunk) != 0) return hipErrorInvalidValue;   // quads of chunks
    // whole rounds of 8 groups (see the XCD order in the kernel)
    const int n_groups = n_items / a.nb;
    const int grid = (n_groups + 7) / 8 * 8 * a.nb;
    hipLaunchKernelGGL((nvfp4_gemm_lds<7, R, 8, AM, EP>), dim3(grid), dim3(8 * 64), 0, s, a);
    return hipGetLastError();
  }
  if (nw != kNW) return hipErrorInvalidValue;
  switch (maxc) {
    case 2: hipLaunchKernelGGL((nvfp4_gemm_lds<2, R, kNW, AM, EP>), dim3(n_items), dim3(kNW * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((nvfp4_gemm_lds<4, R, kNW, AM, EP>), dim3(n_items), dim3(kNW * 64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((nvfp4_gemm_lds<8, R, kNW, AM, EP>), dim3(n_items), dim3(kNW * 64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int AM, int EP>
hipError_t dispatch(const GemmArgs& a, GemmShape sh, int n_groups, hipStream_t s) {
  const int n_items = n_groups * a.nb;
  if (sh.maxc == 1) {
    // barrier-free kernels: 2 fragments per wave (4 would not fit the
    // register budget of 4 waves per SIMD)
    if (sh.r != 2) return hipErrorInvalidValue;
    return launch_direct<AM, EP, 2>(a, n_items, s);
  }
  switch (sh.r) {
    case 2: return launch_lds<AM, EP, 2>(a, sh.maxc, sh.nw, n_items, s);
    case 4: return launch_lds<AM, EP, 4>(a, sh.maxc, sh.nw, n_items, s);
    default: return hipErrorInvalidValue;
  }
}

__global__ __launch_bounds__(256) void nvfp4_split_reduce(const float4* part, int S, int64_t n4, uint2* y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float4 v = part[i];
  for (int s = 1; s < S; ++s) {
    const float4 u = part[(int64_t)s * n4 + i];
    v.x += u.x;
    v.y += u.y;
    v.z += u.z;
    v.w += u.w;
  }
  uint2 o;
  o.x = float_to_bf16_bits(v.x) | (float_to_bf16_bits(v.y) << 16);
  o.y = float_to_bf16_bits(v.z) | (float_to_bf16_bits(v.w) << 16);
  y[i] = o;
}

}  // namespace

hipError_t launch_split_reduce(const float* part, int S, int64_t n, uint16_t* y, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(nvfp4_split_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float4*>(part), S, n4, reinterpret_cast<uint2*>(y));
  return hipGetLastError();
}

SkinnyPlan skinny_plan(int64_t T, int64_t G, int64_t N, int64_t K, bool fp4) {
  SkinnyPlan p;
  (void)fp4;   // both activation forms stage the same fp16 slots
  if (T < 1 || T > kSkinnyRows || G < 1 || N < 16 || N % 16 != 0 || K < kChunk || K % kChunk != 0) return p;
  const int64_t nkc = K / kChunk, nfrag = N / 16;
  // The shortest ranges the 16 waves of a workgroup and its LDS allow (one
  // chunk per wave up to 16 chunks; measured on MI355X, more waves with less
  // each beat fewer waves with all of K requested at once); one fragment per
  // wave unless that gives more than about 16 waves per compute unit.
  constexpr int64_t kWaveCap = 4096;
  for (int64_t u = 1; u <= 4 && !p.kp_ok(); ++u) {
    const int64_t kp = (nkc + u - 1) / u;
    if (kp <= kSkinnyMaxWaves && kp * 2 * T * kSkinnyPitch <= kSkinnyLds && kp * 2 * 64 * 16 <= kSkinnyLds) {
      p.u = (int)((nkc + kp - 1) / kp);
      p.kp = (int)kp;
    }
  }
  if (!p.kp_ok()) return p;
  p.r = G * nfrag * p.kp > kWaveCap && nfrag >= 2 ? 2 : 1;
  p.nb = (int)((nfrag + p.r - 1) / p.r);
  p.lds = (int)std::max<int64_t>((int64_t)p.kp * 2 * T * kSkinnyPitch, p.kp > 1 ? (int64_t)p.kp * p.r * 64 * 16 : 0);
  p.ok = G * p.nb < ((int64_t)1 << 31);
  return p;
}

namespace {
template <int R, int AM>
hipError_t launch_skinny_u(const GemmArgs& a, int u, dim3 grid, dim3 block, int lds, hipStream_t s) {
  switch (u) {
    case 1: hipLaunchKernelGGL((nvfp4_gemm_skinny<R, 1, AM>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((nvfp4_gemm_skinny<R, 2, AM>), grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((nvfp4_gemm_skinny<R, 3, AM>), grid, block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((nvfp4_gemm_skinny<R, 4, AM>), grid, block, lds, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, int amode, const SkinnyPlan& p, hipStream_t s) {
  const int64_t nkc = a.K / kChunk;
  if (!p.ok || a.gl_T < 1 || a.gl_T > kSkinnyRows || a.gl_G < 1 || a.sk_kp != p.kp || a.sk_u != p.u ||
      a.nb != p.nb || p.u < 1 || p.u > 4 || p.kp < 1 || p.kp > kSkinnyMaxWaves ||
      (int64_t)(p.kp - 1) * p.u >= nkc || (int64_t)p.kp * p.u < nkc || p.lds > kSkinnyLds ||
      (int64_t)p.kp * 2 * a.gl_T * kSkinnyPitch > p.lds || (p.kp > 1 && p.kp * p.r * 64 * 16 > p.lds) ||
      (int64_t)p.nb * p.r * 16 < a.N || (p.r != 1 && p.r != 2))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.gl_G * p.nb)), block((unsigned)(p.kp * 64));
  if (amode == A_F16) {
    return p.r == 1 ? launch_skinny_u<1, A_F16>(a, p.u, grid, block, p.lds, s)
                    : launch_skinny_u<2, A_F16>(a, p.u, grid, block, p.lds, s);
  }
  if (amode == A_FP4) {
    return p.r == 1 ? launch_skinny_u<1, A_FP4>(a, p.u, grid, block, p.lds, s)
                    : launch_skinny_u<2, A_FP4>(a, p.u, grid, block, p.lds, s);
  }
  return hipErrorInvalidValue;
}

int gemm_rows_per_block(int epi, GemmShape sh) {
  const bool sw = epi == EPI_SWIGLU_F32 || epi == EPI_SWIGLU_FP4;
  return sw ? sh.nw * (sh.r / 2) * 16 : sh.nw * sh.r * 16;
}

hipError_t launch_gemm(const GemmArgs& a, int amode, int epi, GemmShape sh, int n_groups, hipStream_t s) {
  if (amode == A_F16 && epi == EPI_Y_BF16) return dispatch<A_F16, EPI_Y_BF16>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_Y_BF16) return dispatch<A_FP4, EPI_Y_BF16>(a, sh, n_groups, s);
  if (amode == A_F16 && epi == EPI_SWIGLU_F32) return dispatch<A_F16, EPI_SWIGLU_F32>(a, sh, n_groups, s);
  if (amode == A_F16 && epi == EPI_SWIGLU_FP4) return dispatch<A_F16, EPI_SWIGLU_FP4>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SWIGLU_F32) return dispatch<A_FP4, EPI_SWIGLU_F32>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SWIGLU_FP4) return dispatch<A_FP4, EPI_SWIGLU_FP4>(a, sh, n_groups, s);
  if (amode == A_F16 && epi == EPI_SLOT) return dispatch<A_F16, EPI_SLOT>(a, sh, n_groups, s);
  if (amode == A_FP4 && epi == EPI_SLOT) return dispatch<A_FP4, EPI_SLOT>(a, sh, n_groups, s);
  if (epi == EPI_PART_F32) {
    // K splits run on the four-wave LDS kernel and the compact kernel
    if (sh.nw != kNW || a.ksplit < 1 || (sh.maxc == 1 && amode != A_F16)) return hipErrorInvalidValue;
    if (amode == A_F16) return dispatch<A_F16, EPI_PART_F32>(a, sh, n_groups, s);
    if (amode == A_FP4) return dispatch<A_FP4, EPI_PART_F32>(a, sh, n_groups, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
