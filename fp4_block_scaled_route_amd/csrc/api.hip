// C ABI of libnvfp4.so: argument validation, workspace layout and launches.
// Declarations and the contract of every entry point are in include/nvfp4.h.
#include <algorithm>
#include <cstdint>

#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int kMaxExperts = 512;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

// Number of 16-row activation chunks a group pass holds, from the expected rows per group.
int pick_maxc(double rows_per_group) {
  const double want = rows_per_group * 1.25 / 16.0;
  if (want <= 1.0) return 1;
  if (want <= 2.0) return 2;
  if (want <= 4.0) return 4;
  return 8;
}

// Workspace layout of nvfp4_moe_grouped.
struct MoeLayout {
  size_t offsets, glist, gcount, perm, inv, rowshift, hmax, h, hq, hq_sf, slot, total;
};

MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int has_shared, int h_fp4) {
  const int64_t S = has_shared ? 1 : 0;
  const int64_t Pt = T * topk + S * T;
  MoeLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = round_up(off + bytes, 256); return o; };
  L.offsets = take(sizeof(int32_t) * (E + 2));
  L.glist = take(sizeof(int32_t) * (E + 1));
  L.gcount = take(sizeof(int32_t));
  L.perm = take(sizeof(int32_t) * Pt);
  L.inv = take(sizeof(int32_t) * Pt);
  L.rowshift = take(sizeof(int32_t) * T);
  L.hmax = take(sizeof(uint32_t) * Pt);
  if (h_fp4) {
    L.h = 0;
    L.hq = take((size_t)Pt * (I / 2));
    L.hq_sf = take((size_t)Pt * (I / 16));
  } else {
    L.h = take(sizeof(float) * (size_t)Pt * I);
    L.hq = L.hq_sf = 0;
  }
  L.slot = take(sizeof(float) * (size_t)Pt * H);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case NVFP4_ERR_ALIGN: return "a pointer is not aligned as required";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_LAUNCH: return "a kernel launch failed";
    case NVFP4_ERR_ARG: return "incompatible combination of optional arguments";
    default: return "unknown status";
  }
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

int nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, float* gs, int compute_gs, uint8_t* x_fp4,
                       uint8_t* x_sf, void* stream) {
  if (M < 0 || K <= 0 || K % 16 != 0 || M >= kMaxDim || K >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (!gs) return NVFP4_ERR_NULL;
  if (!aligned(gs, 4)) return NVFP4_ERR_ALIGN;
  if (M > 0) {
    if (!x_bf16 || !x_fp4 || !x_sf) return NVFP4_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(x_fp4, 8)) return NVFP4_ERR_ALIGN;
  }
  return launch_status(launch_quantize_act(static_cast<const uint16_t*>(x_bf16), M, K, gs, compute_gs, x_fp4,
                                           x_sf, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return M > 0 ? round_up(sizeof(int32_t) * (size_t)M, 256) : 0;
}

int nvfp4_linear(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa,
                 const uint8_t* w_fp4, const uint8_t* w_sf, const float* gsb, int64_t M, int64_t N, int64_t K,
                 void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (K % 256 != 0 || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M == 0) return NVFP4_OK;
  const bool fp4 = x_fp4 != nullptr;
  if (fp4 && (x_bf16 || !x_sf || !gsa)) return x_bf16 ? NVFP4_ERR_ARG : NVFP4_ERR_NULL;
  if (!fp4 && (!x_bf16)) return NVFP4_ERR_NULL;
  if (!fp4 && (x_sf || gsa)) return NVFP4_ERR_ARG;
  if (!w_fp4 || !w_sf || !gsb || !y_bf16) return NVFP4_ERR_NULL;
  if (!aligned(w_fp4, 16) || !aligned(w_sf, 16) || !aligned(gsb, 4) || !aligned(y_bf16, 16)) return NVFP4_ERR_ALIGN;
  if (fp4 && (!aligned(x_fp4, 16) || !aligned(x_sf, 16) || !aligned(gsa, 4))) return NVFP4_ERR_ALIGN;
  if (!fp4 && !aligned(x_bf16, 16)) return NVFP4_ERR_ALIGN;
  const size_t need = nvfp4_linear_workspace_size(M, N, K);
  if (!fp4 && need > 0) {
    if (!workspace || workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* rowshift = static_cast<int*>(workspace);
  if (!fp4) {
    hipError_t e = launch_rowshift_bf16(static_cast<const uint16_t*>(x_bf16), (int)M, (int)K, rowshift, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  GemmArgs g{};
  g.w = w_fp4;
  g.w_sf = w_sf;
  g.w_ws2 = gsb;
  g.n_routed = 1;
  g.N = (int)N;
  g.K = (int)K;
  g.M = (int)M;
  g.a = fp4 ? static_cast<const void*>(x_fp4) : x_bf16;
  g.a_sf = x_sf;
  g.rowshift = rowshift;
  g.gsa = fp4 ? gsa : nullptr;
  g.y = static_cast<uint16_t*>(y_bf16);
  const int amode = fp4 ? A_FP4 : A_BF16;
  GemmShape sh{pick_maxc((double)M), 2};
  const int rows = gemm_rows_per_block(EPI_Y_BF16, sh);
  g.nb = (int)((N + rows - 1) / rows);
  return launch_status(launch_gemm(g, amode, EPI_Y_BF16, sh, 1, s));
}

size_t nvfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int has_shared,
                                int h_fp4) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  return moe_layout(T, H, I, E, topk, has_shared, h_fp4).total;
}

int nvfp4_moe_grouped(const nvfp4_moe_args* a, void* stream) {
  if (!a) return NVFP4_ERR_NULL;
  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, k = a->topk;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return NVFP4_ERR_SHAPE;
  if (H % 256 != 0 || I % 256 != 0 || E > kMaxExperts || k > E) return NVFP4_ERR_SHAPE;
  if (T >= kMaxDim || H >= kMaxDim || I >= kMaxDim || T * k + T >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  const bool fp4 = a->x_fp4 != nullptr;
  const bool has_shared = a->s1 != nullptr;
  const bool h_fp4 = a->a2_gs != nullptr;
  if (fp4 && (a->x || !a->x_sf || !a->a1_gs)) return a->x ? NVFP4_ERR_ARG : NVFP4_ERR_NULL;
  if (!fp4 && !a->x) return NVFP4_ERR_NULL;
  if (!fp4 && (a->x_sf || a->a1_gs)) return NVFP4_ERR_ARG;
  if (h_fp4 && a->a2_gs_out) return NVFP4_ERR_ARG;
  if (!a->topk_ids || !a->topk_w || !a->w1 || !a->w1_sf || !a->w1_ws2 || !a->w2 || !a->w2_sf || !a->w2_ws2 ||
      !a->y)
    return NVFP4_ERR_NULL;
  if (has_shared && (!a->s1_sf || !a->s1_ws2 || !a->s2 || !a->s2_sf || !a->s2_ws2)) return NVFP4_ERR_NULL;
  if (!has_shared && (a->s1_sf || a->s1_ws2 || a->s2 || a->s2_sf || a->s2_ws2)) return NVFP4_ERR_ARG;
  const void* p16[] = {a->x, a->x_fp4, a->x_sf, a->w1, a->w1_sf, a->w2, a->w2_sf, a->s1, a->s1_sf,
                       a->s2, a->s2_sf, a->y};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return NVFP4_ERR_ALIGN;
  const void* p4[] = {a->a1_gs, a->a2_gs, a->a2_gs_out, a->topk_ids, a->topk_w, a->w1_ws2, a->w2_ws2,
                      a->s1_ws2, a->s2_ws2, a->offsets_out, a->perm_out};
  for (const void* p : p4)
    if (p && !aligned(p, 4)) return NVFP4_ERR_ALIGN;
  const MoeLayout L = moe_layout(T, H, I, E, k, has_shared, h_fp4);
  if (!a->workspace || a->workspace_bytes < L.total) return NVFP4_ERR_WORKSPACE;
  if (!aligned(a->workspace, 256)) return NVFP4_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  int* offsets = reinterpret_cast<int*>(ws + L.offsets);
  int* glist = reinterpret_cast<int*>(ws + L.glist);
  int* gcount = reinterpret_cast<int*>(ws + L.gcount);
  int* perm = reinterpret_cast<int*>(ws + L.perm);
  int* inv = reinterpret_cast<int*>(ws + L.inv);
  int* rowshift = reinterpret_cast<int*>(ws + L.rowshift);
  unsigned* hmax = reinterpret_cast<unsigned*>(ws + L.hmax);
  float* slot = reinterpret_cast<float*>(ws + L.slot);
  const int S = has_shared ? 1 : 0;
  const int P = (int)(T * k);
  const int Pt = P + S * (int)T;
  const int G = (int)E + S;
  auto ev = [&](int i) {
    if (a->stage_events) (void)hipEventRecord(static_cast<hipEvent_t>(a->stage_events[i]), s);
  };

  // 1. permutation, group order, bf16 row shifts, clearing of the h row maxima
  ev(0);
  PermuteArgs pa{};
  pa.ids = a->topk_ids;
  pa.T = (int)T;
  pa.topk = (int)k;
  pa.E = (int)E;
  pa.shared = S;
  pa.offsets = offsets;
  pa.perm = perm;
  pa.inv = inv;
  pa.glist = glist;
  pa.gcount = gcount;
  pa.offsets_out = a->offsets_out;
  pa.perm_out = a->perm_out;
  pa.x = fp4 ? nullptr : static_cast<const uint16_t*>(a->x);
  pa.H = (int)H;
  pa.rowshift = rowshift;
  pa.zero_buf = h_fp4 ? nullptr : hmax;
  pa.n_zero = Pt;
  if (launch_permute(pa, s) != hipSuccess) return NVFP4_ERR_LAUNCH;

  const double rows_per_group = (double)Pt / (double)G;
  const int maxc = pick_maxc(rows_per_group);

  // 2. gate/up GEMM with fused SwiGLU
  ev(1);
  GemmArgs g1{};
  g1.w = a->w1;
  g1.w_sf = a->w1_sf;
  g1.w_ws2 = a->w1_ws2;
  g1.w_gstride = 2 * I * (H / 2);
  g1.sf_gstride = 2 * I * (H / 16);
  g1.sw = a->s1;
  g1.sw_sf = a->s1_sf;
  g1.sw_ws2 = a->s1_ws2;
  g1.n_routed = (int)E;
  g1.N = (int)(2 * I);
  g1.K = (int)H;
  g1.I = (int)I;
  g1.offsets = offsets;
  g1.glist = glist;
  g1.gcount = gcount;
  g1.a = fp4 ? static_cast<const void*>(a->x_fp4) : a->x;
  g1.a_sf = a->x_sf;
  g1.a_by_token = 1;
  g1.perm = perm;
  g1.topk = (int)k;
  g1.P = P;
  g1.rowshift = rowshift;
  g1.gsa = fp4 ? a->a1_gs : nullptr;
  g1.h = h_fp4 ? nullptr : reinterpret_cast<float*>(ws + L.h);
  g1.hmax = hmax;
  g1.hq = h_fp4 ? ws + L.hq : nullptr;
  g1.hq_sf = h_fp4 ? ws + L.hq_sf : nullptr;
  g1.h_gs = a->a2_gs;
  GemmShape sh1{maxc, maxc >= 4 ? 4 : 2};
  const int epi1 = h_fp4 ? EPI_SWIGLU_FP4 : EPI_SWIGLU_F32;
  g1.nb = (int)((I + gemm_rows_per_block(epi1, sh1) - 1) / gemm_rows_per_block(epi1, sh1));
  if (launch_gemm(g1, fp4 ? A_FP4 : A_BF16, epi1, sh1, G, s) != hipSuccess) return NVFP4_ERR_LAUNCH;
  if (!h_fp4 && a->a2_gs_out)
    if (launch_amax_to_gs(hmax, Pt, a->a2_gs_out, s) != hipSuccess) return NVFP4_ERR_LAUNCH;

  // 3. down GEMM, scattering each pair's row (scaled by its weight_scale_2)
  ev(2);
  GemmArgs g2{};
  g2.w = a->w2;
  g2.w_sf = a->w2_sf;
  g2.w_ws2 = a->w2_ws2;
  g2.w_gstride = H * (I / 2);
  g2.sf_gstride = H * (I / 16);
  g2.sw = a->s2;
  g2.sw_sf = a->s2_sf;
  g2.sw_ws2 = a->s2_ws2;
  g2.n_routed = (int)E;
  g2.N = (int)H;
  g2.K = (int)I;
  g2.offsets = offsets;
  g2.glist = glist;
  g2.gcount = gcount;
  g2.a = h_fp4 ? static_cast<const void*>(ws + L.hq) : static_cast<const void*>(ws + L.h);
  g2.a_sf = h_fp4 ? ws + L.hq_sf : nullptr;
  g2.a_by_token = 0;
  g2.perm = perm;
  g2.topk = (int)k;
  g2.P = P;
  g2.rowmax = hmax;
  g2.gsa = h_fp4 ? a->a2_gs : nullptr;
  g2.slot = slot;
  GemmShape sh2{maxc, 4};
  g2.nb = (int)((H + gemm_rows_per_block(EPI_SLOT, sh2) - 1) / gemm_rows_per_block(EPI_SLOT, sh2));
  if (launch_gemm(g2, h_fp4 ? A_FP4 : A_F32, EPI_SLOT, sh2, G, s) != hipSuccess) return NVFP4_ERR_LAUNCH;

  // 4. weighted combine
  ev(3);
  CombineArgs ca{};
  ca.slot = slot;
  ca.ids = a->topk_ids;
  ca.w = a->topk_w;
  ca.T = (int)T;
  ca.topk = (int)k;
  ca.E = (int)E;
  ca.H = (int)H;
  ca.shared = S;
  ca.y = static_cast<uint16_t*>(a->y);
  if (launch_combine(ca, s) != hipSuccess) return NVFP4_ERR_LAUNCH;
  ev(4);
  return NVFP4_OK;
}

}  // extern "C"
