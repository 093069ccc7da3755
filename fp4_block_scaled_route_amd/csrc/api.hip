// C ABI of libnvfp4.so: argument validation, workspace layout and launches.
// Declarations and the contract of every entry point are in include/nvfp4.h.
#include <algorithm>
#include <cstdint>
#include <mutex>

#include "../../include/nvfp4.h"
#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxBuffer = (int64_t)1 << 32;
constexpr int kMaxExperts = 512;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int launch_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH; }

// Number of 16-row activation chunks a group pass holds, from the expected rows per group.
int pick_maxc(double rows_per_group) {
  const double want = rows_per_group * 1.25 / 16.0;
  if (want <= 2.0) return 2;
  if (want <= 4.0) return 4;
  return 8;
}

// K splits of a MoE GEMM's groups of more than 4 rows (four-wave LDS kernel)
// at decode-sized batches (at most 2 rows per group on average): there those
// groups are few and each work item is a chain of dependent K chunks, so a K
// range of at least 16 chunks is split 4 or 2 ways (at least 4 chunks per
// split; the gate/up GEMM at hidden 7168: 4 x 7).  Shorter ranges are not
// split (measured on MI355X at decode: the down GEMM's 8 chunks split 2 ways
// gained nothing, 4 ways lost 17 us).
int moe_splits(int64_t T, int64_t topk, int64_t E, int64_t S, int64_t K) {
  if ((double)(T * topk + S * T) / (double)(E + S) > 2.0) return 1;
  const int64_t nkc = K / 256;
  if (nkc < 16) return 1;
  for (int s : {4, 2})
    if (nkc % s == 0 && nkc / s >= 4) return s;
  return 1;
}

// Groups of more than 4 rows: at most this many (the big-group launch's list part).
int64_t moe_big_groups(int64_t T, int64_t topk, int64_t E, int64_t S) {
  return std::min<int64_t>(E + S, (T * topk + S * T) / (kBigGroupRows + 1));
}

// Rows per pass of the four-wave LDS kernel at decode/prefill (GemmShape{4, 2, 4}).
constexpr int kMoeSmallPassRows = 64;

// Workspace layout of nvfp4_moe_grouped.
struct MoeLayout {
  size_t offsets, glist, gcount, perm, inv, bcnt, rowshift, x16, hmax, hshift, h, h16, hq, hq_sf, slot, mpart, mcnt,
      total;
  int s1, s2;        // K splits of the gate/up and down GEMMs
  int mpass, nbmax;  // split counters: G * nbmax * mpass
};

MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int has_shared, int h_fp4) {
  const int64_t S = has_shared ? 1 : 0;
  const int64_t Pt = T * topk + S * T;
  MoeLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = round_up(off + bytes, 256); return o; };
  L.offsets = take(sizeof(int32_t) * (E + 2));
  L.glist = take(sizeof(int32_t) * (E + 1));
  L.gcount = take(sizeof(int32_t) * 2);
  L.perm = take(sizeof(int32_t) * Pt);
  L.inv = take(sizeof(int32_t) * Pt);
  L.bcnt = take(sizeof(int32_t) * (size_t)permute_blocks(T * topk) * E);
  L.rowshift = take(sizeof(int32_t) * T);
  L.x16 = take(sizeof(uint16_t) * (size_t)T * H);
  L.hmax = take(sizeof(uint32_t) * Pt);
  if (h_fp4) {
    L.h = L.h16 = L.hshift = 0;
    L.hq = take((size_t)Pt * (I / 2));
    L.hq_sf = take((size_t)Pt * (I / 16));
  } else {
    L.hshift = take(sizeof(int32_t) * Pt);
    L.h = take(sizeof(float) * (size_t)Pt * I);
    L.h16 = take(sizeof(uint16_t) * (size_t)Pt * I);
    L.hq = L.hq_sf = 0;
  }
  L.slot = take(sizeof(uint16_t) * (size_t)Pt * H);
  L.s1 = moe_splits(T, topk, E, S, H);
  L.s2 = moe_splits(T, topk, E, S, I);
  // the partial sums are addressed with 32-bit offsets
  if ((int64_t)sizeof(float) * Pt * std::max<int64_t>(L.s1 * 2 * I, L.s2 * H) >= kMaxBuffer) L.s1 = L.s2 = 1;
  // a group holds at most max(T * topk, T) rows (ids need not be distinct)
  L.mpass = (int)((std::max(T * topk, T) + kMoeSmallPassRows - 1) / kMoeSmallPassRows);
  L.nbmax = (int)std::max(L.s1 > 1 ? I / gemm_rows_per_block(EPI_SWIGLU_F32, GemmShape{4, 2, 4}) : 0,
                          L.s2 > 1 ? H / gemm_rows_per_block(EPI_SLOT, GemmShape{4, 2, 4}) : 0);
  L.mpart = L.mcnt = 0;
  if (L.s1 > 1 || L.s2 > 1) {
    L.mpart = take(sizeof(float) * (size_t)Pt * std::max<int64_t>(L.s1 * 2 * I, L.s2 * H));
    L.mcnt = take(sizeof(uint32_t) * (size_t)moe_big_groups(T, topk, E, S) * L.nbmax * L.mpass);
  }
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
    case NVFP4_ERR_SCRATCH:
      return "the call needs more scratch memory than nvfp4_moe_grouped_noalloc holds "
             "(NVFP4_MOE_NOALLOC_SCRATCH_BYTES); use nvfp4_moe_grouped with a workspace";
    default: return "unknown status";
  }
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

size_t nvfp4_quantize_act_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || M >= kMaxDim || K >= kMaxDim) return 0;
  return quantize_workspace_bytes();
}

int nvfp4_quantize_act(const void* x_bf16, int64_t M, int64_t K, float* gs, int compute_gs, uint8_t* x_fp4,
                       uint8_t* x_sf, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || K <= 0 || K % 16 != 0 || M >= kMaxDim || K >= kMaxDim || M * K >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (!gs) return NVFP4_ERR_NULL;
  if (!aligned(gs, 4)) return NVFP4_ERR_ALIGN;
  if (M > 0) {
    if (!x_bf16 || !x_fp4 || !x_sf) return NVFP4_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(x_fp4, 8)) return NVFP4_ERR_ALIGN;
    if (compute_gs) {
      if (!workspace || workspace_bytes < nvfp4_quantize_act_workspace_size(M, K)) return NVFP4_ERR_WORKSPACE;
      if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
    }
  }
  return launch_status(launch_quantize_act(static_cast<const uint16_t*>(x_bf16), M, K, gs, compute_gs, x_fp4,
                                           x_sf, static_cast<unsigned*>(workspace), static_cast<hipStream_t>(stream)));
}

int nvfp4_router_prepare(const void* w_bf16, int64_t E, int64_t H, float* scale, void* w_rt_bf16, void* stream) {
  if (E <= 0 || H <= 0 || H % 256 != 0 || E >= kMaxDim || H >= kMaxDim || E * H >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (!w_bf16 || !scale || !w_rt_bf16) return NVFP4_ERR_NULL;
  if (!aligned(w_bf16, 16) || !aligned(w_rt_bf16, 16) || !aligned(scale, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* w = static_cast<const uint16_t*>(w_bf16);
  if (launch_bf16_amax(w, E * H, scale, s) != hipSuccess) return NVFP4_ERR_LAUNCH;
  return launch_status(launch_router_prepare(w, E * H, scale, static_cast<uint16_t*>(w_rt_bf16), s));
}

size_t nvfp4_router_workspace_size(int64_t T, int64_t H, int64_t E) {
  if (T <= 0 || H <= 0 || E <= 0 || H % 256 != 0 || T >= kMaxDim || E > 512) return 0;
  return sizeof(float) * (size_t)router_ksplit((int)T, (int)H, (int)E) * T * E;
}

int nvfp4_router_topk(const void* x_bf16, const void* w_rt_bf16, int64_t T, int64_t H, int64_t E, int64_t topk,
                      float* logits, int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (T < 0 || H <= 0 || H % 256 != 0 || E <= 0 || E > 512 || topk <= 0 || topk > E || topk > 64)
    return NVFP4_ERR_SHAPE;
  if (T >= kMaxDim || H >= kMaxDim || T * H * 2 >= kMaxBuffer || E * H * 2 >= kMaxBuffer || T * E >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  if (!x_bf16 || !w_rt_bf16 || !logits || !topk_ids || !topk_w) return NVFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_rt_bf16, 16) || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return NVFP4_ERR_ALIGN;
  if (!workspace || workspace_bytes < nvfp4_router_workspace_size(T, H, E)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  return launch_status(launch_router_topk(static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(w_rt_bf16),
                                          (int)T, (int)H, (int)E, (int)topk, logits, topk_ids, topk_w,
                                          static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Launch plan of the dense and grouped linear (G groups of T rows each; the
// dense linear is G = 1).  Each group's T rows: up to 4 rows on the
// barrier-free kernels; on the 8-wave kernel in 112-row passes when that
// gives at least one work item (group, pass, 512-row block) per CU (K a
// multiple of 1024); otherwise on the 4-wave kernel.  Work items on the
// 4-wave and compact kernels are latency chains over K: when they are too
// few to fill the GPU, K is split into S parts (S divides the 256-element
// chunk count, at least 2 chunks per part, S <= 16) and the fp32 partial sums
// are added in split order.  (NVFP4 activations on the barrier-free path are
// not split.)
struct GlPlan {
  GemmShape sh{1, 2};
  int pr = 0, npass = 1, ksplit = 1, nb = 1;
};

GlPlan gl_plan(int64_t T, int64_t G, int64_t N, int64_t K, bool fp4) {
  GlPlan p;
  p.pr = (int)T;
  if (T > kBigGroupRows) {
    const int64_t items8 = G * ((T + 111) / 112) * ((N + 511) / 512);
    if (items8 >= 256 && K % 1024 == 0) {
      p.sh = GemmShape{7, 4, 8};
    } else {
      p.sh = GemmShape{pick_maxc((double)T), 2};
    }
    p.pr = 16 * p.sh.maxc;
  }
  p.npass = (int)((T + p.pr - 1) / p.pr);
  const int brows = gemm_rows_per_block(EPI_Y_BF16, p.sh);
  p.nb = (int)((N + brows - 1) / brows);
  if (p.sh.nw == 4 && !(p.sh.maxc == 1 && fp4)) {
    const int64_t items = G * p.npass * p.nb;
    const int64_t nkc = K / 256;
    for (int s = 16; s >= 2; --s)
      if (nkc % s == 0 && nkc / s >= 2 && items * s <= 256) {
        p.ksplit = s;
        break;
      }
  }
  return p;
}

// Workspace: per-row shifts and the fp16 copy of bf16 activations, then the
// fp32 partial sums of a K split.
size_t staging_bytes(int64_t rows, int64_t K) {
  return round_up(sizeof(int32_t) * (size_t)rows, 256) + round_up(sizeof(uint16_t) * (size_t)rows * K, 256);
}

// Bytes one call needs (0 on the skinny kernel, which stages in LDS).
size_t gl_need(int64_t T, int64_t G, int64_t N, int64_t K, bool fp4) {
  if (skinny_plan(T, G, N, K, fp4).ok) return 0;
  const GlPlan p = gl_plan(T, G, N, K, fp4);
  size_t need = fp4 ? 0 : staging_bytes(T * G, K);
  if (p.ksplit > 1) need = staging_bytes(T * G, K) + round_up(sizeof(float) * (size_t)p.ksplit * T * G * N, 256);
  return need;
}

size_t gl_workspace(int64_t T, int64_t G, int64_t N, int64_t K) {
  if (T <= 0 || G <= 0 || N <= 0 || K <= 0 || K % 256 != 0 || T * G >= kMaxDim) return 0;
  return std::max(gl_need(T, G, N, K, false), gl_need(T, G, N, K, true));
}

// The dense linear (G = 1) and the grouped linear: validation, then the launches.
int gl_run(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa, const uint8_t* w_fp4,
           const uint8_t* w_sf, const float* ws2, int64_t T, int64_t G, int64_t N, int64_t K, void* y_bf16,
           void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || G <= 0 || N <= 0 || K <= 0 || T >= kMaxDim || G >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return NVFP4_ERR_SHAPE;
  if (K % 256 != 0 || N % 16 != 0 || T * G >= kMaxDim || G * N >= kMaxDim) return NVFP4_ERR_SHAPE;
  // every tensor a kernel reads through a buffer resource must span < 4 GiB
  if (N * (K / 2) >= kMaxBuffer || T * G * K * 2 >= kMaxBuffer) return NVFP4_ERR_SHAPE;
  if (T == 0) return NVFP4_OK;
  const bool fp4 = x_fp4 != nullptr;
  if (fp4 && (x_bf16 || !x_sf || !gsa)) return x_bf16 ? NVFP4_ERR_ARG : NVFP4_ERR_NULL;
  if (!fp4 && !x_bf16) return NVFP4_ERR_NULL;
  if (!fp4 && (x_sf || gsa)) return NVFP4_ERR_ARG;
  if (!w_fp4 || !w_sf || !ws2 || !y_bf16) return NVFP4_ERR_NULL;
  if (!aligned(w_fp4, 16) || !aligned(w_sf, 16) || !aligned(ws2, 4) || !aligned(y_bf16, 16)) return NVFP4_ERR_ALIGN;
  if (fp4 && (!aligned(x_fp4, 16) || !aligned(x_sf, 16) || !aligned(gsa, 4))) return NVFP4_ERR_ALIGN;
  if (!fp4 && !aligned(x_bf16, 16)) return NVFP4_ERR_ALIGN;
  const int64_t rows = T * G;   // activation rows of K: row t * G + g
  hipStream_t s = static_cast<hipStream_t>(stream);
  const SkinnyPlan sk = skinny_plan(T, G, N, K, fp4);
  if (sk.ok) {
    // one launch, no workspace
    GemmArgs g{};
    g.w = w_fp4;
    g.w_sf = w_sf;
    g.w_ws2 = ws2;
    g.w_gstride = N * (K / 2);
    g.sf_gstride = N * (K / 16);
    g.n_routed = (int)G;
    g.N = (int)N;
    g.K = (int)K;
    g.a = fp4 ? static_cast<const void*>(x_fp4) : x_bf16;
    g.a_rows = (int)rows;
    g.a_sf = x_sf;
    g.gsa = fp4 ? gsa : nullptr;
    g.y = static_cast<uint16_t*>(y_bf16);
    g.gl_T = (int)T;
    g.gl_G = (int)G;
    g.nb = sk.nb;
    g.sk_kp = sk.kp;
    g.sk_u = sk.u;
    return launch_status(launch_gemm_skinny(g, fp4 ? A_FP4 : A_F16, sk, s));
  }
  const GlPlan plan = gl_plan(T, G, N, K, fp4);
  if (!fp4 || plan.ksplit > 1) {
    if (!workspace || workspace_bytes < gl_workspace(T, G, N, K)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  }
  uint8_t* wsp = static_cast<uint8_t*>(workspace);
  int* rowshift = reinterpret_cast<int*>(wsp);
  f16* x16 = fp4 ? nullptr : reinterpret_cast<f16*>(wsp + round_up(sizeof(int32_t) * (size_t)rows, 256));
  float* part = plan.ksplit > 1 ? reinterpret_cast<float*>(wsp + staging_bytes(rows, K)) : nullptr;
  if (!fp4) {
    hipError_t e = launch_rows_to_f16(static_cast<const uint16_t*>(x_bf16), (int)rows, (int)K, rowshift, x16, s);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
  }
  GemmArgs g{};
  g.w = w_fp4;
  g.w_sf = w_sf;
  g.w_ws2 = ws2;
  g.w_gstride = N * (K / 2);
  g.sf_gstride = N * (K / 16);
  g.n_routed = (int)G;
  g.N = (int)N;
  g.K = (int)K;
  g.list_part = 2;
  g.a = fp4 ? static_cast<const void*>(x_fp4) : static_cast<const void*>(x16);
  g.a_rows = (int)rows;
  g.a_sf = x_sf;
  g.rowshift = fp4 ? nullptr : rowshift;
  g.gsa = fp4 ? gsa : nullptr;
  g.y = static_cast<uint16_t*>(y_bf16);
  g.gl_T = (int)T;
  g.gl_G = (int)G;
  g.gl_pr = plan.pr;
  g.gl_npass = plan.npass;
  g.nb = plan.nb;
  const int items = (int)G * plan.npass * plan.ksplit;
  if (plan.ksplit == 1) return launch_status(launch_gemm(g, fp4 ? A_FP4 : A_F16, EPI_Y_BF16, plan.sh, items, s));
  g.ksplit = plan.ksplit;
  g.part = part;
  if (launch_gemm(g, fp4 ? A_FP4 : A_F16, EPI_PART_F32, plan.sh, items, s) != hipSuccess) return NVFP4_ERR_LAUNCH;
  return launch_status(launch_split_reduce(part, plan.ksplit, rows * N, static_cast<uint16_t*>(y_bf16), s));
}

}  // namespace

extern "C" {

size_t nvfp4_linear_workspace_size(int64_t M, int64_t N, int64_t K) { return gl_workspace(M, 1, N, K); }

int nvfp4_linear(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa,
                 const uint8_t* w_fp4, const uint8_t* w_sf, const float* gsb, int64_t M, int64_t N, int64_t K,
                 void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return NVFP4_ERR_SHAPE;
  return gl_run(x_bf16, x_fp4, x_sf, gsa, w_fp4, w_sf, gsb, M, 1, N, K, y_bf16, workspace, workspace_bytes, stream);
}

size_t nvfp4_grouped_linear_workspace_size(int64_t T, int64_t G, int64_t N, int64_t K) {
  return gl_workspace(T, G, N, K);
}

int nvfp4_grouped_linear(const void* x_bf16, const uint8_t* x_fp4, const uint8_t* x_sf, const float* gsa,
                         const uint8_t* w_fp4, const uint8_t* w_sf, const float* ws2, int64_t T, int64_t G, int64_t N,
                         int64_t K, void* y_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  return gl_run(x_bf16, x_fp4, x_sf, gsa, w_fp4, w_sf, ws2, T, G, N, K, y_bf16, workspace, workspace_bytes, stream);
}

size_t nvfp4_rmsnorm_quantize_workspace_size(int64_t T) {
  if (T <= 0 || T >= kMaxDim) return 0;
  return rmsnorm_workspace_bytes((int)T);
}

int nvfp4_rmsnorm_quantize(const void* x_bf16, const void* w_bf16, float eps, int64_t T, int64_t K, void* y_bf16,
                           float* gs, int compute_gs, uint8_t* x_fp4, uint8_t* x_sf, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (T < 0 || K <= 0 || K % 16 != 0 || T >= kMaxDim || K >= kMaxDim || T * K >= kMaxDim) return NVFP4_ERR_SHAPE;
  if (!(eps > 0.0f) || eps == __builtin_inff()) return NVFP4_ERR_ARG;
  if (T == 0) {
    // nothing to normalise; a computed gs is that of no elements (0), as in nvfp4_quantize_act
    if (!compute_gs) return NVFP4_OK;
    if (!gs) return NVFP4_ERR_NULL;
    if (!aligned(gs, 4)) return NVFP4_ERR_ALIGN;
    return launch_status(launch_rmsnorm_quantize(nullptr, nullptr, eps, 0, K, nullptr, gs, 1, nullptr, nullptr,
                                                 nullptr, static_cast<hipStream_t>(stream)));
  }
  if (!x_bf16 || !w_bf16 || !gs || !x_fp4 || !x_sf) return NVFP4_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16) || !aligned(x_fp4, 16) || !aligned(x_sf, 16) || !aligned(gs, 4) ||
      (y_bf16 && !aligned(y_bf16, 16)))
    return NVFP4_ERR_ALIGN;
  if (!workspace || workspace_bytes < nvfp4_rmsnorm_quantize_workspace_size(T)) return NVFP4_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NVFP4_ERR_ALIGN;
  return launch_status(launch_rmsnorm_quantize(static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(w_bf16),
                                               eps, (int)T, (int)K, static_cast<uint16_t*>(y_bf16), gs, compute_gs,
                                               x_fp4, x_sf, workspace, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_moe_workspace_size(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int has_shared,
                                int h_fp4) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  return moe_layout(T, H, I, E, topk, has_shared, h_fp4).total;
}

}  // extern "C"

namespace {

// Scratch memory of nvfp4_moe_grouped_noalloc: one array per GPU the
// library runs on, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept in scratch_ptr.
__device__ __align__(256) uint8_t scratch[NVFP4_MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

// nvfp4_moe_grouped with the workspace taken from the caller's arguments
// (noalloc == false) or from the scratch array (noalloc == true).
int moe_grouped_impl(const nvfp4_moe_args* a, void* stream, bool noalloc) {
  if (!a) return NVFP4_ERR_NULL;
  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, k = a->topk;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0) return NVFP4_ERR_SHAPE;
  if (H % 256 != 0 || I % 256 != 0 || E > kMaxExperts || k > E) return NVFP4_ERR_SHAPE;
  if (T >= kMaxDim || H >= kMaxDim || I >= kMaxDim || T * k + T >= kMaxDim) return NVFP4_ERR_SHAPE;
  // every tensor a kernel reads through a buffer resource must span < 4 GiB
  if (2 * I * (H / 2) >= kMaxBuffer || T * H * 2 >= kMaxBuffer || (T * k + T) * I * 2 >= kMaxBuffer)
    return NVFP4_ERR_SHAPE;
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
  uint8_t* ws;
  if (noalloc) {
    if (a->workspace || a->workspace_bytes) return NVFP4_ERR_ARG;
    if (L.total > NVFP4_MOE_NOALLOC_SCRATCH_BYTES) return NVFP4_ERR_SCRATCH;
    ws = static_cast<uint8_t*>(scratch_for_current_device());
    if (!ws) return NVFP4_ERR_LAUNCH;
  } else {
    if (!a->workspace || a->workspace_bytes < L.total) return NVFP4_ERR_WORKSPACE;
    if (!aligned(a->workspace, 256)) return NVFP4_ERR_ALIGN;
    ws = static_cast<uint8_t*>(a->workspace);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  int* offsets = reinterpret_cast<int*>(ws + L.offsets);
  int* glist = reinterpret_cast<int*>(ws + L.glist);
  int* gcount = reinterpret_cast<int*>(ws + L.gcount);
  int* perm = reinterpret_cast<int*>(ws + L.perm);
  int* inv = reinterpret_cast<int*>(ws + L.inv);
  int* rowshift = reinterpret_cast<int*>(ws + L.rowshift);
  f16* x16 = reinterpret_cast<f16*>(ws + L.x16);
  unsigned* hmax = reinterpret_cast<unsigned*>(ws + L.hmax);
  uint16_t* slot = reinterpret_cast<uint16_t*>(ws + L.slot);
  const int S = has_shared ? 1 : 0;
  const int P = (int)(T * k);
  const int Pt = P + S * (int)T;
  const int G = (int)E + S;
  auto ev = [&](int i) {
    if (a->stage_events && a->stage_events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(a->stage_events[i]), s);
  };
  // Groups with more than kBigGroupRows rows run on the LDS-staged kernel; at
  // most Pt / (kBigGroupRows + 1) groups can be that big.
  const int n_big_max = (int)moe_big_groups(T, k, E, S);
  const double rows_per_group = (double)Pt / (double)G;
  // big groups: 64-row passes on 4-wave workgroups (a few hot groups), or
  // 112-row passes on 8-wave workgroups sharing one LDS tile (large batches)
  const bool large_batch = rows_per_group > 16;
  // ev_big / ev_small: stage events recorded before each of the two launches
  auto two_launches = [&](GemmArgs g, int amode, int epi, int r, int ev_big, int ev_small, int msplit) -> bool {
    // (the 8-wave configuration walks K in quads of 256-element chunks)
    GemmShape big = !large_batch ? GemmShape{4, r, 4} : g.K % 1024 == 0 ? GemmShape{7, 4, 8} : GemmShape{8, r, 4};
    GemmShape small{1, r, 4};
    const int half = epi == EPI_SWIGLU_F32 || epi == EPI_SWIGLU_FP4 ? 2 : 1;
    ev(ev_big);
    if (large_batch) {
      // groups of at most 4 rows are rare here: all groups go to the LDS
      // kernel (it takes any row count), so no launch runs empty
      g.list_part = 2;
      g.nb = (int)((g.N / half + gemm_rows_per_block(epi, big) - 1) / gemm_rows_per_block(epi, big));
      if (launch_gemm(g, amode, epi, big, G, s) != hipSuccess) return false;
      ev(ev_small);
      return true;
    }
    g.list_part = 0;
    g.nb = (int)((g.N / half + gemm_rows_per_block(epi, big) - 1) / gemm_rows_per_block(epi, big));
    g.mks = 1;
    if (msplit > 1) {
      g.mks = msplit;
      g.mpart = reinterpret_cast<float*>(ws + L.mpart);
      g.mrows = Pt;
      g.mcols = g.N;
      g.mpass = L.mpass;
      g.mcnt = reinterpret_cast<unsigned*>(ws + L.mcnt);
    }
    if (launch_gemm(g, amode, epi, big, n_big_max * g.mks, s) != hipSuccess) return false;
    g.mks = 1;
    ev(ev_small);
    g.list_part = 1;
    g.nb = (int)((g.N / half + gemm_rows_per_block(epi, small) - 1) / gemm_rows_per_block(epi, small));
    // more than 2 rows per group on average: a group's workgroups on one XCD
    // (measured on MI355X: prefill 1.3-1.6% faster; decode 0.5% slower)
    g.xcd_order = rows_per_group > 2.0;
    return launch_gemm(g, amode, epi, small, G, s) == hipSuccess;
  };

  // 1. permutation, group order, fp16 copy of x with row shifts, clearing of the h row maxima
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
  pa.x16 = x16;
  pa.zero_buf = h_fp4 ? nullptr : hmax;
  pa.n_zero = Pt;
  if (L.mcnt) {
    pa.zero_buf2 = reinterpret_cast<unsigned*>(ws + L.mcnt);
    pa.n_zero2 = (int)(moe_big_groups(T, k, E, S) * L.nbmax * L.mpass);
  }
  if (launch_permute(pa, reinterpret_cast<int*>(ws + L.bcnt), s) != hipSuccess) return NVFP4_ERR_LAUNCH;

  // 2. gate/up GEMM with fused SwiGLU
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
  g1.a = fp4 ? static_cast<const void*>(a->x_fp4) : static_cast<const void*>(x16);
  g1.a_rows = (int)T;
  g1.a_sf = a->x_sf;
  g1.a_by_token = 1;
  g1.perm = perm;
  g1.topk = (int)k;
  g1.P = P;
  g1.rowshift = fp4 ? nullptr : rowshift;
  g1.gsa = fp4 ? a->a1_gs : nullptr;
  g1.h = h_fp4 ? nullptr : reinterpret_cast<float*>(ws + L.h);
  g1.hmax = hmax;
  g1.hq = h_fp4 ? ws + L.hq : nullptr;
  g1.hq_sf = h_fp4 ? ws + L.hq_sf : nullptr;
  g1.h_gs = a->a2_gs;
  const int epi1 = h_fp4 ? EPI_SWIGLU_FP4 : EPI_SWIGLU_F32;
  if (!two_launches(g1, fp4 ? A_FP4 : A_F16, epi1, 2, 1, 2, L.s1)) return NVFP4_ERR_LAUNCH;

  // 3. calibration and fp16 copy of h (unless it is NVFP4), down GEMM scattering each pair's row
  ev(3);
  if (!h_fp4 && a->a2_gs_out)
    if (launch_amax_to_gs(hmax, Pt, a->a2_gs_out, s) != hipSuccess) return NVFP4_ERR_LAUNCH;
  int* hshift = h_fp4 ? nullptr : reinterpret_cast<int*>(ws + L.hshift);
  f16* h16 = h_fp4 ? nullptr : reinterpret_cast<f16*>(ws + L.h16);
  if (!h_fp4)
    if (launch_h_to_f16(reinterpret_cast<const float*>(ws + L.h), hmax, offsets, (int)E + 1, Pt, (int)I, h16, hshift,
                        s) != hipSuccess)
      return NVFP4_ERR_LAUNCH;
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
  g2.a = h_fp4 ? static_cast<const void*>(ws + L.hq) : static_cast<const void*>(h16);
  g2.a_rows = Pt;
  g2.a_sf = h_fp4 ? ws + L.hq_sf : nullptr;
  g2.a_by_token = 0;
  g2.perm = perm;
  g2.topk = (int)k;
  g2.P = P;
  g2.rowshift = hshift;
  g2.gsa = h_fp4 ? a->a2_gs : nullptr;
  g2.slot = slot;
  if (!two_launches(g2, h_fp4 ? A_FP4 : A_F16, EPI_SLOT, 2, 4, 5, L.s2)) return NVFP4_ERR_LAUNCH;

  // 4. weighted combine
  ev(6);
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
  ev(7);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_moe_grouped(const nvfp4_moe_args* a, void* stream) { return moe_grouped_impl(a, stream, false); }

int nvfp4_moe_grouped_noalloc(const nvfp4_moe_args* a, void* stream) { return moe_grouped_impl(a, stream, true); }

}  // extern "C"
