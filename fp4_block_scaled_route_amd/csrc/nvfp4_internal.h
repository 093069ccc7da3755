// Internal declarations of the gfx950 NVFP4 kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// One K chunk = 256 elements: 128 code bytes + 16 scale bytes per weight row.
constexpr int kChunk = 256;
// LDS row pitch of the staged activation chunk, in bytes (256 fp16 + 16 pad).
constexpr int kLdsRow = kChunk * 2 + 16;

// Activation operand sources of the grouped GEMM.
enum AMode {
  A_F16 = 0,   // fp16 rows holding bf16/fp32 values times 2^rowshift[row] (exact)
  A_FP4 = 2    // NVFP4 rows, decoded exactly to fp16 (global scale in the epilogue)
};

// Groups with more rows than this go to the LDS-staged GEMM kernel; smaller
// ones to the barrier-free kernels (fp16 activations: at most 4 rows per pass).
constexpr int kBigGroupRows = 4;

// Epilogues of the grouped GEMM.
enum EpiMode {
  EPI_Y_BF16 = 0,      // y[row, n] = bf16(alpha * acc)                    (dense linear)
  EPI_SWIGLU_F32 = 1,  // h[row, i] = silu(alpha*gate) * (alpha*up), fp32, + row max |h|
  EPI_SWIGLU_FP4 = 2,  // same h, quantized to NVFP4 with a supplied global scale
  EPI_SLOT = 3,        // slot[pair, n] = bf16(alpha * acc)                (down GEMM)
  EPI_PART_F32 = 4     // part[ks, row, n] = alpha * acc, fp32 (one K split of the grouped linear)
};

struct GemmArgs {
  // Weights: group g < n_routed at w + g*w_gstride, shared expert (g == n_routed) at sw.
  const uint8_t* w;
  const uint8_t* w_sf;
  const float* w_ws2;
  int64_t w_gstride;   // bytes between groups of codes
  int64_t sf_gstride;  // bytes between groups of scales
  const uint8_t* sw;
  const uint8_t* sw_sf;
  const float* sw_ws2;
  int n_routed;        // number of routed groups (1 for the dense linear)
  int N;               // weight rows of one group (2I for gate/up, H for down, N for linear)
  int K;               // reduction length (multiple of 256)
  int I;               // gate/up split: gate rows [0, I), up rows [I, 2I) (SwiGLU epilogues)
  // Groups: rows of group g are [off[g], off[g+1]) of the sorted row space;
  // glist gives the processing order (largest first); gcount[0] = non-empty
  // groups, gcount[1] = groups with more than kBigGroupRows rows.  list_part:
  // 0 = the big groups, 1 = the others, 2 = all.
  // Dense: offsets == nullptr, one group of rows [0, M).
  const int* offsets;
  const int* glist;
  const int* gcount;
  int list_part;
  int M;               // dense row count
  // Grouped linear (gl_G > 0, offsets == nullptr): gl_G groups of gl_T rows;
  // sorted row r = g * gl_T + t is activation and output row t * gl_G + g
  // (the [T, G, K] -> [T, G, N] layout); work item = (group, pass of gl_pr rows),
  // gl_npass passes per group.
  int gl_T, gl_G, gl_npass, gl_pr;
  // K split of the grouped linear (four-wave LDS kernel only): ksplit parts
  // of K / ksplit each, item = ((group, pass), split); partial sums to part
  // (EPI_PART_F32), added in split order by launch_split_reduce.
  int ksplit;
  float* part;
  // K split of the MoE groups on the four-wave LDS kernel (mks > 1; decode-
  // sized batches): item = ((group list index, split), weight-row block); each
  // split writes its fp32 sums to mpart [mks, rows, mcols] (rows = sorted
  // rows) and counts itself in mcnt[(list position * nb + block) * mpass + pass]
  // (zeroed before the launch); the last one adds the mks partial sums in
  // split order and runs the epilogue, then clears the counter.
  // MoE groups on the barrier-free kernels in XCD order (see the kernels)
  int xcd_order;
  int mks;
  float* mpart;
  int mrows, mcols, mpass;
  unsigned* mcnt;
  int nb;              // weight-row blocks per group (grid = groups * nb)
  // Skinny kernel (grouped linear with gl_T <= 4): workgroup = (group, R
  // fragments); its sk_kp waves take ranges of sk_u chunks of K.
  int sk_kp, sk_u;
  // Activation operand.
  const void* a;       // see AMode; row pitch in elements = K
  int a_rows;          // rows of the activation tensor (bounds of its buffer resource)
  const uint8_t* a_sf; // NVFP4 block scales [rows, K/16]
  int a_by_token;      // 1: A row = token of the sorted row (via perm); 0: A row = sorted row
  const int* perm;     // sorted row -> pair id (pair < P: token = pair / topk; else pair - P)
  int topk;
  int P;               // T * topk
  const int* rowshift; // A_F16: per A row, the power-of-two shift of its fp16 copy (nullptr = 0)
  const float* gsa;    // activation global scale (nullptr = 1)
  // Outputs.
  float* h;            // [rows, I] fp32 (EPI_SWIGLU_F32)
  unsigned* hmax;      // [rows] bits of max|h| (EPI_SWIGLU_F32)
  uint8_t* hq;         // [rows, I/2] (EPI_SWIGLU_FP4)
  uint8_t* hq_sf;      // [rows, I/16]
  const float* h_gs;   // global scale used to quantize h (EPI_SWIGLU_FP4)
  uint16_t* slot;      // [pairs, N] bf16 (EPI_SLOT), row = perm[sorted row]
  uint16_t* y;         // [M, N] bf16 (EPI_Y_BF16)
};

// Tile shape choice of one GEMM launch.
struct GemmShape {
  int maxc;   // token chunks of 16 per pass (1 = barrier-free kernels; 2, 4, 7, 8 = LDS kernel)
  int r;      // 16-row weight fragments per wave
  int nw = 4; // waves per workgroup
};

hipError_t launch_gemm(const GemmArgs& a, int amode, int epi, GemmShape shape, int n_groups,
                       hipStream_t stream);
// Rows per workgroup for a shape/epilogue (used by the host to size the grid).
int gemm_rows_per_block(int epi, GemmShape shape);

struct PermuteArgs {
  const int32_t* ids;  // [T, topk]
  int T, topk, E, shared;
  int* offsets;        // [E + 2]
  int* perm;           // [P + T]
  int* inv;            // [P + T]
  int* glist;          // [E + 1]
  int* gcount;         // [2]: non-empty groups, groups with > kBigGroupRows rows
  int32_t* offsets_out;  // optional copies
  int32_t* perm_out;
  // fp16 copy of the bf16 activations with per-row shifts (optional) and
  // zeroing of a row-max buffer
  const uint16_t* x;   // [T, H] bf16 or nullptr
  int H;
  int* rowshift;       // [T]
  f16* x16;            // [T, H]
  unsigned* zero_buf;  // [n_zero] set to 0, or nullptr
  int n_zero;
  unsigned* zero_buf2; // [n_zero2] set to 0, or nullptr
  int n_zero2;
};
// Workgroups of the multi-workgroup permutation for P pairs (0: one
// workgroup does it all); it needs bcnt[blocks * E] ints of workspace.
int permute_blocks(int64_t P);
hipError_t launch_permute(const PermuteArgs& a, int* bcnt, hipStream_t stream);

// fp16 copy of bf16 rows scaled by per-row powers of two (rowshift[r]).
hipError_t launch_rows_to_f16(const uint16_t* x, int rows, int cols, int* rowshift, f16* x16,
                              hipStream_t stream);
// fp16 copy of the fp32 hidden rows [0, offsets[n_groups]) with per-row shifts
// from their max |h| bits.
hipError_t launch_h_to_f16(const float* h, const unsigned* hmax, const int* offsets, int end_index,
                           int rows_max, int cols, f16* h16, int* hshift, hipStream_t stream);
hipError_t launch_amax_to_gs(const unsigned* rowmax, int rows, float* gs_out, hipStream_t stream);

struct CombineArgs {
  const uint16_t* slot; // [P + T, H] bf16
  const int32_t* ids;   // [T, topk]
  const float* w;       // [T, topk]
  int T, topk, E, H, shared;
  uint16_t* y;          // [T, H] bf16
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// y[i] = bf16(sum over s = 0..S-1, in that order, of part[s * n + i]), n % 4 == 0.
hipError_t launch_split_reduce(const float* part, int S, int64_t n, uint16_t* y, hipStream_t stream);

// Launch plan of the skinny kernel (one launch per call, no workspace) for a
// grouped linear of G groups of T <= 4 rows, or ok = false.
struct SkinnyPlan {
  bool ok = false;
  int r = 1;           // fragments per wave (1 or 2)
  int u = 0, kp = 0;   // chunks per range, ranges of K (= waves per workgroup)
  int nb = 1;          // workgroups per group
  int lds = 0;         // dynamic LDS bytes
  bool kp_ok() const { return kp > 0; }
};
SkinnyPlan skinny_plan(int64_t T, int64_t G, int64_t N, int64_t K, bool fp4);
hipError_t launch_gemm_skinny(const GemmArgs& a, int amode, const SkinnyPlan& p, hipStream_t stream);

// Fused RMSNorm + NVFP4 quantization of x [T, K] with weight w [K]: y [T, K]
// bf16 if y != nullptr, codes q [T, K/2], scale bytes sf [T, K/16]; gs
// computed (compute_gs) or read from *gs.  The workspace (rmsnorm_workspace_bytes(T))
// holds r per row and the per-workgroup maxima of |y|.
size_t rmsnorm_workspace_bytes(int T);
hipError_t launch_rmsnorm_quantize(const uint16_t* x, const uint16_t* w, float eps, int T, int K, uint16_t* y,
                                   float* gs, int compute_gs, uint8_t* q, uint8_t* sf, void* workspace,
                                   hipStream_t stream);

// word = max |x| over n bf16 values (n % 8 == 0), as a float (zeroed first).
hipError_t launch_bf16_amax(const uint16_t* x, int64_t n, float* word, hipStream_t stream);

// Router gate (page P1, note on the router gate).  Prepare: scale = amax(w)/448,
// w_rt = bf16(E4M3(RNE(w / scale)) * scale) over n elements; `scale` holds
// amax on entry (from launch_bf16_amax) and amax/448 on exit.
hipError_t launch_router_prepare(const uint16_t* w, int64_t n, float* scale, uint16_t* w_rt, hipStream_t stream);
// logits[t, e] = sum_k x[t, k] * w_rt[e, k] (fp32 accumulate: K splits of
// router_ksplit(T, H, E) partial sums in part [ks, T, E], added in split
// order), then per token the top-k (descending, ties to the lower id) and the
// softmax of the k values.
int router_ksplit(int T, int H, int E);
hipError_t launch_router_topk(const uint16_t* x, const uint16_t* w_rt, int T, int H, int E, int topk, float* logits,
                              int32_t* ids, float* wts, float* part, hipStream_t stream);

// NVFP4 quantization of x [M, K]; with compute_gs the per-workgroup maxima of
// |x| go to slots (quantize_workspace_bytes()) and gs = amax / 2688 is
// written to *gs, else *gs is read.
size_t quantize_workspace_bytes();
hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, float* gs, int compute_gs,
                               uint8_t* q, uint8_t* sf, unsigned* slots, hipStream_t stream);

}  // namespace nvfp4
