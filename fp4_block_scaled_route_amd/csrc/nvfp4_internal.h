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
  A_BF16 = 0,  // bf16 rows, widened to fp16 with a per-row power-of-two shift
  A_F32 = 1,   // fp32 rows (hidden h), same per-row shift taken from a row max
  A_FP4 = 2    // NVFP4 rows, decoded exactly to fp16 (global scale in the epilogue)
};

// Epilogues of the grouped GEMM.
enum EpiMode {
  EPI_Y_BF16 = 0,      // y[row, n] = bf16(alpha * acc)                    (dense linear)
  EPI_SWIGLU_F32 = 1,  // h[row, i] = silu(alpha*gate) * (alpha*up), fp32, + row max |h|
  EPI_SWIGLU_FP4 = 2,  // same h, quantized to NVFP4 with a supplied global scale
  EPI_SLOT = 3         // slot[pair, n] = alpha * acc, fp32                (down GEMM)
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
  // glist/gcount give the processing order.  Dense: offsets == nullptr, rows [0, M).
  const int* offsets;
  const int* glist;
  const int* gcount;
  int M;               // dense row count
  int nb;              // weight-row blocks per group (grid = groups * nb)
  // Activation operand.
  const void* a;       // see AMode; row pitch in elements = K
  const uint8_t* a_sf; // NVFP4 block scales [rows, K/16]
  int a_by_token;      // 1: A row = token of the sorted row (via perm); 0: A row = sorted row
  const int* perm;     // sorted row -> pair id (pair < P: token = pair / topk; else pair - P)
  int topk;
  int P;               // T * topk
  const int* rowshift; // A_BF16: per A row, power-of-two shift applied when staging
  const unsigned* rowmax;  // A_F32: per A row, bits of max |value|
  const float* gsa;    // activation global scale (nullptr = 1)
  // Outputs.
  float* h;            // [rows, I] fp32 (EPI_SWIGLU_F32)
  unsigned* hmax;      // [rows] bits of max|h| (EPI_SWIGLU_F32)
  uint8_t* hq;         // [rows, I/2] (EPI_SWIGLU_FP4)
  uint8_t* hq_sf;      // [rows, I/16]
  const float* h_gs;   // global scale used to quantize h (EPI_SWIGLU_FP4)
  float* slot;         // [pairs, N] (EPI_SLOT), row = perm[sorted row]
  uint16_t* y;         // [M, N] bf16 (EPI_Y_BF16)
};

// Tile shape choice of one GEMM launch.
struct GemmShape {
  int maxc;   // token chunks of 16 per pass (1, 2, 4, 8)
  int r;      // 16-row weight fragments per wave
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
  int* gcount;         // [1]
  int32_t* offsets_out;  // optional copies
  int32_t* perm_out;
  // row shifts of the bf16 activations (optional) and zeroing of a row-max buffer
  const uint16_t* x;   // [T, H] bf16 or nullptr
  int H;
  int* rowshift;       // [T]
  unsigned* zero_buf;  // [n_zero] set to 0, or nullptr
  int n_zero;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);

hipError_t launch_rowshift_bf16(const uint16_t* x, int rows, int cols, int* rowshift,
                                hipStream_t stream);
hipError_t launch_amax_to_gs(const unsigned* rowmax, int rows, float* gs_out, hipStream_t stream);

struct CombineArgs {
  const float* slot;    // [P + T, H]
  const int32_t* ids;   // [T, topk]
  const float* w;       // [T, topk]
  int T, topk, E, H, shared;
  uint16_t* y;          // [T, H] bf16
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, float* gs, int compute_gs,
                               uint8_t* q, uint8_t* sf, hipStream_t stream);

}  // namespace nvfp4
