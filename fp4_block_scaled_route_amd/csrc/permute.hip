// Token -> expert permutation for the grouped GEMM (gfx950).
//
// The grouped GEMM takes int32 segment offsets of the rows of each expert
// (page "nvfp4-megamoe-kernel, commit 4c6464e - vllm", note on the custom-op
// GEMM implementation).  Rows are the (token, slot) pairs f = t*topk + j,
// grouped by expert id, stable in f; the shared expert's group of T rows
// follows the routed groups.
//
// A workgroup of 16 waves ranks a contiguous range of the pairs:
//   1. wave w counts the ids of its contiguous piece of the range into its own
//      LDS histogram row (LDS atomics: order-free, exact);
//   2. per expert, an exclusive scan over the 16 rows gives each wave's base
//      inside the expert's group; an exclusive scan over experts gives the
//      group offsets;
//   3. each wave walks its piece 64 pairs at a time; lanes holding the same
//      expert find each other with one ballot per id bit, rank themselves by
//      lane order (so the order inside a group is the pair order), and the
//      highest of them advances the wave's counter for that expert.
// Up to 8191 pairs one workgroup takes them all.  Beyond, several workgroups
// take consecutive ranges (three launches: counts per workgroup and expert; a
// scan over the workgroups; ranks), so the rows of a group still come in pair
// order.  The group offsets also give the processing order of the groups for
// the GEMM (non-empty groups, largest first by a counting sort over the
// sizes, ties by id), so that the GEMM grid needs no host synchronisation.
// Extra workgroups compute the per-row staging shifts of the bf16 activations
// and clear the row-max buffer of the hidden activations.
#include <algorithm>

#include "device_util.h"

namespace nvfp4 {

namespace {
constexpr int kPermWaves = 16;
constexpr int kMaxExperts = 512;
// pair counts from which the permutation runs on several workgroups, and
// their largest number (each takes whole steps of 1024 pairs)
constexpr int kPermMultiMin = 8192;
constexpr int kPermMaxBlocks = 64;
}  // namespace

// One wave per row: max |x| of the bf16 row, the power-of-two shift that maps
// it into [2^14, 2^15), and the fp16 copy of the row scaled by that power of
// two (exact: bf16 values have 8 significant bits), stored step-major.
//
// Rows of at most NV * 512 elements are read once, all loads of the row
// issued together and held in registers (one memory round trip per row);
// longer rows are read twice, 512 elements per step.
template <int NV>
__device__ void rows_to_f16_held(const uint16_t* x, int rows, int cols, int* rowshift, f16* x16, int first_wave,
                                 int wave_stride) {
  const int lane = threadIdx.x & 63;
  for (int r = first_wave; r < rows; r += wave_stride) {
    const uint16_t* row = x + (int64_t)r * cols;
    uint4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (lane + 64 * i) * 8;
      v[i] = c < cols ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx = max(mx, u[e] & 0x7FFFu);
        mx = max(mx, (u[e] >> 16) & 0x7FFFu);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    const int sh = shift_from_maxbits(mx << 16);
    if (lane == 0) rowshift[r] = sh;
    f16* out = x16 + (int64_t)r * cols;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = (lane + 64 * i) * 8;
      if (c >= cols) continue;
      const uint32_t u[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] & 0xFFFFu), sh);
        o[2 * e + 1] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] >> 16), sh);
      }
      *reinterpret_cast<f16x8*>(out + step_major_pos(c)) = o;
    }
  }
}

__device__ void rows_to_f16(const uint16_t* x, int rows, int cols, int* rowshift, f16* x16, int first_wave,
                            int wave_stride) {
  if (cols <= 4 * 512) return rows_to_f16_held<4>(x, rows, cols, rowshift, x16, first_wave, wave_stride);
  if (cols <= 8 * 512) return rows_to_f16_held<8>(x, rows, cols, rowshift, x16, first_wave, wave_stride);
  if (cols <= 16 * 512) return rows_to_f16_held<16>(x, rows, cols, rowshift, x16, first_wave, wave_stride);
  const int lane = threadIdx.x & 63;
  for (int r = first_wave; r < rows; r += wave_stride) {
    const uint16_t* row = x + (int64_t)r * cols;
    uint32_t mx = 0;
    for (int c = lane * 8; c < cols; c += 64 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx = max(mx, u[e] & 0x7FFFu);
        mx = max(mx, (u[e] >> 16) & 0x7FFFu);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    const int sh = shift_from_maxbits(mx << 16);
    if (lane == 0) rowshift[r] = sh;
    f16* out = x16 + (int64_t)r * cols;
    for (int c = lane * 8; c < cols; c += 64 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] & 0xFFFFu), sh);
        o[2 * e + 1] = (f16)__builtin_ldexpf(bf16_bits_to_float(u[e] >> 16), sh);
      }
      *reinterpret_cast<f16x8*>(out + step_major_pos(c)) = o;
    }
  }
}

namespace {

// LDS of one permutation workgroup (16 waves).
struct PermLds {
  int hist[kPermWaves][kMaxExperts];  // per wave: id counts, then the wave's base inside each expert
  int base[kMaxExperts + 2];          // per expert: first sorted row of this workgroup's pairs / group offsets
  int gsize[kMaxExperts + 4];         // rows of each group (group order)
};

// Phase 1: wave w of the workgroup counts the ids of its contiguous piece of
// the pairs [b0, b1) into hist[w] (LDS atomics: order-free, exact).  The
// piece is a multiple of 64 pairs; ids are read kBatch steps at a time, so
// the global load latency is paid once per batch.
__device__ void count_ids(const int32_t* ids, int E, int b0, int b1, PermLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kPermWaves * E; i += blockDim.x) L.hist[i / E][i % E] = 0;
  __syncthreads();
  const int seg = ((b1 - b0 + kPermWaves - 1) / kPermWaves + 63) & ~63;
  const int f0 = b0 + wave * seg, f1 = min(b1, f0 + seg);
  constexpr int kBatch = 8;
  for (int fb = f0; fb < f1; fb += 64 * kBatch) {
    int idv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int f = fb + 64 * u + lane;
      idv[u] = f < f1 ? ids[f] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (idv[u] >= 0 && idv[u] < E) atomicAdd(&L.hist[wave][idv[u]], 1);
  }
  __syncthreads();
}

// Phase 2a: per expert, exclusive scan of the counts over the waves (wave
// order = pair order); returns nothing, the totals go to tot[e] if tot.
__device__ void scan_waves(int E, PermLds& L, int* tot) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      const int c = L.hist[w][e];
      L.hist[w][e] = run;
      run += c;
    }
    if (tot) tot[e] = run;
  }
  __syncthreads();
}

// Phase 2b: L.base[e + 1] holds group e's row count on entry; on exit L.base
// holds the exclusive prefix (group offsets), base[E] = routed rows and
// base[E + 1] = base[E] + the shared group's T rows.  Wave 0: each lane sums
// a contiguous piece of experts, then a shuffle scan of the lane sums.
__device__ void scan_experts(int E, int shared_rows, PermLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int per = (E + 63) / 64;
    const int e0 = lane * per, e1 = min(E, e0 + per);
    int s = 0;
    for (int e = e0; e < e1; ++e) s += L.base[e + 1];
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - s;
    for (int e = e0; e < e1; ++e) {
      const int c = L.base[e + 1];
      L.base[e] = run;
      run += c;
    }
    if (lane == 63) {
      L.base[E] = incl;
      L.base[E + 1] = incl + shared_rows;
    }
  }
  __syncthreads();
}

// Phase 3: stable ranks.  Wave w walks its piece of [b0, b1) 64 pairs at a
// time; lanes holding the same expert find each other with one ballot per id
// bit and rank themselves by lane order, so the order inside a group is the
// pair order: row = L.base[id] + L.hist[w][id] + rank; the highest of those
// lanes advances the wave's count.  Pairs with an id outside [0, E) get
// inv = -1 and no row.
__device__ void rank_pairs(const PermuteArgs& a, int b0, int b1, PermLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E;
  const int seg = ((b1 - b0 + kPermWaves - 1) / kPermWaves + 63) & ~63;
  const int f0 = b0 + wave * seg, f1 = min(b1, f0 + seg);
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  constexpr int kBatch = 8;
  int idv[kBatch];
  for (int fb = f0; fb < f1; fb += 64) {
    const int u = ((fb - f0) >> 6) % kBatch;   // wave-uniform
    if (u == 0) {
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int fv = fb + 64 * v + lane;
        idv[v] = fv < f1 ? a.ids[fv] : -1;
      }
    }
    const int f = fb + lane;
    int id = -1;
#pragma unroll
    for (int v = 0; v < kBatch; ++v)
      if (v == u) id = idv[v];
    if (id < 0 || id >= E) id = -1;
    uint64_t peers = __ballot(id >= 0);
#pragma unroll 1
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot(id >= 0 && ((id >> b) & 1));
      peers &= ((id >> b) & 1) ? bal : ~bal;
    }
    if (id >= 0) {
      const uint64_t below = peers & ((1ull << lane) - 1ull);
      const int rank = __popcll(below);
      const int pos = L.base[id] + L.hist[wave][id] + rank;
      a.perm[pos] = f;
      a.inv[f] = pos;
      if (a.perm_out) a.perm_out[pos] = f;
      if ((peers >> lane) == 1ull) L.hist[wave][id] += __popcll(peers);  // highest peer lane
    } else if (f < f1) {
      a.inv[f] = -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
}

// Phase 4, with the group offsets in L.base: the shared expert's rows, the
// offsets, and the processing order of the groups for the GEMM (non-empty
// groups, largest first, ties by id; sizes of kSizeKeys - 1 rows or more
// count as equal), so that the GEMM grid needs no host synchronisation.  A
// counting sort: the groups per size (LDS atomics, order-free), an exclusive
// scan over the sizes from the largest down gives each size's first list
// position, and one wave places the groups in id order, 64 at a time (lanes
// of equal size find each other with one ballot per size bit and take
// consecutive positions in lane order).
constexpr int kSizeKeys = 4096;
__device__ void finish_groups(const PermuteArgs& a, PermLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.T * a.topk;
  const int pv = L.base[E];
  if (a.shared) {
    for (int t = tid; t < a.T; t += blockDim.x) {
      a.perm[pv + t] = P + t;
      a.inv[P + t] = pv + t;
      if (a.perm_out) a.perm_out[pv + t] = P + t;
    }
  }
  for (int i = tid; i < E + 2; i += blockDim.x) {
    a.offsets[i] = L.base[i];
    if (a.offsets_out) a.offsets_out[i] = L.base[i];
  }
  const int G = E + (a.shared ? 1 : 0);
  const int G4 = (G + 3) & ~3;
  // the per-wave histograms are free now: counts per size, then per-wave sums
  static_assert(sizeof(L.hist) >= (kSizeKeys + 64) * sizeof(int), "size keys fit the histogram rows");
  int* cnt = &L.hist[0][0];
  int* wsum = cnt + kSizeKeys;
  __syncthreads();   // (the ranks of phase 3 read L.hist)
  for (int i = tid; i < kSizeKeys; i += blockDim.x) cnt[i] = 0;
  for (int h = tid; h < G4; h += blockDim.x) L.gsize[h] = h < G ? L.base[h + 1] - L.base[h] : -1;
  __syncthreads();
  for (int g = tid; g < G; g += blockDim.x) {
    const int m = L.gsize[g];
    if (m > 0) atomicAdd(&cnt[min(m, kSizeKeys - 1)], 1);
  }
  __syncthreads();
  // exclusive scan from the largest size down: thread j takes the sizes
  // kSizeKeys - 1 - (per*j .. per*j + per - 1)
  {
    const int nthr = blockDim.x, per = kSizeKeys / nthr;   // (the 1024-thread workgroups: 4 sizes each)
    int s = 0;
    for (int u = 0; u < per; ++u) s += cnt[kSizeKeys - 1 - (per * tid + u)];
    int incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int run = before + incl - s;
    for (int u = 0; u < per; ++u) {
      const int key = kSizeKeys - 1 - (per * tid + u);
      const int c = cnt[key];
      cnt[key] = run;   // first list position of this size
      run += c;
    }
  }
  __syncthreads();
  if (wave == 0) {
    for (int c0 = 0; c0 < G; c0 += 64) {
      const int g = c0 + lane;
      const int m = g < G ? L.gsize[g] : 0;
      const bool valid = m > 0;
      const int key = min(max(m, 0), kSizeKeys - 1);
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 12; ++b) {
        const uint64_t bal = __ballot(valid && ((key >> b) & 1));
        peers &= ((key >> b) & 1) ? bal : ~bal;
      }
      if (valid) {
        const int pos = cnt[key] + __popcll(peers & ((1ull << lane) - 1ull));
        a.glist[pos] = g;
        if ((peers >> lane) == 1ull) cnt[key] += __popcll(peers);   // the highest lane of this size
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  if (tid < 64) {
    int cnt = 0, big = 0;
    for (int g = lane; g < G; g += 64) {
      const int mg = L.gsize[g];
      cnt += mg > 0;
      big += mg > kBigGroupRows;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      cnt += __shfl_xor(cnt, o);
      big += __shfl_xor(big, o);
    }
    if (lane == 0) {
      a.gcount[0] = cnt;
      a.gcount[1] = big;
    }
  }
}

// Work of the workgroups after the permutation's own: row shifts and fp16
// copy of x, clearing of the row-max buffer of the hidden activations and of
// the GEMMs' split counters.
__device__ void side_work(const PermuteArgs& a, int first_block) {
  const int nblk = gridDim.x - first_block, b = blockIdx.x - first_block;
  const int nwav = nblk * (blockDim.x / 64);
  const int w = b * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (a.x) rows_to_f16(a.x, a.T, a.H, a.rowshift, a.x16, w, nwav);
  if (a.zero_buf)
    for (int i = b * blockDim.x + threadIdx.x; i < a.n_zero; i += nblk * blockDim.x) a.zero_buf[i] = 0u;
  if (a.zero_buf2)
    for (int i = b * blockDim.x + threadIdx.x; i < a.n_zero2; i += nblk * blockDim.x) a.zero_buf2[i] = 0u;
}

}  // namespace

// One workgroup does the whole permutation (pair counts below
// kPermMultiMin); workgroups 1.. do the side work.
__global__ __launch_bounds__(1024) void nvfp4_moe_permute(const PermuteArgs a) {
  if (blockIdx.x > 0) {
    side_work(a, 1);
    return;
  }
  __shared__ __attribute__((aligned(16))) PermLds L;
  const int E = a.E, P = a.T * a.topk;
  count_ids(a.ids, E, 0, P, L);
  scan_waves(E, L, &L.base[1]);
  scan_experts(E, a.shared ? a.T : 0, L);
  rank_pairs(a, 0, P, L);
  finish_groups(a, L);
}

// Larger pair counts: nb workgroups, workgroup b taking the pairs
// [b * seg, (b + 1) * seg), in three launches.
// 1. per workgroup and expert, the number of pairs: bcnt[b * E + e]
//    (workgroups nb.. do the side work);
__global__ __launch_bounds__(1024) void nvfp4_perm_count(const PermuteArgs a, int nb, int seg, int* bcnt) {
  if ((int)blockIdx.x >= nb) {
    side_work(a, nb);
    return;
  }
  __shared__ __attribute__((aligned(16))) PermLds L;
  const int E = a.E, P = a.T * a.topk;
  const int b0 = blockIdx.x * seg, b1 = max(b0, min(P, b0 + seg));
  count_ids(a.ids, E, b0, b1, L);
  scan_waves(E, L, bcnt + (int64_t)blockIdx.x * E);
}

// 2. one workgroup: per expert, exclusive scan over the workgroups (in place:
//    bcnt[b * E + e] becomes workgroup b's first row inside group e), group
//    offsets, shared rows and group order;
__global__ __launch_bounds__(1024) void nvfp4_perm_scan(const PermuteArgs a, int nb, int* bcnt) {
  __shared__ __attribute__((aligned(16))) PermLds L;
  const int E = a.E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    // counts requested 16 at a time before their first use (one memory
    // round trip per 16 workgroups instead of one per workgroup)
    constexpr int kB = 16;
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = b0 + u < nb ? bcnt[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (b0 + u < nb) bcnt[(int64_t)(b0 + u) * E + e] = run;
        run += c[u];
      }
    }
    L.base[e + 1] = run;
  }
  __syncthreads();
  scan_experts(E, a.shared ? a.T : 0, L);
  finish_groups(a, L);
}

// 3. per workgroup: the counts again, scanned over its waves; ranks from the
//    group offset + the workgroup's first row in the group.
__global__ __launch_bounds__(1024) void nvfp4_perm_rank(const PermuteArgs a, int seg, const int* bcnt) {
  __shared__ __attribute__((aligned(16))) PermLds L;
  const int E = a.E, P = a.T * a.topk;
  const int b0 = blockIdx.x * seg, b1 = max(b0, min(P, b0 + seg));
  count_ids(a.ids, E, b0, b1, L);
  scan_waves(E, L, nullptr);
  for (int e = threadIdx.x; e < E; e += blockDim.x) L.base[e] = a.offsets[e] + bcnt[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  rank_pairs(a, b0, b1, L);
}

__global__ __launch_bounds__(256) void nvfp4_rows_to_f16(const uint16_t* x, int rows, int cols, int* rowshift,
                                                         f16* x16) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  rows_to_f16(x, rows, cols, rowshift, x16, w, gridDim.x * 4);
}

// fp16 copy of the fp32 hidden rows with per-row shifts from max |h|, stored
// step-major.
__global__ __launch_bounds__(256) void nvfp4_h_to_f16(const float* h, const unsigned* hmax, const int* offsets,
                                                      int end_index, int cols, f16* h16, int* hshift) {
  const int rows = offsets[end_index];
  const int lane = threadIdx.x & 63;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += gridDim.x * 4) {
    const int sh = shift_from_maxbits(hmax[r]);
    if (lane == 0) hshift[r] = sh;
    const float* src = h + (int64_t)r * cols;
    f16* dst = h16 + (int64_t)r * cols;
    for (int c = lane * 8; c < cols; c += 64 * 8) {
      const float4 v0 = *reinterpret_cast<const float4*>(src + c);
      const float4 v1 = *reinterpret_cast<const float4*>(src + c + 4);
      const f16x8 o = {(f16)__builtin_ldexpf(v0.x, sh), (f16)__builtin_ldexpf(v0.y, sh),
                       (f16)__builtin_ldexpf(v0.z, sh), (f16)__builtin_ldexpf(v0.w, sh),
                       (f16)__builtin_ldexpf(v1.x, sh), (f16)__builtin_ldexpf(v1.y, sh),
                       (f16)__builtin_ldexpf(v1.z, sh), (f16)__builtin_ldexpf(v1.w, sh)};
      *reinterpret_cast<f16x8*>(dst + step_major_pos(c)) = o;
    }
  }
}

// gs = (max over rows of the row maxima) / 2688 for calibrating the global
// scale of the hidden activations (page "commit 4c6464e", notes on warm-up
// calibration of the activation global scale).
__global__ __launch_bounds__(1024) void nvfp4_amax_to_gs(const unsigned* rowmax, int rows, float* gs_out) {
  __shared__ unsigned wmax[16];
  unsigned m = 0;
  for (int i = threadIdx.x; i < rows; i += blockDim.x) m = max(m, rowmax[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = max(r, wmax[w]);
    gs_out[0] = __uint_as_float(r) / 2688.0f;
  }
}

int permute_blocks(int64_t P) {
  if (P < kPermMultiMin) return 0;
  return (int)std::min<int64_t>(kPermMaxBlocks, (P + kPermMultiMin / 8 - 1) / (kPermMultiMin / 8));
}

hipError_t launch_permute(const PermuteArgs& a, int* bcnt, hipStream_t s) {
  if (a.E > kMaxExperts) return hipErrorInvalidValue;
  int extra = 0;
  if (a.x || a.zero_buf || a.zero_buf2) {
    const int by_rows = a.x ? (a.T + 15) / 16 : 0;   // 16 waves per block, one row each
    // (clearing takes at most 4 extra workgroups: they loop over the words)
    const int by_zero = min(4, max(a.zero_buf ? (a.n_zero + 1023) / 1024 : 0, a.zero_buf2 ? (a.n_zero2 + 1023) / 1024 : 0));
    extra = max(1, min(1024, max(by_rows, by_zero)));
  }
  const int P = a.T * a.topk;
  const int nb = permute_blocks(P);
  if (nb == 0) {
    hipLaunchKernelGGL(nvfp4_moe_permute, dim3(1 + extra), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  if (!bcnt) return hipErrorInvalidValue;
  // pieces of whole 1024-pair steps (64 pairs per wave)
  const int seg = ((P + nb - 1) / nb + 1023) & ~1023;
  hipLaunchKernelGGL(nvfp4_perm_count, dim3(nb + extra), dim3(1024), 0, s, a, nb, seg, bcnt);
  hipLaunchKernelGGL(nvfp4_perm_scan, dim3(1), dim3(1024), 0, s, a, nb, bcnt);
  hipLaunchKernelGGL(nvfp4_perm_rank, dim3(nb), dim3(1024), 0, s, a, seg, static_cast<const int*>(bcnt));
  return hipGetLastError();
}

hipError_t launch_rows_to_f16(const uint16_t* x, int rows, int cols, int* rowshift, f16* x16, hipStream_t s) {
  const int grid = max(1, min(2048, (rows + 3) / 4));
  hipLaunchKernelGGL(nvfp4_rows_to_f16, dim3(grid), dim3(256), 0, s, x, rows, cols, rowshift, x16);
  return hipGetLastError();
}

hipError_t launch_h_to_f16(const float* h, const unsigned* hmax, const int* offsets, int end_index, int rows_max,
                           int cols, f16* h16, int* hshift, hipStream_t s) {
  const int grid = max(1, min(2048, (rows_max + 3) / 4));
  hipLaunchKernelGGL(nvfp4_h_to_f16, dim3(grid), dim3(256), 0, s, h, hmax, offsets, end_index, cols, h16, hshift);
  return hipGetLastError();
}

hipError_t launch_amax_to_gs(const unsigned* rowmax, int rows, float* gs_out, hipStream_t s) {
  hipLaunchKernelGGL(nvfp4_amax_to_gs, dim3(1), dim3(1024), 0, s, rowmax, rows, gs_out);
  return hipGetLastError();
}

}  // namespace nvfp4
