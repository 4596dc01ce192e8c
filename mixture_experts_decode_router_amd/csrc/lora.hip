// LoRA down-projections of the grouped expert GEMMs: for every routed row p
// of a work item (expert e, up to 16 of its rows),
//   U[p][j] = sum_k A[e][j][k] * src[row(p)][k],   j < 16 (the adapter rank)
// with src the block input x (row = the token of slot perm[p]) for the
// gate/up adapter, or h (row = p) for the down adapter.  The expert GEMM
// epilogues then add scale * sum_j B[e][n][j] * U[p][j] to their fp32
// accumulators (the rank-16, fp32-adapter LoRA of the unsloth commit
// 4f2bfe7f69 page's workload, injected into the grouped GEMMs).
//
// One workgroup per item; K is cut into 64-k blocks, block b going to wave
// b % 16 (at most four per wave).  The 16 x 16 tile U^T = A[e] (16 x K) *
// src^T (K x 16 rows) is one fp32 MFMA accumulation per wave over its blocks
// in order (16x16x4: lane (r, g) feeds A row r and the column of row r,
// k = 16g + i in the i-th MFMA of a block, so every lane reads 16 consecutive
// k of each operand); the waves' tiles are then added in wave order.  A row's U depends only on its input row and expert, never
// on the batch.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRank = 16;
constexpr int kWaves = 16;
constexpr int kMaxBlocks = 4;  // 64-k blocks per wave (K <= 64 * 4 * 16 = 4096)

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(64 * kWaves) void lora_a_kernel(LoraAArgs a) {
  __shared__ f32x4_t s_part[kWaves][64];
  const int item = blockIdx.x;
  if (item >= *a.n_items) return;  // uniform over the workgroup
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int c = a.counts[e] - m0;
  const int M = c < 16 ? c : 16, base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = a.K / 64;                  // 64-k blocks
  const int nw = nb < kWaves ? nb : kWaves;  // waves holding at least one
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (wave < nw) {
    const bool tv = r < M;
    const int row = tv ? (a.by_token ? a.perm[base + r] / a.k : base + r) : 0;
    const uint16_t* xr = a.src + (size_t)row * a.K + 16 * g;
    const float* ar = a.A + ((size_t)e * kRank + r) * a.K + 16 * g;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    f32x4_t av[kMaxBlocks][4];
    u32x4_t xv[kMaxBlocks][2];
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      const int b = wave + kWaves * i;
      if (b < nb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) av[i][v] = *reinterpret_cast<const f32x4_t*>(ar + 64 * b + 4 * v);
#pragma unroll
        for (int v = 0; v < 2; ++v) xv[i][v] = tv ? ld16(xr + 64 * b + 8 * v) : zero;
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      if (wave + kWaves * i < nb) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const uint32_t w = xv[i][m >> 3][(m & 7) >> 1];
          acc = mfma_f32(av[i][m >> 2][m & 3], (m & 1) ? bf16hi(w) : bf16lo(w), acc);
        }
      }
    }
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  // lane l of each wave holds D[4(l/16) + q][l % 16] = U[row l % 16][j = 4(l/16) + q]
  if (tid < 256) {
    const int l = tid & 63, q = tid >> 6;
    const int tok = l & 15, j = 4 * (l >> 4) + q;
    if (tok < M) {
      float sum = 0.f;
      for (int w = 0; w < nw; ++w) sum += s_part[w][l][q];
      a.U[(size_t)(base + tok) * kRank + j] = sum;
    }
  }
}

}  // namespace

hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s) {
  if (a.K % 64 || a.K > 64 * kMaxBlocks * kWaves) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_a_kernel, dim3(a.max_items), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
