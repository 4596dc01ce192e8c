// LoRA down-projections of the grouped expert GEMMs: for every routed row p
// of a work item (expert e, up to 16 of its rows),
//   U[p][j] = sum_k A[e][j][k] * src[row(p)][k],   j < 16 (the adapter rank)
// with src the block input x (row = the token of slot perm[p]) for the
// gate/up adapter, or h (row = p) for the down adapter.  The expert GEMM
// epilogues then add scale * sum_j B[e][n][j] * U[p][j] to their fp32
// accumulators (the rank-16, fp32-adapter LoRA of the unsloth commit
// 4f2bfe7f69 page's workload, injected into the grouped GEMMs).
//
// One workgroup per item, 16 waves each taking a 1/16 slice of K; lane
// (t, g) forms rows j = 4g..4g+3 of token t over its slice with fp32 fma in k
// order; the 16 slice sums are then added in wave order.  A row's U depends
// only on its input row and expert, never on the batch.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRank = 16;
constexpr int kWaves = 16;

__global__ __launch_bounds__(64 * kWaves) void lora_a_kernel(LoraAArgs a) {
  __shared__ float s_part[kWaves][16][kRank + 1];
  const int item = blockIdx.x;
  if (item >= *a.n_items) return;  // uniform over the workgroup
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int c = a.counts[e] - m0;
  const int M = c < 16 ? c : 16, base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15, g = lane >> 4;
  const bool tv = t < M;
  const int row = tv ? (a.by_token ? a.perm[base + t] / a.k : base + t) : 0;
  const int kr = a.K / kWaves, k0 = wave * kr;
  const uint16_t* xr = a.src + (size_t)row * a.K + k0;
  const float* ar = a.A + ((size_t)e * kRank + 4 * g) * a.K + k0;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < kr; kk += 8) {
    const u32x4_t xv = tv ? ld16(xr + kk) : zero;
    float xf[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xf[2 * q] = bf16lo(xv[q]);
      xf[2 * q + 1] = bf16hi(xv[q]);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(ar + (size_t)jj * a.K + kk);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(ar + (size_t)jj * a.K + kk + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[jj] = fmaf(xf[q], a0[q], acc[jj]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[jj] = fmaf(xf[4 + q], a1[q], acc[jj]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) s_part[wave][t][4 * g + jj] = acc[jj];
  __syncthreads();
  if (tid < 16 * kRank) {
    const int tt = tid / kRank, j = tid - tt * kRank;
    if (tt < M) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += s_part[w][tt][j];
      a.U[(size_t)(base + tt) * kRank + j] = sum;
    }
  }
}

}  // namespace

hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lora_a_kernel, dim3(a.max_items), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
