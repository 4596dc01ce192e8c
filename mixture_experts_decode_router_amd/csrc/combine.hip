// Deterministic per-token combine: out[t][c] = sum_{j=0..k-1} w[t][j] * y[t*k+j][c],
// j ascending, fp32 fused multiply-adds in a fixed order and no atomics.  It
// takes the place of the index_add_ of the grouped MoE path (unsloth commit
// 80aaf1121b page, third paragraph), whose float atomics make the sum order,
// and so the result, vary from run to run.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 16;  // largest top-k the configuration check accepts

template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * kThreads + threadIdx.x) * 4;
  if (c >= a.H) return;
  if (a.live && t >= *a.live) return;  // row past the live count of a graph replay
  const float* w = a.wts + (size_t)t * a.k;
  const float* y = a.y + (size_t)t * a.k * a.H + c;
  // all k rows are loaded before the first multiply-add (one memory round
  // trip instead of k), with the streaming hint since each is read once; the
  // sum still runs over j ascending
  f32x4_t v[kMaxK];
  float wv[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < a.k) {
      wv[j] = w[j];
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + (size_t)j * a.H));
    }
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < a.k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wv[j], v[j][q], acc[q]);
    }
  }
  if (BF16) {
    const u32x2_t pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + (size_t)t * a.H + c) = pk;
  } else {
    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + (size_t)t * a.H + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const dim3 grid(a.T, (a.H / 4 + kThreads - 1) / kThreads);
  if (a.out_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}


}  // namespace moe
