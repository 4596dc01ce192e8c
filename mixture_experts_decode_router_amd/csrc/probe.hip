// Measurement probes: the achievable rates of this chip for the two kinds
// of work the block does, measured beside it (HBM streaming for the decode
// expert GEMMs, bf16 matrix-core throughput for the prefill ones).
//
// read:  every byte of a buffer is loaded once with the load form the decode
//        expert GEMMs stream their weights with (16-byte non-temporal loads,
//        each wave instruction one contiguous KiB, each wave walking its own
//        contiguous range with 8 loads in flight) and folded into one XOR
//        per wave, so no load can be dropped.
// mfma:  each wave issues `iters` rounds of independent bf16 MFMAs on
//        register operands (16x16x32: 8 accumulators; 32x32x16: 4), no
//        memory traffic, and writes the sum of its accumulators.
// gather: each wave copies 16-row x 64-byte tiles of a row-major buffer
//        global -> LDS with global_load_lds_dwordx4, as the prefill expert
//        GEMMs copy gathered token rows, with the lanes either one row each
//        (the MFMA operand order) or four per 64-byte row segment.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeU = 8;

// wave w of the grid streams its own contiguous range of whole kilobytes
// (as a decode expert GEMM wave streams its weight tile), kProbeU of them
// in flight; the tail past the last whole kilobyte goes to the first waves
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* src, size_t n16, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const size_t nwaves = (size_t)gridDim.x * (kProbeThreads / 64);
  const size_t w = (size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const size_t nkb = n16 / 64;
  const size_t per = (nkb + nwaves - 1) / nwaves;
  const size_t k0 = min(nkb, w * per), k1 = min(nkb, k0 + per);
  uint32_t acc = 0u;
  size_t kb = k0;
  for (; kb + kProbeU <= k1; kb += kProbeU) {
    u32x4_t v[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) v[u] = __builtin_nontemporal_load(src + (kb + u) * 64 + lane);
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; kb < k1; ++kb) {
    const u32x4_t v = __builtin_nontemporal_load(src + kb * 64 + lane);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (size_t i = nkb * 64 + w * 64 + lane; i < n16; i += nwaves * 64) {
    const u32x4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) sink[w] = acc;
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// at least four workgroups per CU: with no occupancy bound the compiler put
// the 16x16x32 accumulators in accumulation registers and rotated them
// through moves between the MFMAs of every iteration
template <int SHAPE>  // 0: 16x16x32 bf16, 1: 32x32x16 bf16
__global__ __launch_bounds__(kProbeThreads, 4) void probe_mfma_kernel(float* sink, int iters) {
  const uint32_t l = threadIdx.x;
  // operands: small bf16 values (1 + l/64 and 2^-4), so the sums stay finite
  const uint32_t av = 0x3f80u + (l & 63u), bv = 0x3d80u;
  const u32x4_t a = {av | (av << 16), av | (av << 16), av | (av << 16), av | (av << 16)};
  const u32x4_t b = {bv | (bv << 16), bv | (bv << 16), bv | (bv << 16), bv | (bv << 16)};
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{(float)j, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = mfma16(a, b, acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][q] = (float)j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                         acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) s += acc[j][q];
  }
  sink[(size_t)blockIdx.x * kProbeThreads + l] = s;
}

typedef __attribute__((address_space(3))) char probe_lds_t;
#define MOE_P_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Tile u of the buffer: row group u >> seg_log (16 rows), 64-byte segment
// u & (segs - 1) of each row.  Wave w copies tiles w, w + nwaves, ... (mod
// the tile count), 8 per batch into its 8 KiB of LDS, then folds the batch
// into its XOR (one read of each LDS word), so no copy can be dropped.
__global__ __launch_bounds__(kProbeThreads) void probe_gather_kernel(const uint8_t* src, uint32_t row_bytes,
                                                                      uint32_t seg_log, uint32_t tiles, int iters,
                                                                      int order, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) u32x4_t s_buf[kProbeThreads / 64][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t nwaves = gridDim.x * (kProbeThreads / 64);
  uint32_t u = (blockIdx.x * (kProbeThreads / 64) + wave) % tiles;
  const uint32_t step = nwaves % tiles;
  const int row = order == 0 ? (lane & 15) : (lane >> 2);
  const int chunk = order == 0 ? (lane >> 4) : (lane & 3);
  const size_t lane_off = (size_t)row * row_bytes + chunk * 16;
  uint32_t acc = 0u;
  for (int it = 0; it < iters; it += 8) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (it + b < iters) {
        const size_t off = (size_t)(u >> seg_log) * 16 * row_bytes + (size_t)(u & ((1u << seg_log) - 1u)) * 64;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + off + lane_off),
                                         (probe_lds_t*)&s_buf[wave][b][0], 16, 0, 0);
        u += step;
        if (u >= tiles) u -= tiles;
      }
    }
    __builtin_amdgcn_s_waitcnt(MOE_P_VMCNT(0));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (it + b < iters) {
        const u32x4_t v = s_buf[wave][b][lane];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads are done before the next copies land
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) sink[(size_t)blockIdx.x * (kProbeThreads / 64) + wave] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(n_wg), dim3(kProbeThreads), 0, s,
                     static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(float* sink, int n_wg, int iters, int shape, hipStream_t s) {
  if (shape == 0)
    hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3(n_wg), dim3(kProbeThreads), 0, s, sink, iters);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3(n_wg), dim3(kProbeThreads), 0, s, sink, iters);
  return hipGetLastError();
}

hipError_t launch_probe_gather(const void* src, uint32_t row_bytes, uint32_t seg_log, uint32_t tiles, int iters,
                               int order, uint32_t* sink, int n_wg, hipStream_t s) {
  hipLaunchKernelGGL(probe_gather_kernel, dim3(n_wg), dim3(kProbeThreads), 0, s, static_cast<const uint8_t*>(src),
                     row_bytes, seg_log, tiles, iters, order, sink);
  return hipGetLastError();
}

}  // namespace moe
