// One-time conversion of row-major expert weights into the tiled
// ("MFMA-fragment") layout the expert kernels stream fastest: every 16-row x
// 32-k bf16 fragment (16-row x 128-k for 4-bit codes) is 1 KiB of contiguous
// memory in the order the 64 lanes of a wave consume it, so each 16-byte load
// of a wave covers one contiguous kilobyte.
//
// Per expert, for a matrix of R rows x K columns (gate/up: R = 2I, K = H;
// down: R = H, K = I), with rt < R/16, r < 16, g < 4:
//   bf16   16-byte chunk ((rt * K/32 + ks) * 64 + 16 g + r)
//              = W[16 rt + r][32 ks + 8 g .. 32 ks + 8 g + 7]
//   codes  16-byte chunk ((rt * K/128 + kb) * 64 + 16 g + r), dword st (0..3)
//              = codes of row 16 rt + r, k in [128 kb + 32 st + 8 g, +8)
//   scales float ((rt * K/128 + kb) * 32 + 2 r + h)
//              = absmax of row 16 rt + r, 64-block 2 kb + h
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// chunk_k: k covered by one 16-byte chunk (8 for bf16, 32 for codes)
// frag_k: k covered by one 1-KiB fragment (32 for bf16, 128 for codes)
__global__ void pack_chunks(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst, size_t n_chunks,
                            int R, int K, int chunk_k, int frag_k) {
  const size_t d = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= n_chunks) return;
  const int row_chunks = K / chunk_k;            // chunks per row
  const size_t per_expert = (size_t)R * row_chunks;
  const size_t e = d / per_expert;
  const size_t rem = d - e * per_expert;
  const int lane = (int)(rem & 63);
  const size_t frag = rem >> 6;                 // rt * (K / frag_k) + kf
  const int n_kf = K / frag_k;
  const int rt = (int)(frag / n_kf), kf = (int)(frag % n_kf);
  const int r = lane & 15, g = lane >> 4;
  const size_t row = (size_t)rt * 16 + r;
  const size_t s = e * per_expert + row * row_chunks + (size_t)kf * (frag_k / chunk_k) + g;
  dst[d] = src[s];
}

// 4-bit codes: one thread per output dword (8 codes)
__global__ void pack_codes(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, size_t n_dwords, int R,
                           int K) {
  const size_t d = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= n_dwords) return;
  const int row_dw = K / 8;                     // dwords per row
  const size_t per_expert = (size_t)R * row_dw;
  const size_t e = d / per_expert;
  const size_t rem = d - e * per_expert;
  const int st = (int)(rem & 3);
  const int lane = (int)((rem >> 2) & 63);
  const size_t blk = rem >> 8;                  // rt * (K / 128) + kb
  const int nkb = K / 128;
  const int rt = (int)(blk / nkb), kb = (int)(blk % nkb);
  const int r = lane & 15, g = lane >> 4;
  dst[d] = src[e * per_expert + ((size_t)rt * 16 + r) * row_dw + 16 * kb + 4 * st + g];
}

__global__ void pack_scales(const float* __restrict__ src, float* __restrict__ dst, size_t n, int R, int K) {
  const size_t d = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= n) return;
  const int row_sc = K / 64;
  const size_t per_expert = (size_t)R * row_sc;
  const size_t e = d / per_expert;
  const size_t rem = d - e * per_expert;
  const int n_kb = K / 128;
  const size_t blk = rem / 32;                  // rt * n_kb + kb
  const int w = (int)(rem % 32);
  const int rt = (int)(blk / n_kb), kb = (int)(blk % n_kb);
  const int r = w >> 1, h = w & 1;
  dst[d] = src[e * per_expert + ((size_t)rt * 16 + r) * row_sc + 2 * kb + h];
}

hipError_t run_chunks(const void* src, void* dst, int E, int R, int K, int chunk_k, int frag_k, hipStream_t s) {
  const size_t n = (size_t)E * R * (K / chunk_k);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(pack_chunks, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4_t*>(src),
                     static_cast<u32x4_t*>(dst), n, R, K, chunk_k, frag_k);
  return hipGetLastError();
}

hipError_t run_codes(const void* src, void* dst, int E, int R, int K, hipStream_t s) {
  const size_t n = (size_t)E * R * (K / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(pack_codes, dim3(blocks), dim3(256), 0, s, static_cast<const uint32_t*>(src),
                     static_cast<uint32_t*>(dst), n, R, K);
  return hipGetLastError();
}

hipError_t run_scales(const float* src, float* dst, int E, int R, int K, hipStream_t s) {
  const size_t n = (size_t)E * R * (K / 64);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(pack_scales, dim3(blocks), dim3(256), 0, s, src, dst, n, R, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  hipError_t e;
  if (!a.nf4) {
    if ((e = run_chunks(a.src_gate_up, a.dst_gate_up, a.E, 2 * a.I, a.H, 8, 32, s)) != hipSuccess) return e;
    return run_chunks(a.src_down, a.dst_down, a.E, a.H, a.I, 8, 32, s);
  }
  if ((e = run_codes(a.src_gate_up, a.dst_gate_up, a.E, 2 * a.I, a.H, s)) != hipSuccess) return e;
  if ((e = run_codes(a.src_down, a.dst_down, a.E, a.H, a.I, s)) != hipSuccess) return e;
  if ((e = run_scales(a.src_s_gate_up, a.dst_s_gate_up, a.E, 2 * a.I, a.H, s)) != hipSuccess) return e;
  return run_scales(a.src_s_down, a.dst_s_down, a.E, a.H, a.I, s);
}

}  // namespace moe
