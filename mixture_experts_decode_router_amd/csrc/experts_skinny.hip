// Grouped expert GEMMs, "skinny" form for decode-sized groups.
//
// One workgroup = one work-list item (expert e, up to 16 of its routed rows)
// times one tile of output columns.  The item's 16 activation rows are
// gathered once into LDS (16-byte chunks XOR-swizzled by row, so the 16
// rows of one MFMA fragment fall in different banks); the weights stream
// from HBM straight into MFMA A-operands, each byte read exactly once per
// item, 8 k-steps in flight per wave.  Tokens are the 16-wide MFMA column
// block, so no cross-lane reduction is needed.  This is the grouped_mm of
// the grouped MoE path (unsloth commit 80aaf1121b page, third paragraph)
// with its gate/up GEMM, SiLU*up and down GEMM.
//
//   gate/up:  h[p][n] = silu(sum_k x[tok(p)][k] Wg[e][n][k]) * sum_k x[tok(p)][k] Wu[e][n][k]
//             (bf16 h in sorted-slot order p; 64 n per workgroup, 16 per wave)
//   down:     y[perm[p]][c] = sum_n h[p][n] Wd[e][c][n]
//             (fp32 y in flat-slot order s = t*k + j; 128 c per workgroup)
//
// 4-bit weights (NF4_B64): each lane loads 16 bytes = 32 codes of one row and
// feeds four MFMA steps with them (lane group g covers k in
// [kb + 32g, kb + 32g + 32) of a 128-k block; the activation fragment uses the
// same k assignment), dequantising codebook[code] * absmax to bf16 in
// registers.  A lane's 32 k lie in one 64-weight scale block.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kTile = kSkinnyTile;  // rows per item (MFMA column block)
constexpr int kThreads = 256;       // 4 waves

struct Item {
  int e, M, base;
};

__device__ __forceinline__ bool load_item(const ExpertArgs& a, int item, Item& it) {
  if (item >= *a.n_items) return false;
  it.e = a.items[2 * item];
  const int m0 = a.items[2 * item + 1];
  const int c = a.counts[it.e] - m0;
  it.M = c < kTile ? c : kTile;
  it.base = a.offsets[it.e] + m0;
  return true;
}

// LDS tile: 16 rows x nck 16-byte chunks, chunk c of row r stored at
// r * nck + (c ^ (r & sw)).
__device__ __forceinline__ int swz(int r, int c, int nck, int sw) { return r * nck + (c ^ (r & sw)); }

// Stage columns [kc, kc + 8*nck) of the item's activation rows.
// gather: row rr of the tile is x row perm[base + rr] / k (gate/up) or
// h row base + rr (down).
template <bool GATHER>
__device__ __forceinline__ void stage_rows(u32x4_t* s, const uint16_t* src, int ld, int kc, int nck,
                                           int sw, const Item& it, const int32_t* perm, int k) {
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < kTile * nck; i += kThreads) {
    const int rr = i / nck, c = i - rr * nck;
    u32x4_t v = zero;
    if (rr < it.M) {
      const int row = GATHER ? perm[it.base + rr] / k : it.base + rr;
      v = ld16(src + (size_t)row * ld + kc + c * 8);
    }
    s[swz(rr, c, nck, sw)] = v;
  }
}

__host__ __device__ __forceinline__ int lds_chunks_for(int K, int& KC) {
  const int nchunks = (K + 2047) / 2048;
  KC = K / nchunks;
  return KC / 8;
}

// ------------------------------------------------------------------ bf16
template <int U>
__global__ __launch_bounds__(kThreads) void gate_up_bf16(ExpertArgs a) {
  extern __shared__ u32x4_t s_x[];
  const int ntile = a.I / 64;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  const uint16_t* wg = a.w_gate_up + ((size_t)it.e * 2 * I + n0 + r) * H + g * 8;
  const uint16_t* wu = wg + (size_t)I * H;
  int KC;
  const int nck = lds_chunks_for(H, KC);
  const int sw = (nck & 15) == 0 ? 15 : 7;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < H; kc += KC) {
    if (kc) __syncthreads();
    stage_rows<true>(s_x, a.x, H, kc, nck, sw, it, a.perm, a.k);
    __syncthreads();
    for (int kk = 0; kk < KC; kk += 32 * U) {
      u32x4_t ga[U], ua[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ga[u] = ld16_stream(wg + kc + kk + u * 32);
        ua[u] = ld16_stream(wu + kc + kk + u * 32);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4_t b = s_x[swz(r, (kk + u * 32) / 8 + g, nck, sw)];
        accg = mfma16(ga[u], b, accg);
        accu = mfma16(ua[u], b, accu);
      }
    }
  }
  // lane holds rows n0 + 4g + q (q = 0..3) of token column r
  if (r < it.M) {
    float hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = silu(accg[q]) * accu[q];
    u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + r) * I + n0 + 4 * g) = pk;
  }
}

template <int U>
__global__ __launch_bounds__(kThreads) void down_bf16(ExpertArgs a) {
  extern __shared__ u32x4_t s_h[];
  const int ctile = a.H / 128;
  const int item = blockIdx.x / ctile, ct = blockIdx.x - item * ctile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  const uint16_t* w0 = a.w_down + ((size_t)it.e * H + c0 + r) * I + g * 8;
  const uint16_t* w1 = w0 + (size_t)16 * I;
  int KC;
  const int nck = lds_chunks_for(I, KC);
  const int sw = (nck & 15) == 0 ? 15 : 7;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < I; kc += KC) {
    if (kc) __syncthreads();
    stage_rows<false>(s_h, a.h, I, kc, nck, sw, it, a.perm, a.k);
    __syncthreads();
    for (int kk = 0; kk < KC; kk += 32 * U) {
      u32x4_t a0[U], a1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a0[u] = ld16_stream(w0 + kc + kk + u * 32);
        a1[u] = ld16_stream(w1 + kc + kk + u * 32);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const u32x4_t b = s_h[swz(r, (kk + u * 32) / 8 + g, nck, sw)];
        acc0 = mfma16(a0[u], b, acc0);
        acc1 = mfma16(a1[u], b, acc1);
      }
    }
  }
  if (r < it.M) {
    const int slot = a.perm[it.base + r];
    float* yrow = a.y + (size_t)slot * H;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 4 * g) = acc0;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 16 + 4 * g) = acc1;
  }
}

// ------------------------------------------------------------------ 4-bit
// 8 codes (one 32-bit word, element 2i in the low nibble of byte i) ->
// 8 bf16 weights codebook[code] * scale, packed in k order.
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, float sc, const float* cb) {
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (w >> (8 * i)) & 0xffu;
    o[i] = pack_bf16x2(cb[byte & 15u] * sc, cb[byte >> 4] * sc);
  }
  return o;
}

__global__ __launch_bounds__(kThreads) void gate_up_nf4(ExpertArgs a) {
  extern __shared__ u32x4_t s_x[];
  __shared__ float s_cb[16];
  const int ntile = a.I / 64;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  if (threadIdx.x < 16) s_cb[threadIdx.x] = a.codebook[threadIdx.x];
  const size_t rowg = (size_t)it.e * 2 * I + n0 + r;
  const size_t rowu = rowg + I;
  const uint8_t* qg = a.q_gate_up + rowg * (H / 2);
  const uint8_t* qu = a.q_gate_up + rowu * (H / 2);
  const float* sg = a.s_gate_up + rowg * (H / 64);
  const float* su = a.s_gate_up + rowu * (H / 64);
  int KC;
  const int nck = lds_chunks_for(H, KC);
  const int sw = (nck & 15) == 0 ? 15 : 7;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < H; kc += KC) {
    if (kc) __syncthreads();
    stage_rows<true>(s_x, a.x, H, kc, nck, sw, it, a.perm, a.k);
    __syncthreads();
    for (int kb = 0; kb < KC; kb += 128) {
      const int k0 = kc + kb + 32 * g;  // this lane's 32 k
      const u32x4_t cg = ld16_stream(qg + k0 / 2);
      const u32x4_t cu = ld16_stream(qu + k0 / 2);
      const float scg = sg[k0 / 64], scu = su[k0 / 64];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t b = s_x[swz(r, (kb + 32 * g) / 8 + st, nck, sw)];
        accg = mfma16(dequant8(cg[st], scg, s_cb), b, accg);
        accu = mfma16(dequant8(cu[st], scu, s_cb), b, accu);
      }
    }
  }
  if (r < it.M) {
    float hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = silu(accg[q]) * accu[q];
    u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + r) * I + n0 + 4 * g) = pk;
  }
}

__global__ __launch_bounds__(kThreads) void down_nf4(ExpertArgs a) {
  extern __shared__ u32x4_t s_h[];
  __shared__ float s_cb[16];
  const int ctile = a.H / 128;
  const int item = blockIdx.x / ctile, ct = blockIdx.x - item * ctile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  if (threadIdx.x < 16) s_cb[threadIdx.x] = a.codebook[threadIdx.x];
  const size_t row0 = (size_t)it.e * H + c0 + r;
  const size_t row1 = row0 + 16;
  const uint8_t* q0 = a.q_down + row0 * (I / 2);
  const uint8_t* q1 = a.q_down + row1 * (I / 2);
  const float* s0 = a.s_down + row0 * (I / 64);
  const float* s1 = a.s_down + row1 * (I / 64);
  int KC;
  const int nck = lds_chunks_for(I, KC);
  const int sw = (nck & 15) == 0 ? 15 : 7;
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int kc = 0; kc < I; kc += KC) {
    if (kc) __syncthreads();
    stage_rows<false>(s_h, a.h, I, kc, nck, sw, it, a.perm, a.k);
    __syncthreads();
    for (int kb = 0; kb < KC; kb += 128) {
      const int k0 = kc + kb + 32 * g;
      const u32x4_t c0v = ld16_stream(q0 + k0 / 2);
      const u32x4_t c1v = ld16_stream(q1 + k0 / 2);
      const float sc0 = s0[k0 / 64], sc1 = s1[k0 / 64];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t b = s_h[swz(r, (kb + 32 * g) / 8 + st, nck, sw)];
        acc0 = mfma16(dequant8(c0v[st], sc0, s_cb), b, acc0);
        acc1 = mfma16(dequant8(c1v[st], sc1, s_cb), b, acc1);
      }
    }
  }
  if (r < it.M) {
    const int slot = a.perm[it.base + r];
    float* yrow = a.y + (size_t)slot * H;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 4 * g) = acc0;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 16 + 4 * g) = acc1;
  }
}

size_t lds_bytes(int K) {
  int KC;
  const int nck = lds_chunks_for(K, KC);
  return (size_t)kTile * nck * 16;
}

template <typename F8, typename F4, typename F2>
hipError_t launch_u(int KC, F8 f8, F4 f4, F2 f2, dim3 grid, size_t lds, hipStream_t s, const ExpertArgs& a) {
  if (KC % 256 == 0)
    hipLaunchKernelGGL(f8, grid, dim3(kThreads), lds, s, a);
  else if (KC % 128 == 0)
    hipLaunchKernelGGL(f4, grid, dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL(f2, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const ExpertArgs& a, bool nf4, hipStream_t s) {
  const dim3 grid(a.max_items * (a.I / 64));
  const size_t lds = lds_bytes(a.H);
  if (nf4) {
    hipLaunchKernelGGL(gate_up_nf4, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
  }
  int KC;
  lds_chunks_for(a.H, KC);
  return launch_u(KC, gate_up_bf16<8>, gate_up_bf16<4>, gate_up_bf16<2>, grid, lds, s, a);
}

hipError_t launch_down(const ExpertArgs& a, bool nf4, hipStream_t s) {
  const dim3 grid(a.max_items * (a.H / 128));
  const size_t lds = lds_bytes(a.I);
  if (nf4) {
    hipLaunchKernelGGL(down_nf4, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
  }
  int KC;
  lds_chunks_for(a.I, KC);
  return launch_u(KC, down_bf16<8>, down_bf16<4>, down_bf16<2>, grid, lds, s, a);
}

}  // namespace moe
