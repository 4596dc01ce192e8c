// Grouped expert GEMMs, "skinny" form for decode-sized groups.
//
// One work unit = one work-list item (expert e, up to 16 of its routed rows)
// times one tile of output columns (four waves' 16-row sub-tiles).  Tokens are the 16-wide column block of
// a 16x16x32 bf16 MFMA, weights the 16-row A operand, so each wave computes
// a 16 x 16 output tile with no cross-lane reduction.  Every k-step a lane
// loads one 16-byte weight chunk per row tile (streamed from HBM once, with a
// non-temporal hint) and the matching 16-byte chunk of its token's row (hot
// in L2: a token is read by every column tile of its experts); U k-steps of
// loads are issued before any MFMA consumes them.  There is no LDS staging
// and no barrier, so weight streaming starts as soon as a wave starts.  This
// is the grouped_mm of the grouped MoE path (unsloth commit 80aaf1121b page,
// third paragraph) with its gate/up GEMM, SiLU*up and down GEMM.
//
//   gate/up:  h[p][n] = silu(sum_k x[tok(p)][k] Wg[e][n][k]) * sum_k x[tok(p)][k] Wu[e][n][k]
//             (bf16 h in sorted-slot order p; 64 n per workgroup, 16 per wave)
//   down:     y[perm[p]][c] = sum_n h[p][n] Wd[e][c][n]
//             (fp32 y in flat-slot order s = t*k + j; 128 c per workgroup)
//
// Rows of the 16-column block beyond the item's M rows carry zeros; output
// column j depends only on B column j, so they never touch valid outputs.
//
// Weights are row-major ([E][rows][K], each 16-row MFMA fragment read as 16
// rows x 64 B) or tiled (each fragment one contiguous kilobyte in lane
// order, written once by the pack kernel): the tiled layout turns every wave
// load into one contiguous 1 KiB read.
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

// ------------------------------------------------------------------ bf16
// The bf16 kernels run one wave per workgroup (4 per item x column tile):
// the finer grain keeps HBM busy through the last workgroups of the launch.
constexpr int kSub = 4;  // waves (16-row sub-tiles) per column tile

template <int U, bool TILED>
__global__ __launch_bounds__(64) void gate_up_bf16(ExpertArgs a) {
  const int ntile = a.I / 64;
  const int wave = blockIdx.x % kSub, bq = blockIdx.x / kSub;
  const int item = bq / ntile, nt = bq - item * ntile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  const bool rv = r < it.M;
  const int tok = rv ? a.perm[it.base + r] / a.k : 0;
  const uint16_t* xr = a.x + (size_t)tok * H + g * 8;
  // row-major: row n0 + r, k offset 8g, step 32 elements; tiled: fragment
  // (row tile, k-step) is 512 elements, this lane's 8 at offset 8 * lane
  const uint16_t* wg = TILED ? a.w_gate_up + (((size_t)it.e * (2 * I / 16) + n0 / 16) * (H / 32) * 64 + lane) * 8
                             : a.w_gate_up + ((size_t)it.e * 2 * I + n0 + r) * H + g * 8;
  const uint16_t* wu = TILED ? wg + (size_t)(I / 16) * (H / 32) * 512 : wg + (size_t)I * H;
  const int wstep = TILED ? 512 : 32;  // elements per k-step
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < H; kk += 32 * U) {
    u32x4_t ga[U], ua[U], xb[U];
    const size_t wo = (size_t)(kk / 32) * wstep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ga[u] = ld16_stream(wg + wo + u * wstep);
      ua[u] = ld16_stream(wu + wo + u * wstep);
      xb[u] = rv ? ld16(xr + kk + u * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accg = mfma16(ga[u], xb[u], accg);
      accu = mfma16(ua[u], xb[u], accu);
    }
  }
  // lane holds rows n0 + 4g + q (q = 0..3) of token column r
  if (rv) {
    float hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = silu(accg[q]) * accu[q];
    u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + r) * I + n0 + 4 * g) = pk;
  }
}

template <int U, bool TILED>
__global__ __launch_bounds__(64) void down_bf16(ExpertArgs a) {
  const int ctile = a.H / 128;
  const int wave = blockIdx.x % kSub, bq = blockIdx.x / kSub;
  const int item = bq / ctile, ct = bq - item * ctile;
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  const bool rv = r < it.M;
  const uint16_t* hr = a.h + (size_t)(it.base + (rv ? r : 0)) * I + g * 8;
  const uint16_t* w0 = TILED ? a.w_down + (((size_t)it.e * (H / 16) + c0 / 16) * (I / 32) * 64 + lane) * 8
                             : a.w_down + ((size_t)it.e * H + c0 + r) * I + g * 8;
  const uint16_t* w1 = TILED ? w0 + (size_t)(I / 32) * 512 : w0 + (size_t)16 * I;
  const int wstep = TILED ? 512 : 32;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < I; kk += 32 * U) {
    u32x4_t a0[U], a1[U], hb[U];
    const size_t wo = (size_t)(kk / 32) * wstep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a0[u] = ld16_stream(w0 + wo + u * wstep);
      a1[u] = ld16_stream(w1 + wo + u * wstep);
      hb[u] = rv ? ld16(hr + kk + u * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc0 = mfma16(a0[u], hb[u], acc0);
      acc1 = mfma16(a1[u], hb[u], acc1);
    }
  }
  if (rv) {
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

template <int NB, bool TILED>  // NB: 128-k blocks per loop iteration (H % (128 * NB) == 0)
__global__ __launch_bounds__(kThreads) void gate_up_nf4(ExpertArgs a) {
  __shared__ float s_cb[16];
  const int ntile = a.I / 64;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  Item it;
  if (!load_item(a, item, it)) return;
  if (threadIdx.x < 16) s_cb[threadIdx.x] = a.codebook[threadIdx.x];
  __syncthreads();
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  const bool rv = r < it.M;
  const int tok = rv ? a.perm[it.base + r] / a.k : 0;
  const uint16_t* xr = a.x + (size_t)tok * H + 32 * g;
  // per 128-k block kb: codes at qg + kb * qstep, scale at sg[kb * sstep]
  const int nkb = H / 128;
  const size_t rowg = (size_t)it.e * 2 * I + n0 + r;
  const size_t rowu = rowg + I;
  const size_t tg = (size_t)it.e * (2 * I / 16) + n0 / 16, tu = tg + I / 16;  // row tiles
  const uint8_t* qg = TILED ? a.q_gate_up + (tg * nkb * 64 + lane) * 16 : a.q_gate_up + rowg * (H / 2) + 16 * g;
  const uint8_t* qu = TILED ? a.q_gate_up + (tu * nkb * 64 + lane) * 16 : a.q_gate_up + rowu * (H / 2) + 16 * g;
  const float* sg = TILED ? a.s_gate_up + tg * nkb * 32 + 2 * r + g / 2 : a.s_gate_up + rowg * (H / 64) + g / 2;
  const float* su = TILED ? a.s_gate_up + tu * nkb * 32 + 2 * r + g / 2 : a.s_gate_up + rowu * (H / 64) + g / 2;
  const int qstep = TILED ? 1024 : 64;  // bytes per 128-k block
  const int sstep = TILED ? 32 : 2;     // floats per 128-k block
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < H; kb += 128 * NB) {
    u32x4_t cg[NB], cu[NB], xb[NB][4];
    float scg[NB], scu[NB];
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const int k0 = kb + 128 * h;
      cg[h] = ld16_stream(qg + (size_t)(k0 / 128) * qstep);
      cu[h] = ld16_stream(qu + (size_t)(k0 / 128) * qstep);
      scg[h] = sg[(k0 / 128) * sstep];
      scu[h] = su[(k0 / 128) * sstep];
#pragma unroll
      for (int st = 0; st < 4; ++st) xb[h][st] = rv ? ld16(xr + k0 + 8 * st) : zero;
    }
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        accg = mfma16(dequant8(cg[h][st], scg[h], s_cb), xb[h][st], accg);
        accu = mfma16(dequant8(cu[h][st], scu[h], s_cb), xb[h][st], accu);
      }
  }
  if (rv) {
    float hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = silu(accg[q]) * accu[q];
    u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + r) * I + n0 + 4 * g) = pk;
  }
}

template <bool TILED>
__global__ __launch_bounds__(kThreads) void down_nf4(ExpertArgs a) {
  __shared__ float s_cb[16];
  const int ctile = a.H / 128;
  const int item = blockIdx.x / ctile, ct = blockIdx.x - item * ctile;
  Item it;
  if (!load_item(a, item, it)) return;
  if (threadIdx.x < 16) s_cb[threadIdx.x] = a.codebook[threadIdx.x];
  __syncthreads();
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  const bool rv = r < it.M;
  const uint16_t* hr = a.h + (size_t)(it.base + (rv ? r : 0)) * I + 32 * g;
  const int nkb = I / 128;
  const size_t row0 = (size_t)it.e * H + c0 + r;
  const size_t row1 = row0 + 16;
  const size_t t0 = (size_t)it.e * (H / 16) + c0 / 16, t1 = t0 + 1;  // row tiles
  const uint8_t* q0 = TILED ? a.q_down + (t0 * nkb * 64 + lane) * 16 : a.q_down + row0 * (I / 2) + 16 * g;
  const uint8_t* q1 = TILED ? a.q_down + (t1 * nkb * 64 + lane) * 16 : a.q_down + row1 * (I / 2) + 16 * g;
  const float* s0 = TILED ? a.s_down + t0 * nkb * 32 + 2 * r + g / 2 : a.s_down + row0 * (I / 64) + g / 2;
  const float* s1 = TILED ? a.s_down + t1 * nkb * 32 + 2 * r + g / 2 : a.s_down + row1 * (I / 64) + g / 2;
  const int qstep = TILED ? 1024 : 64;
  const int sstep = TILED ? 32 : 2;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < I; kb += 128) {
    const u32x4_t c0v = ld16_stream(q0 + (size_t)(kb / 128) * qstep);
    const u32x4_t c1v = ld16_stream(q1 + (size_t)(kb / 128) * qstep);
    const float sc0 = s0[(kb / 128) * sstep], sc1 = s1[(kb / 128) * sstep];
    u32x4_t hb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) hb[st] = rv ? ld16(hr + kb + 8 * st) : zero;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      acc0 = mfma16(dequant8(c0v[st], sc0, s_cb), hb[st], acc0);
      acc1 = mfma16(dequant8(c1v[st], sc1, s_cb), hb[st], acc1);
    }
  }
  if (rv) {
    const int slot = a.perm[it.base + r];
    float* yrow = a.y + (size_t)slot * H;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 4 * g) = acc0;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 16 + 4 * g) = acc1;
  }
}

template <typename F8, typename F4>
hipError_t launch_u(int K, F8 f8, F4 f4, dim3 grid, hipStream_t s, const ExpertArgs& a, int threads = kThreads) {
  if (K % 256 == 0)
    hipLaunchKernelGGL(f8, grid, dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL(f4, grid, dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  const dim3 grid(a.max_items * (a.I / 64));
  if (nf4)
    return tiled ? launch_u(a.H, gate_up_nf4<2, true>, gate_up_nf4<1, true>, grid, s, a)
                 : launch_u(a.H, gate_up_nf4<2, false>, gate_up_nf4<1, false>, grid, s, a);
  const dim3 gw(grid.x * kSub);
  return tiled ? launch_u(a.H, gate_up_bf16<8, true>, gate_up_bf16<4, true>, gw, s, a, 64)
               : launch_u(a.H, gate_up_bf16<8, false>, gate_up_bf16<4, false>, gw, s, a, 64);
}

hipError_t launch_down(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  const dim3 grid(a.max_items * (a.H / 128));
  if (nf4) {
    if (tiled)
      hipLaunchKernelGGL(down_nf4<true>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(down_nf4<false>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 gw(grid.x * kSub);
  return tiled ? launch_u(a.I, down_bf16<8, true>, down_bf16<4, true>, gw, s, a, 64)
               : launch_u(a.I, down_bf16<8, false>, down_bf16<4, false>, gw, s, a, 64);
}

}  // namespace moe
