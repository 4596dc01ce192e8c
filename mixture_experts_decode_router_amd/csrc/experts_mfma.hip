// Grouped expert GEMMs for large per-expert row counts (prefill-sized T):
// LDS double-buffered MFMA tiles.
//
// Work item = (expert e, up to 128 of its routed rows) x one 128-wide tile of
// weight rows; a 256-thread workgroup computes the 128 x 128 output tile,
// each of its 2 x 2 waves a 64 x 64 quarter as 4 x 4 MFMA 16x16x32 tiles.
// Per 64-k step the workgroup copies its 128 x 64 weight slab (16 fragments
// of the tiled layout, each one contiguous kilobyte) and its 128 x 64 token
// slab (gathered rows) into LDS in fragment order, so every ds_read_b128 of a
// wave reads one kilobyte (token fragments with a row swizzle that keeps the
// stores free of bank conflicts).  Global loads run two stages ahead of the
// MFMAs (two register slots, two LDS buffers).
//
// The MFMA instruction, the k assignment of lanes (lane group g <-> k offset
// 8g of each 32-k step) and the order of the k-steps are the same as in the
// skinny kernels, so every output element is the bit-identical result
// whichever kernel computes it: a token's output does not depend on the batch
// size that selected the kernel.
//
//   gate/up:  tile = 64 gate rows + the matching 64 up rows; epilogue
//             h = silu(gate) * up -> bf16 h[p][n]
//   down:     tile = 128 rows of W_down; epilogue y[perm[p]][c] (fp32)
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBM = 128;           // rows of an item (tokens)
constexpr int kBK = 64;            // k per LDS stage (two MFMA k-steps)
constexpr int kThreads = 256;
constexpr int kFragBytes = 1024;   // one 16 x 32 bf16 MFMA operand fragment
constexpr int kStageBytes = 2 * 16 * kFragBytes;  // weights 16 KiB + tokens 16 KiB

struct Item {
  int e, M, base;
};

__device__ __forceinline__ bool load_item(const ExpertArgs& a, int item, Item& it) {
  if (item >= *a.n_items) return false;
  it.e = a.items[2 * item];
  const int m0 = a.items[2 * item + 1];
  const int c = a.counts[it.e] - m0;
  it.M = c < kBM ? c : kBM;
  it.base = a.offsets[it.e] + m0;
  return it.M > 0;  // group padding items are empty
}

// Blocks are dealt round-robin over the 8 XCDs; hand each XCD a contiguous
// range of logical tiles (expert-major) so tiles sharing weights meet in one
// L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = (nb + 7) / 8;
  const int x = b & 7, i = b >> 3;
  const int full = nb - (per - 1) * 8;  // XCDs that get `per` blocks
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

// One stage: weights (16 fragments) then tokens (16 fragments) in LDS.
// Weight fragment (rtl, ks) at rtl*2 + ks; token fragment (tt, ks) at 16 + tt*2 + ks.
template <bool GATE_UP>
__global__ __launch_bounds__(kThreads) void expert_mfma(ExpertArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_raw[];
  const int ntile = GATE_UP ? a.I / 64 : a.H / 128;
  // the grid is sized for the longest possible work list; the real tiles are
  // the first n_items * ntile blocks, spread evenly over the XCDs
  const int nblk = *a.n_items * ntile;
  if ((int)blockIdx.x >= nblk) return;
  const int lb = xcd_remap(blockIdx.x, nblk);
  // logical order: groups of kMfmaGroup items (one expert), inside a group
  // column tile nt major and the group's items minor
  const int gsz = kMfmaGroup * ntile;
  const int grp = lb / gsz, rem = lb - grp * gsz;
  const int nt = rem / kMfmaGroup;
  const int item = grp * kMfmaGroup + (rem - nt * kMfmaGroup);
  Item it;
  if (!load_item(a, item, it)) return;
  const int H = a.H, I = a.I;
  const int K = GATE_UP ? H : I;
  const int nks = K / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- global sources of this thread's 4 weight chunks and 4 token chunks per stage
  // weight chunk j = tid + 256 i: fragment f = j / 64 (rtl = f / 2, ks = f % 2), slot j % 64
  const uint16_t* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = tid + 256 * i;
    const int f = j >> 6, slot = j & 63;
    const int rtl = f >> 1, ks = f & 1;
    size_t rt;
    if (GATE_UP) {
      const size_t rt_gate = (size_t)it.e * (2 * I / 16) + nt * 4;  // first gate row tile of this item tile
      rt = rtl < 4 ? rt_gate + rtl : rt_gate + I / 16 + (rtl - 4);
    } else {
      rt = (size_t)it.e * (H / 16) + nt * 8 + rtl;
    }
    wsrc[i] = (GATE_UP ? a.w_gate_up : a.w_down) + ((rt * nks + ks) * 64 + slot) * 8;
  }
  // token chunk q = tid + 256 i: row = q / 8, chunk c = q % 8 (k offset 8c within the stage)
  const uint16_t* xsrc[4];
  int xdst[4];
  bool xok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    const int row = q >> 3, c = q & 7;
    xok[i] = row < it.M;
    const size_t srow = !xok[i] ? 0 : (GATE_UP ? (size_t)(a.perm[it.base + row] / a.k) : (size_t)(it.base + row));
    xsrc[i] = (GATE_UP ? a.x : a.h) + srow * K + c * 8;
    const int tt = row >> 4, r = row & 15, ks = c >> 2, g = c & 3;
    // the 8 lanes storing one row's 8 chunks must hit 8 different bank
    // groups: row r of lane group g sits at slot r ^ (4 ks + g)
    xdst[i] = (16 + tt * 2 + ks) * kFragBytes + (g * 16 + (r ^ (4 * ks + g))) * 16;
  }

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // two register slots of global loads (stage s lives in slot s & 1), so the
  // loads of stage kb + 2 are in flight while stage kb is multiplied
  u32x4_t wreg[2][4], xreg[2][4];
#define MOE_LOAD_STAGE(SLOT, KB)                                               \
  do {                                                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                            \
      wreg[SLOT][i] = ld16_stream(wsrc[i] + (size_t)(KB) * 2 * 512);           \
      xreg[SLOT][i] = xok[i] ? ld16(xsrc[i] + (KB) * kBK) : zero;              \
    }                                                                          \
  } while (0)
#define MOE_STORE_STAGE(SLOT, BUF)                                             \
  do {                                                                         \
    unsigned char* sb = s_raw + (BUF) * kStageBytes;                           \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                            \
      *reinterpret_cast<u32x4_t*>(sb + (tid + 256 * i) * 16) = wreg[SLOT][i];  \
      *reinterpret_cast<u32x4_t*>(sb + xdst[i]) = xreg[SLOT][i];               \
    }                                                                          \
  } while (0)

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // weight row tiles of this wave (rtl) and token tiles (tt)
  int wrt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wrt[i] = GATE_UP ? (i < 2 ? wn * 2 + i : 4 + wn * 2 + (i - 2)) : wn * 4 + i;

  // token fragments are stored row-swizzled (see xdst); lane (g, r) reads slot r ^ (4 ks + g)
  const int lg = lane >> 4, lr = lane & 15;
  const int bslot0 = (lg * 16 + (lr ^ lg)) * 16, bslot1 = (lg * 16 + (lr ^ (4 + lg))) * 16;
  auto compute = [&](int buf) {
    const unsigned char* base = s_raw + buf * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const u32x4_t*>(base + (wrt[i] * 2 + ks) * kFragBytes + lane * 16);
        bf[i] = *reinterpret_cast<const u32x4_t*>(base + (16 + (wm * 4 + i) * 2 + ks) * kFragBytes +
                                                   (ks ? bslot1 : bslot0));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
    }
  };

  // K / 64 stages (an even number: K is a multiple of 128)
  const int nstage = K / kBK;
  MOE_LOAD_STAGE(0, 0);
  MOE_LOAD_STAGE(1, 1);
  MOE_STORE_STAGE(0, 0);
  __syncthreads();
  for (int kb = 0; kb < nstage; kb += 2) {
    // even stage kb: LDS buffer 0, register slot 0 is free once stored
    if (kb + 2 < nstage) MOE_LOAD_STAGE(0, kb + 2);
    compute(0);
    MOE_STORE_STAGE(1, 1);  // stage kb + 1 (always exists: nstage is even)
    __syncthreads();
    // odd stage kb + 1: LDS buffer 1
    if (kb + 3 < nstage) MOE_LOAD_STAGE(1, kb + 3);
    compute(1);
    if (kb + 2 < nstage) MOE_STORE_STAGE(0, 0);
    __syncthreads();
  }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE

  // ---- epilogue: lane (r, g) holds rows 4g+q of weight tile i, token column r of token tile j
  const int r = lane & 15, g = lane >> 4;
  if (GATE_UP) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (wm * 4 + j) * 16 + r;
      if (row < it.M) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu(acc[i][j][q]) * acc[i + 2][j][q];
          const int n = nt * 64 + (wn * 2 + i) * 16 + 4 * g;
          u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + row) * I + n) = pk;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (wm * 4 + j) * 16 + r;
      if (row < it.M) {
        float* yrow = a.y + (size_t)a.perm[it.base + row] * H;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = nt * 128 + (wn * 4 + i) * 16 + 4 * g;
          *reinterpret_cast<f32x4_t*>(yrow + c) = acc[i][j];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_up_mfma(const ExpertArgs& a, hipStream_t s) {
  const dim3 grid(a.max_items * (a.I / 64));
  hipLaunchKernelGGL(expert_mfma<true>, grid, dim3(kThreads), 2 * kStageBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const ExpertArgs& a, hipStream_t s) {
  const dim3 grid(a.max_items * (a.H / 128));
  hipLaunchKernelGGL(expert_mfma<false>, grid, dim3(kThreads), 2 * kStageBytes, s, a);
  return hipGetLastError();
}

}  // namespace moe
