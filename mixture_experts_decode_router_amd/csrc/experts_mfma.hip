// Grouped expert GEMMs for large per-expert row counts (prefill-sized T):
// LDS-tiled MFMA with the operands copied global -> LDS by the load unit.
//
// Work item = (expert e, up to kBM of its routed rows) x one tile of 256
// weight rows (gate/up: 128 gate rows + the matching 128 up rows; down: 256
// rows of W_down).  A 512-thread workgroup computes the kBM x 256 output
// tile; each of its 8 waves owns 64 tokens x (16 kNT) weight rows as kNT x 4
// MFMA 16x16x32 tiles.  A wave whose 64 rows all lie past the item's last row
// skips its MFMAs, and so does a wave's 16-row token tile that lies wholly
// past it, so a short item costs its weight stream, not its padding.
//
// Per 32-k stage the workgroup needs 16 weight fragments (each one contiguous
// kilobyte of the tiled layout) and kBM/16 token fragments (16 gathered rows
// x 32 k); the waves move them with global_load_lds_dwordx4, which writes the
// 64 lanes' 16-byte pieces to LDS in lane order, so no register staging is
// needed.  A weight fragment arrives in MFMA operand order.  A token
// fragment is fetched row by row (lanes 4p .. 4p+3 bring the 64 bytes of
// row p, in the order of xchunk): the load unit serves four lanes that read
// one contiguous row segment about twice as fast as sixteen lanes that each
// read another row, which the operand order would need (moe_probe_gather
// over 16 MiB of 4 KiB rows: 20 against 9.7 TB/s).  The MFMA lanes then
// read their 16 bytes from slot 4r + xchunk(r, g), an order in which every
// 8 consecutive lanes of a read hit distinct banks.  kRing LDS stages form a
// ring: loads run kRing - 1 stages ahead of the MFMAs.  Each iteration waits for the wave's
// own loads of the stage to be multiplied (s_waitcnt vmcnt), then one barrier
// publishes the whole stage and retires the buffer the next loads overwrite.
//
// Block order: the tiles of one expert are consecutive, weight tile major and
// item minor, so all the items of a heavily routed expert stream each weight
// tile through L2 together (the gathered tokens are small and stay in the
// last-level cache); consecutive ranges go to one XCD.
//
// The MFMA instruction, the k assignment of lanes (lane group g <-> k offset
// 8g of each 32-k step) and the order of the k-steps are the same as in the
// skinny kernels, so every output element is the bit-identical result
// whichever kernel computes it: a token's output does not depend on the batch
// size that selected the kernel.
//
//   gate/up:  h[p][n] = silu(gate) * up -> bf16 (sorted-slot order); a
//             training forward also keeps gate and up (fp32) for the backward
//   down:     y[perm[p]][c] (fp32, flat-slot order)
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

#ifndef MOE_MFMA_RING
#define MOE_MFMA_RING 3
#endif
constexpr int kBM = kMfmaTile;                        // token rows of an item
#ifndef MOE_MFMA_BN
#define MOE_MFMA_BN 256
#endif
constexpr int kBN = MOE_MFMA_BN;                      // weight rows of a tile
#ifndef MOE_MFMA_WAVES
#define MOE_MFMA_WAVES 8
#endif
constexpr int kWaves = MOE_MFMA_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kWM = kBM / 64;                         // waves along the tokens (64 rows each)
constexpr int kWN = kWaves / kWM;                     // waves along the weight rows
constexpr int kNT = kBN / 16 / kWN;                   // weight row tiles per wave
constexpr int kFragBytes = 1024;                      // one 16 x 32 bf16 operand fragment
constexpr int kWFrags = kBN / 16;                     // weight fragments per stage
constexpr int kXFrags = kBM / 16;                     // token fragments per stage
constexpr int kXBase = kWFrags * kFragBytes;          // token fragments follow the weights
constexpr int kStageBytes = (kWFrags + kXFrags) * kFragBytes;
constexpr int kRing = MOE_MFMA_RING;                  // LDS stages in the ring
constexpr int kLdsBytes = kRing * kStageBytes;
constexpr int kWLoads = kWFrags / kWaves;             // weight fragment loads per wave per stage
constexpr int kXTiles = kXFrags / kWaves;             // token fragment loads per wave per stage
constexpr int kLoads = kWLoads + kXTiles;
constexpr int kHalfT = kWFrags / 2;                   // gate/up: gate row tiles of a weight tile
constexpr int kBlocksPerCU = 3 * kLdsBytes <= 160 * 1024 ? 3 : (2 * kLdsBytes <= 160 * 1024 ? 2 : 1);
static_assert((kBM == 128 || kBM == 256) && kWFrags % kWaves == 0 && kXFrags % kWaves == 0, "tile split");
static_assert(kNT % 2 == 0 && kNT <= 8, "gate/up pairs per wave");
static_assert(kLdsBytes <= 160 * 1024, "LDS");

typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
#define MOE_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// wait until at most `later` stages of this wave's loads are still in flight;
// nl = the wave's loads per stage (kLoads, or kLoads - kXTiles when its token
// tiles lie past the item's end and are not loaded)
template <int NL>
__device__ __forceinline__ void wait_loads_n(int later) {
  if (later <= 0) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(0));
  else if (later == 1) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(NL));
  else if (later == 2) __builtin_amdgcn_s_waitcnt(MOE_VMCNT(2 * NL));
  else __builtin_amdgcn_s_waitcnt(MOE_VMCNT(3 * NL));
}
__device__ __forceinline__ void wait_own_loads(int later, bool tokens) {
  if (tokens) wait_loads_n<kLoads>(later);
  else wait_loads_n<kLoads - kXTiles>(later);
}
static_assert(kRing <= 5 && 3 * kLoads < 64, "wait_own_loads covers up to three later stages");

// Workgroup barrier without __syncthreads' release fence, which would make
// every wave wait for all its LDS-DMA loads, including those of later stages.
// The wave's own LDS reads are complete first (lgkmcnt(0)), so no buffer is
// overwritten while a read of it is in flight; "memory" keeps the compiler
// from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Blocks are dealt round-robin over the 8 XCDs; hand each XCD a contiguous
// range of logical tiles.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = (nb + 7) / 8;
  const int x = b & 7, i = b >> 3;
  const int full = nb - (per - 1) * 8;  // XCDs that get `per` blocks
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

// MFMAs of one k-step for the first NJ token tiles of the wave; xoff: this
// lane's byte offset in a token fragment (xslot)
template <int NJ>
__device__ __forceinline__ void mma_step(const unsigned char* sb, const int (&wrt)[kNT], int wm, int lane, int xoff,
                                         f32x4_t (&acc)[kNT][4]) {
  u32x4_t af[kNT], bf[NJ];
#pragma unroll
  for (int i = 0; i < kNT; ++i) af[i] = *reinterpret_cast<const u32x4_t*>(sb + wrt[i] * kFragBytes + lane * 16);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    bf[j] = *reinterpret_cast<const u32x4_t*>(sb + kXBase + (wm * 4 + j) * kFragBytes + xoff);
#pragma unroll
  for (int i = 0; i < kNT; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
}

// kWaves / 4 waves per SIMD per workgroup; kBlocksPerCU workgroups share a CU.
// LORA: the epilogue adds scale * sum_j B[e][row][j] U[p][j] to each fp32
// accumulator before anything else uses it (lora_tile, as the 16-row kernels).
template <bool GATE_UP, bool LORA>
__global__ __launch_bounds__(kThreads, kWaves / 4 * kBlocksPerCU) void expert_mfma(ExpertArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_raw[];
  const int H = a.H, I = a.I;
  const int ntile = GATE_UP ? I / (kBN / 2) : (H + kBN - 1) / kBN;
  // the grid is sized for the longest possible work list; the real tiles are
  // the first n_items * ntile blocks, spread evenly over the XCDs
  const int nblk = *a.n_items * ntile;
  if ((int)blockIdx.x >= nblk) return;
  const int lb = xcd_remap(blockIdx.x, nblk);
  // the expert's items are contiguous in the work list (its item i starts at
  // row i * kBM); inside the expert: weight tile nt major, item minor
  const int coarse = lb / ntile;
  const int e = a.items[2 * coarse];
  const int first = coarse - a.items[2 * coarse + 1] / kBM;
  const int cnt = a.counts[e];
  const int ne = (cnt + kBM - 1) / kBM;
  const int local = lb - first * ntile;
  const int nt = local / ne;
  const int m0 = (local - nt * ne) * kBM;
  const int M = min(cnt - m0, kBM);
  const int base = a.offsets[e] + m0;
  const int K = GATE_UP ? H : I;
  const int nks = K / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- this wave's loads per stage: weight row tiles kWLoads*wave + i, token tiles kXTiles*wave + t
  const uint16_t* wsrc[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int rtl = kWLoads * wave + i;  // local row tile
    size_t rt;
    if (GATE_UP) {
      const int rloc = rtl < kHalfT ? nt * kHalfT + rtl : I / 16 + nt * kHalfT + (rtl - kHalfT);
      rt = (size_t)e * (2 * I / 16) + rloc;
    } else {
      const int rloc = min(nt * kWFrags + rtl, H / 16 - 1);  // rows past H: any valid tile, never stored
      rt = (size_t)e * (H / 16) + rloc;
    }
    wsrc[i] = (GATE_UP ? a.w_gate_up : a.w_down) + ((rt * nks) * 64 + lane) * 8;
  }
  // lane 4p + c brings row 16 tt + p, k offset 8 xchunk(p, c) of each
  // k-step; a wave whose token tiles all lie past the item's end loads none
  // (their MFMAs are skipped too)
  const bool xload = kXTiles * wave * 16 < M;
  const uint16_t* xsrc[kXTiles];
#pragma unroll
  for (int t = 0; t < kXTiles; ++t) {
    int row = (kXTiles * wave + t) * 16 + (lane >> 2);
    row = row < M ? row : M - 1;  // rows past M repeat a valid row; their outputs are never stored
    const size_t srow = GATE_UP ? (size_t)(a.perm[base + row] / a.k) : (size_t)(base + row);
    xsrc[t] = (GATE_UP ? a.x : a.h) + srow * K + xchunk(lane >> 2, lane & 3) * 8;
  }

  auto issue = [&](int kb, int buf) {
    lds_char* sb = (lds_char*)(s_raw) + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      __builtin_amdgcn_global_load_lds(wsrc[i] + (size_t)kb * 512, sb + (kWLoads * wave + i) * kFragBytes, 16, 0, 0);
    if (xload) {
#pragma unroll
      for (int t = 0; t < kXTiles; ++t)
        __builtin_amdgcn_global_load_lds(xsrc[t] + kb * 32, sb + kXBase + (kXTiles * wave + t) * kFragBytes, 16, 0,
                                         0);
    }
  };

  // ---- compute: wave (wm, wn) = 64 tokens x 16*kNT weight rows
  const int wm = wave % kWM, wn = wave / kWM;
  constexpr int kH = kNT / 2;
  int wrt[kNT];  // local weight row tiles of this wave (gate/up: kH gate tiles, then the matching up tiles)
#pragma unroll
  for (int i = 0; i < kNT; ++i) wrt[i] = GATE_UP ? (i < kH ? wn * kH + i : kHalfT + wn * kH + (i - kH)) : wn * kNT + i;
  f32x4_t acc[kNT][4];
#pragma unroll
  for (int i = 0; i < kNT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the wave's 16-row token tiles that hold rows of the item (0..4); the
  // MFMAs of tiles wholly past the item's end are skipped
  const int nj = min(max((M - wm * 64 + 15) / 16, 0), 4);
  const int xoff = xslot(lane) * 16;

  const int nstage = nks;  // one 32-k step per stage
  constexpr int D = kRing - 1;  // stages in flight ahead of the one multiplied
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (st < nstage) issue(st, st);
  // the k loop; a wave with no live rows still moves its share of every stage
  auto k_loop = [&](auto njc) {
    constexpr int NJ = decltype(njc)::value;
    for (int kb = 0; kb < nstage; ++kb) {
      wait_own_loads(min(D - 1, nstage - 1 - kb), xload);  // stage kb landed (later ones may be in flight)
      stage_barrier();                              // ... for every wave; buffer (kb+D)%kRing is free
      if (kb + D < nstage) issue(kb + D, (kb + D) % kRing);
      if constexpr (NJ > 0) mma_step<NJ>(s_raw + (kb % kRing) * kStageBytes, wrt, wm, lane, xoff, acc);
    }
  };
  switch (nj) {
    case 4: k_loop(std::integral_constant<int, 4>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    default: k_loop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue: lane (r, g) holds weight rows 4g+q of tile i, token row r of token tile j
  const int r = lane & 15, g = lane >> 4;
  if constexpr (LORA) {  // before any accumulator is used; every lane takes part in the MFMAs
    const float* ub = GATE_UP ? a.u_gate_up : a.u_down;
    f32x4_t uq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = (wm * 4 + j) * 16 + r;
      uq[j] = trow < M ? ld4f(ub + (size_t)(base + trow) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kNT; ++i) {
      size_t brow;  // the adapter row of this lane's weight row in tile i
      if (GATE_UP) {
        const int n = nt * (kBN / 2) + (wn * kH + (i % kH)) * 16 + r;
        brow = (size_t)e * 2 * I + (i < kH ? n : I + n);
      } else {
        brow = (size_t)e * H + min(nt * kBN + (wn * kNT + i) * 16 + r, H - 1);  // rows past H are never stored
      }
      const f32x4_t bq = ld4f((GATE_UP ? a.lb_gate_up : a.lb_down) + brow * 16 + 4 * g);
      // each sum is formed here, one tile at a time (the empty asm keeps the
      // compiler from sinking the adds into the stores below, which would
      // hold every rank-16 tile beside the accumulators)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        add_scaled(acc[i][j], lora_tile(bq, uq[j]), a.lora_scale);
        asm volatile("" : "+v"(acc[i][j]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (GATE_UP) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = (wm * 4 + j) * 16 + r;
      if (trow < M) {
#pragma unroll
        for (int i = 0; i < kH; ++i) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu(acc[i][j][q]) * acc[i + kH][j][q];
          const int n = nt * (kBN / 2) + (wn * kH + i) * 16 + 4 * g;
          if (a.gu) {  // training forward: keep the pre-activations the nonlinearity sees
            float* gp = a.gu + (size_t)(base + trow) * 2 * I + n;
            *reinterpret_cast<f32x4_t*>(gp) = acc[i][j];
            *reinterpret_cast<f32x4_t*>(gp + I) = acc[i + kH][j];
          }
          u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          *reinterpret_cast<u32x2_t*>(a.h + (size_t)(base + trow) * I + n) = pk;
        }
      }
    }
  } else {
    // y rows leave row by row: lane L = 4p + c takes over the four columns
    // 4c .. 4c+3 of token row p from lane 16c + p (a lane permutation), so
    // four consecutive lanes store one 64-byte segment of a row; stored with
    // one row per lane, as the accumulators lie, the y writes cost the down
    // GEMM about a third of its time at T = 4096
    const int p = lane >> 2, cq = lane & 3;
    const int src = (16 * cq + p) * 4;  // byte address of the source lane
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = (wm * 4 + j) * 16 + p;
      f32x4_t v[kNT];
#pragma unroll
      for (int i = 0; i < kNT; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[i][q] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(acc[i][j][q])));
      if (trow < M) {
        float* yrow = a.y + (size_t)a.perm[base + trow] * H;
#pragma unroll
        for (int i = 0; i < kNT; ++i) {
          const int c = nt * kBN + (wn * kNT + i) * 16 + 4 * cq;
          if (c < H) *reinterpret_cast<f32x4_t*>(yrow + c) = v[i];
        }
      }
    }
  }
}

// dynamic LDS beyond 64 KiB needs the per-function limit raised, once per device
template <bool GATE_UP, bool LORA>
hipError_t allow_lds() {
  static bool done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_mfma<GATE_UP, LORA>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e == hipSuccess) done[dev] = true;
  return e;
}

template <bool GATE_UP, bool LORA>
hipError_t launch_mfma_t(const ExpertArgs& a, hipStream_t s) {
  hipError_t e = allow_lds<GATE_UP, LORA>();
  if (e != hipSuccess) return e;
  const dim3 grid(a.max_items * (GATE_UP ? a.I / (kBN / 2) : (a.H + kBN - 1) / kBN));
  hipLaunchKernelGGL((expert_mfma<GATE_UP, LORA>), grid, dim3(kThreads), kLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mfma(const ExpertArgs& a, hipStream_t s) {
  return a.lora ? launch_mfma_t<true, true>(a, s) : launch_mfma_t<true, false>(a, s);
}

hipError_t launch_down_mfma(const ExpertArgs& a, hipStream_t s) {
  return a.lora ? launch_mfma_t<false, true>(a, s) : launch_mfma_t<false, false>(a, s);
}

}  // namespace moe
