// Grouped 4-bit expert GEMMs for large per-expert row counts (prefill-sized
// T): the LDS-tiled MFMA form of the 4-bit kernels.
//
// Work item = (expert e, up to kQBM of its routed rows) x one tile of weight
// rows (gate/up: 64 gate rows + the matching 64 up rows, i.e. 64 columns of
// h; down: 128 output columns).  A 512-thread workgroup computes the item's
// kQBM tokens against its 128 weight rows; wave (wm, wn) owns 64 tokens (4
// token tiles) x 32 weight rows (2 row tiles: gate/up one gate and the
// matching up tile, down two adjacent tiles), so every decoded weight
// fragment feeds four MFMA tiles, where the 16-row kernels use it for one.
//
// Tokens (x rows gathered by perm for gate/up, h rows for down) move global
// -> LDS with global_load_lds_dwordx4 in 64-k stages (two 32-k fragments per
// 16-row tile, fetched row by row; a kQRing-stage ring keeps kQRing - 1
// stages of loads ahead), as in the bf16 LDS-tiled kernels.  Weights stay
// 4-bit until a lane needs
// them: each wave loads the 16-byte code chunk and the two absmax values of
// its row in each of its row tiles at the start of each 128-k block (the two
// token-half waves of a tile share them through L2; loading them a block
// ahead cost more in registers, and so occupancy, than it saved) and turns
// the codes of each 32-k step into the hi and lo bf16 parts of their
// codebook entries with the code-pair table in LDS.
//
// Arithmetic: the tokens are the MFMA A operand and the weights the B
// operand, the lanes' k assignment and the order of the steps are those of
// the 16-row 4-bit kernels, and per 64-k absmax block h of a 128-k block
//   p = x0*lo0 + x1*lo1 + x0*hi0 + x1*hi1 (one MFMA chain from 0),
//   acc = fma(absmax_h, p, acc)  (h = 0, then 1),
// which is their fmaf(s1, p1, fmaf(s0, p0, acc)) taken one block at a time:
// every output element gets the same bits whichever kernel computes it.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "nf4.hpp"

namespace moe {
namespace {

constexpr int kQBM = kMfmaTile;                         // token rows of an item
constexpr int kQWaves = 8;
constexpr int kQThreads = 64 * kQWaves;
constexpr int kQWM = kQBM / 64;                         // waves along the tokens (64 rows each)
constexpr int kQWN = kQWaves / kQWM;                    // waves along the weight rows (32 each)
constexpr int kQFrag = 1024;                            // one 16 x 32 bf16 token fragment
constexpr int kQXFrags = kQBM / 16 * 2;                 // token fragments per 64-k stage
constexpr int kQStageBytes = kQXFrags * kQFrag;
constexpr int kQRing = 3;                               // LDS stages in the ring
constexpr int kQLutOff = kQRing * kQStageBytes;         // the code-pair table follows the ring
constexpr int kQLdsBytes = kQLutOff + 256 * kLutRep * 8;
constexpr int kQLoads = kQXFrags / kQWaves;             // token fragment loads per wave per stage
static_assert(kQBM == 128 && kQWN == 4 && kQLoads == 2, "tile split");
static_assert(kQLdsBytes <= 80 * 1024, "two workgroups per CU");

typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
#define MOE_Q_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// Workgroup barrier without __syncthreads' release fence (which would wait
// for every LDS-DMA load in flight, later stages included); the wave's own
// LDS reads are complete first.
__device__ __forceinline__ void q_stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Blocks are dealt round-robin over the 8 XCDs; hand each XCD a contiguous
// range of logical tiles.
__device__ __forceinline__ int q_xcd_remap(int b, int nb) {
  const int per = (nb + 7) / 8;
  const int x = b & 7, i = b >> 3;
  const int full = nb - (per - 1) * 8;
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

// the MFMAs of one 64-k stage (absmax block h of 128-k block cd / sc) for
// the wave's first NJ token tiles
template <int NJ, int HB>
__device__ __forceinline__ void q_stage_mma(const unsigned char* sb, const u32x2_t* sl, const u32x4_t (&cd)[2],
                                            const u32x2_t (&sc)[2], int wm, int xoff, f32x4_t (&acc)[2][4]) {
  u32x4_t hi[2][2], lo[2][2];  // [tile][32-k step]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lut8(sl, cd[i][2 * HB], hi[i][0], lo[i][0]);
    lut8(sl, cd[i][2 * HB + 1], hi[i][1], lo[i][1]);
  }
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4_t x[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      x[ks] = *reinterpret_cast<const u32x4_t*>(sb + (((wm * 4 + j) * 2 + ks) * kQFrag) + xoff);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float s = __uint_as_float(sc[i][HB]);
      f32x4_t p = mfma16(x[0], lo[i][0], zero);
      p = mfma16(x[1], lo[i][1], p);
      p = mfma16(x[0], hi[i][0], p);
      p = mfma16(x[1], hi[i][1], p);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(s, p[q], acc[i][j][q]);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next token tile's reads stay below (register pressure)
  }
}

// four waves per SIMD: two workgroups share a CU
template <bool GATE_UP, bool LORA>
__global__ __launch_bounds__(kQThreads, 4) void expert_mfma_nf4(ExpertArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_raw[];
  const int H = a.H, I = a.I;
  const int ntile = GATE_UP ? I / 64 : H / 128;
  const int nblk = *a.n_items * ntile;
  if ((int)blockIdx.x >= nblk) return;
  u32x2_t* s_lut = reinterpret_cast<u32x2_t*>(s_raw + kQLutOff);
  build_lut(s_lut, a.codebook, threadIdx.x);
  const int lb = q_xcd_remap(blockIdx.x, nblk);
  // the expert's items are contiguous in the work list (its item i starts at
  // row i * kQBM); inside the expert: weight tile nt major, item minor
  const int coarse = lb / ntile;
  const int e = a.items[2 * coarse];
  const int first = coarse - a.items[2 * coarse + 1] / kQBM;
  const int cnt = a.counts[e];
  const int ne = (cnt + kQBM - 1) / kQBM;
  const int local = lb - first * ntile;
  const int nt = local / ne;
  const int m0 = (local - nt * ne) * kQBM;
  const int M = min(cnt - m0, kQBM);
  const int base = a.offsets[e] + m0;
  const int K = GATE_UP ? H : I;
  const int nkb = K / 128;
  const int nstage = K / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  // ---- token loads: wave w brings row tile w, both 32-k halves of a stage,
  // row by row (lane 4p + c: row p, k chunk xchunk(p, c) of each half); a
  // wave whose rows all lie past the item's end loads none
  const bool xload = wave * 16 < M;
  const uint16_t* xsrc;
  {
    int row = wave * 16 + (lane >> 2);
    row = row < M ? row : M - 1;  // rows past M repeat a valid row; their outputs are never stored
    const size_t srow = GATE_UP ? (size_t)(a.perm[base + row] / a.k) : (size_t)(base + row);
    xsrc = (GATE_UP ? a.x : a.h) + srow * K + xchunk(lane >> 2, lane & 3) * 8;
  }
  const int xoff = xslot(lane) * 16;  // this lane's operand in a token fragment
  auto issue = [&](int st, int buf) {
    if (!xload) return;
    lds_char* sb = (lds_char*)(s_raw) + buf * kQStageBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      __builtin_amdgcn_global_load_lds(xsrc + st * 64 + ks * 32, sb + (wave * 2 + ks) * kQFrag, 16, 0, 0);
  };

  // ---- this wave's weight row tiles: codes and absmax of row r, per 128-k block
  const int wm = wave % kQWM, wn = wave / kQWM;
  // first weight row of tile i (gate/up: the gate tile, then the matching up tile)
  auto row0_of = [&](int i) -> size_t {
    return GATE_UP ? (size_t)e * 2 * I + (i ? I : 0) + nt * 64 + wn * 16 : (size_t)e * H + nt * 128 + wn * 32 + 16 * i;
  };
  const uint8_t* qp[2];
  const float* sp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const size_t rt = row0_of(i) / 16;
    qp[i] = (GATE_UP ? a.q_gate_up : a.q_down) + (rt * nkb * 64 + lane) * 16;
    sp[i] = (GATE_UP ? a.s_gate_up : a.s_down) + rt * nkb * 32 + 2 * r;
  }
  u32x4_t cd[2];
  u32x2_t sc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cd[i] = ld16_stream(qp[i]);
    sc[i] = *reinterpret_cast<const u32x2_t*>(sp[i]);
  }

  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the wave's 16-row token tiles that hold rows of the item (0..4); the
  // MFMAs of tiles wholly past the item's end are skipped
  const int nj = min(max((M - wm * 64 + 15) / 16, 0), 4);
  const u32x2_t* sl = lut_copy(s_lut, lane);

  constexpr int D = kQRing - 1;  // stages in flight ahead of the one multiplied
#pragma unroll
  for (int st = 0; st < D; ++st)
    if (st < nstage) issue(st, st);
  q_stage_barrier();  // the table is built (the first stages' loads stay in flight)
  // one 64-k stage: stage st landed (the wave's loads younger than its
  // stage-st copies are the copies of stage st + 1 and, at a block's second
  // stage, the block's codes, loaded after those copies and already waited
  // for by the first stage's MFMAs: waiting until at most kQLoads loads are
  // in flight covers stage st), a
  // barrier for every wave (buffer (st + D) % kQRing is then free), at the
  // block's first stage its codes and absmax, the copies of stage st + D,
  // and the MFMAs of absmax block HB
  auto stage = [&](auto njc, auto hbc, int kb) {
    constexpr int NJ = decltype(njc)::value, HB = decltype(hbc)::value;
    const int st = 2 * kb + HB;
    if (xload && st + 1 < nstage)
      __builtin_amdgcn_s_waitcnt(MOE_Q_VMCNT(kQLoads));
    else
      __builtin_amdgcn_s_waitcnt(MOE_Q_VMCNT(0));
    q_stage_barrier();
    if (HB == 0 && kb > 0) {  // this block's codes and absmax (block 0's were loaded up front)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        cd[i] = ld16_stream(qp[i] + (size_t)kb * 1024);
        sc[i] = *reinterpret_cast<const u32x2_t*>(sp[i] + (size_t)kb * 32);
      }
    }
    if (st + D < nstage) issue(st + D, (st + D) % kQRing);
    if constexpr (NJ > 0) q_stage_mma<NJ, HB>(s_raw + (st % kQRing) * kQStageBytes, sl, cd, sc, wm, xoff, acc);
  };
  auto k_loop = [&](auto njc) {
    for (int kb = 0; kb < nkb; ++kb) {
      stage(njc, std::integral_constant<int, 0>{}, kb);
      stage(njc, std::integral_constant<int, 1>{}, kb);
    }
  };
  switch (nj) {
    case 4: k_loop(std::integral_constant<int, 4>{}); break;
    case 3: k_loop(std::integral_constant<int, 3>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    default: k_loop(std::integral_constant<int, 0>{}); break;
  }

  // ---- epilogue: lane (r, g) holds tokens 4g + q of token tile j for its
  // weight row r of tile i
  if constexpr (LORA) {  // before any accumulator is used; every lane takes part in the MFMAs
    const float* ub = GATE_UP ? a.u_gate_up : a.u_down;
    const float* lbp = GATE_UP ? a.lb_gate_up : a.lb_down;
    f32x4_t bq[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) bq[i] = ld4f(lbp + (row0_of(i) + r) * 16 + 4 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = (wm * 4 + j) * 16 + r;
      const f32x4_t uq = trow < M ? ld4f(ub + (size_t)(base + trow) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 2; ++i) add_scaled(acc[i][j], lora_tile(uq, bq[i]), a.lora_scale);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = (wm * 4 + j) * 16 + 4 * g + q;  // token row of the item
      if (m < M) {
        if (GATE_UP) {
          const int n = nt * 64 + wn * 16 + r;
          if (a.gu) {  // training forward: keep the pre-activations the nonlinearity sees
            float* gp = a.gu + (size_t)(base + m) * 2 * I + n;
            gp[0] = acc[0][j][q];
            gp[I] = acc[1][j][q];
          }
          const float hv = silu(acc[0][j][q]) * acc[1][j][q];
          a.h[(size_t)(base + m) * I + n] = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xffffu);
        } else {
          float* yrow = a.y + (size_t)a.perm[base + m] * H + nt * 128 + wn * 32 + r;
          yrow[0] = acc[0][j][q];
          yrow[16] = acc[1][j][q];
        }
      }
    }
  }
}

// dynamic LDS beyond 64 KiB needs the per-function limit raised, once per device
template <bool GATE_UP, bool LORA>
hipError_t allow_lds_nf4() {
  static bool done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&expert_mfma_nf4<GATE_UP, LORA>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kQLdsBytes);
  if (e == hipSuccess) done[dev] = true;
  return e;
}

template <bool GATE_UP, bool LORA>
hipError_t launch_mfma_nf4_t(const ExpertArgs& a, hipStream_t s) {
  hipError_t e = allow_lds_nf4<GATE_UP, LORA>();
  if (e != hipSuccess) return e;
  const dim3 grid(a.max_items * (GATE_UP ? a.I / 64 : a.H / 128));
  hipLaunchKernelGGL((expert_mfma_nf4<GATE_UP, LORA>), grid, dim3(kQThreads), kQLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_mfma_nf4(const ExpertArgs& a, hipStream_t s) {
  return a.lora ? launch_mfma_nf4_t<true, true>(a, s) : launch_mfma_nf4_t<true, false>(a, s);
}

hipError_t launch_down_mfma_nf4(const ExpertArgs& a, hipStream_t s) {
  return a.lora ? launch_mfma_nf4_t<false, true>(a, s) : launch_mfma_nf4_t<false, false>(a, s);
}

}  // namespace moe
