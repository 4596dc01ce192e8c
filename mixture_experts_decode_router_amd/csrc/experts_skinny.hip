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
// 4-bit weights (NF4_B64): the codebook value of each code (one LDS table
// read per two codes, as a hi and a lo bf16 part) feeds the MFMA unscaled;
// the per-64 absmax scales the MFMA partial sums of each 64-k half block
// (see the 4-bit section).
#include "common.hpp"
#include "kernels.hpp"
#include "nf4.hpp"

namespace moe {
namespace {

constexpr int kTile = kSkinnyTile;  // rows per item (MFMA column block)
constexpr int kThreads = 64;        // bf16 kernels: one wave per workgroup
constexpr int kNf4Threads = 256;    // 4-bit kernels: four waves share a code table

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

template <int U, bool TILED, bool LORA, bool SAVE = false>  // SAVE: also keep g, u in a.gu
__global__ __launch_bounds__(64) void gate_up_bf16(ExpertArgs a) {
  const int ntile = a.I / 64;
  const int wave = blockIdx.x % kSub, bq = blockIdx.x / kSub;
  const int item = bq / ntile, nt = bq - item * ntile;
  if (item >= *a.n_items) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  Item it;
  it.e = a.items[2 * item];
  // row-major: row n0 + r, k offset 8g, step 32 elements; tiled: fragment
  // (row tile, k-step) is 512 elements, this lane's 8 at offset 8 * lane
  const uint16_t* wg = TILED ? a.w_gate_up + (((size_t)it.e * (2 * I / 16) + n0 / 16) * (H / 32) * 64 + lane) * 8
                             : a.w_gate_up + ((size_t)it.e * 2 * I + n0 + r) * H + g * 8;
  const uint16_t* wu = TILED ? wg + (size_t)(I / 16) * (H / 32) * 512 : wg + (size_t)I * H;
  const int wstep = TILED ? 512 : 32;  // elements per k-step
  // the first U k-steps of weights depend on the expert only: they are in
  // flight while the item's rows and tokens are looked up
  u32x4_t ga0[U], ua0[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    ga0[u] = ld16_stream(wg + u * wstep);
    ua0[u] = ld16_stream(wu + u * wstep);
  }
  {
    const int m0 = a.items[2 * item + 1];
    const int c = a.counts[it.e] - m0;
    it.M = c < kTile ? c : kTile;
    it.base = a.offsets[it.e] + m0;
  }
  const bool rv = r < it.M;
  const int tok = rv ? a.perm[it.base + r] / a.k : 0;
  const uint16_t* xr = a.x + (size_t)tok * H + g * 8;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  {
    u32x4_t xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) xb[u] = rv ? ld16(xr + u * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      accg = mfma16(ga0[u], xb[u], accg);
      accu = mfma16(ua0[u], xb[u], accu);
    }
  }
  for (int kk = 32 * U; kk < H; kk += 32 * U) {
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
  if constexpr (LORA) {  // every lane takes part in the MFMAs
    const f32x4_t uq = rv ? ld4f(a.u_gate_up + (size_t)(it.base + r) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* bg = a.lb_gate_up + ((size_t)it.e * 2 * I + n0 + r) * 16 + 4 * g;
    add_scaled(accg, lora_tile(ld4f(bg), uq), a.lora_scale);
    add_scaled(accu, lora_tile(ld4f(bg + (size_t)I * 16), uq), a.lora_scale);
  }
  if (rv) {
    if constexpr (SAVE) {  // the pre-activations the nonlinearity sees
      float* gp = a.gu + (size_t)(it.base + r) * 2 * I + n0 + 4 * g;
      *reinterpret_cast<f32x4_t*>(gp) = accg;
      *reinterpret_cast<f32x4_t*>(gp + I) = accu;
    }
    float hv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hv[q] = silu(accg[q]) * accu[q];
    u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
    *reinterpret_cast<u32x2_t*>(a.h + (size_t)(it.base + r) * I + n0 + 4 * g) = pk;
  }
}

template <int U, bool TILED, bool LORA>
__global__ __launch_bounds__(64) void down_bf16(ExpertArgs a) {
  const int ctile = a.H / 128;
  const int wave = blockIdx.x % kSub, bq = blockIdx.x / kSub;
  const int item = bq / ctile, ct = bq - item * ctile;
  if (item >= *a.n_items) return;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  Item it;
  it.e = a.items[2 * item];
  const uint16_t* w0 = TILED ? a.w_down + (((size_t)it.e * (H / 16) + c0 / 16) * (I / 32) * 64 + lane) * 8
                             : a.w_down + ((size_t)it.e * H + c0 + r) * I + g * 8;
  const uint16_t* w1 = TILED ? w0 + (size_t)(I / 32) * 512 : w0 + (size_t)16 * I;
  const int wstep = TILED ? 512 : 32;
  // the first U k-steps of weights go out before the item's rows are known
  u32x4_t a00[U], a10[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    a00[u] = ld16_stream(w0 + u * wstep);
    a10[u] = ld16_stream(w1 + u * wstep);
  }
  {
    const int m0 = a.items[2 * item + 1];
    const int c = a.counts[it.e] - m0;
    it.M = c < kTile ? c : kTile;
    it.base = a.offsets[it.e] + m0;
  }
  const bool rv = r < it.M;
  const uint16_t* hr = a.h + (size_t)(it.base + (rv ? r : 0)) * I + g * 8;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  {
    u32x4_t hb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) hb[u] = rv ? ld16(hr + u * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc0 = mfma16(a00[u], hb[u], acc0);
      acc1 = mfma16(a10[u], hb[u], acc1);
    }
  }
  for (int kk = 32 * U; kk < I; kk += 32 * U) {
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
  if constexpr (LORA) {  // every lane takes part in the MFMAs
    const f32x4_t uq = rv ? ld4f(a.u_down + (size_t)(it.base + r) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* b0 = a.lb_down + ((size_t)it.e * H + c0 + r) * 16 + 4 * g;
    add_scaled(acc0, lora_tile(ld4f(b0), uq), a.lora_scale);
    add_scaled(acc1, lora_tile(ld4f(b0 + 16 * 16), uq), a.lora_scale);
  }
  if (rv) {
    const int slot = a.perm[it.base + r];
    float* yrow = a.y + (size_t)slot * H;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 4 * g) = acc0;
    *reinterpret_cast<f32x4_t*>(yrow + c0 + 16 + 4 * g) = acc1;
  }
}

// ------------------------------------------------------------------ direct form
// When most experts hold rows (at decode sizes, 2E <= N <= kDirectMaxN
// slots), the grid covers every expert and no work list is formed: the wave
// for (expert e, column tile) finds e's slots itself by scanning the N
// routed ids, so no bucketing kernel runs before it.  Its first batch of
// weights depends on e only and is in flight from the wave's start, and its
// chain of dependent loads before the first MFMA is ids -> token rows
// instead of work list -> counts/offsets -> perm -> token rows.  Lane l holds
// P consecutive slots (P a multiple of 4, at most 16); e's slots in ascending
// order are ranked by a wave prefix sum of the per-lane match counts, and
// e's offset in sorted-slot order is the number of slots routed to lower
// experts: the values the bucketing kernel forms, so h keeps its sorted-slot
// layout, and one wave per expert records counts, offsets, perm and pos.  An
// expert takes its rows 32 at a time (two 16-row MFMA column blocks per
// weight load, half as many k-steps per batch of loads, which keeps the
// register count of the one-block pass), the last pass 16 if no more
// remain; each 16-row block gets the same MFMA chain as in the work-list
// kernels, so rows keep their bits.
struct SlotList {
  int count, off;
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// e's live slots, ascending, into s_slot[0 .. count); every lane gets count
// and the offset.  ids is read in whole 16-byte chunks (the workspace pads
// the array to a multiple of 16 bytes); entries at or past N are ignored.
__device__ __forceinline__ SlotList scan_slots(const ExpertArgs& a, int e, int lane, int* s_slot) {
  const int N = a.live ? min(a.N, *a.live * a.k) : a.N;
  const int P = (((N + 63) >> 6) + 3) & ~3;  // <= 16 for N <= kDirectMaxN
  const int s0 = lane * P;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] = (4 * c < P && s0 + 4 * c < N) ? ld16(a.ids + s0 + 4 * c) : zero;
  uint32_t m = 0u;
  int lt = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int id = (int)v[q >> 2][q & 3];
    const int ce = id < 0 ? 0 : (id >= a.E ? a.E - 1 : id);  // as the bucketing clamps
    const bool ok = q < P && s0 + q < N;
    m |= (ok && ce == e ? 1u : 0u) << q;
    lt += ok && ce < e ? 1 : 0;
  }
  const int cnt = __popc(m);
  const int incl = wave_incl_scan(cnt, lane);
  const int lti = wave_incl_scan(lt, lane);
  SlotList sl;
  sl.count = __builtin_amdgcn_readlane(incl, 63);
  sl.off = __builtin_amdgcn_readlane(lti, 63);
  int rk = incl - cnt;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if ((m >> q) & 1u) s_slot[rk++] = s0 + q;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return sl;
}

// the bucketing of expert e as the bucketing kernel writes it (work list aside)
__device__ __forceinline__ void publish_slots(const ExpertArgs& a, int e, const SlotList& sl, int lane,
                                              const int* s_slot) {
  if (lane == 0) {
    a.r_counts[e] = sl.count;
    a.r_offsets[e] = sl.off;
    if (e == a.E - 1) a.r_offsets[a.E] = sl.off + sl.count;
  }
  for (int i = lane; i < sl.count; i += 64) {
    const int s = s_slot[i];
    a.r_perm[sl.off + i] = s;
    if (a.r_pos) a.r_pos[s] = sl.off + i;
  }
}

// rows m0 .. m0 + 16 RT - 1 of expert e's list through one pass over its
// gate/up weights (wg: this lane's first gate chunk; its up chunk is wuo
// elements further).  PRE: the first U k-steps of weights are already in
// pg / pu (issued before the slot scan).
template <int U, int RT, bool PRE = false>
__device__ __forceinline__ void gate_up_pass(const ExpertArgs& a, const uint16_t* wg, size_t wuo, int wstep,
                                             const SlotList& sl, int m0, const int* s_slot, int n0, int lane,
                                             const u32x4_t* pg = nullptr, const u32x4_t* pu = nullptr) {
  const int H = a.H, I = a.I, r = lane & 15, g = lane >> 4;
  bool rv[RT];
  const uint16_t* xr[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const int i = m0 + 16 * j + r;
    rv[j] = i < sl.count;
    const int tok = rv[j] ? s_slot[i] / a.k : 0;
    xr[j] = a.x + (size_t)tok * H + g * 8;
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t accg[RT], accu[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) accg[j] = accu[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto batch = [&](const u32x4_t* ga, const u32x4_t* ua, int kk) {
    u32x4_t xb[RT][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < RT; ++j) xb[j][u] = rv[j] ? ld16(xr[j] + kk + u * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        accg[j] = mfma16(ga[u], xb[j][u], accg[j]);
        accu[j] = mfma16(ua[u], xb[j][u], accu[j]);
      }
    }
  };
  int kk0 = 0;
  if constexpr (PRE) {
    batch(pg, pu, 0);
    __builtin_amdgcn_sched_barrier(0);  // the loop's loads stay below: pg, pu and them are not live together
    kk0 = 32 * U;
  }
  for (int kk = kk0; kk < H; kk += 32 * U) {
    u32x4_t ga[U], ua[U];
    const size_t wo = (size_t)(kk / 32) * wstep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ga[u] = ld16_stream(wg + wo + u * wstep);
      ua[u] = ld16_stream(wg + wuo + wo + u * wstep);
    }
    batch(ga, ua, kk);
  }
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    if (rv[j]) {
      float hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = silu(accg[j][q]) * accu[j][q];
      u32x2_t pk = {pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
      *reinterpret_cast<u32x2_t*>(a.h + (size_t)(sl.off + m0 + 16 * j + r) * I + n0 + 4 * g) = pk;
    }
  }
}

// k-steps per batch of weight loads in the direct kernels' one-block pass
// (the first batch is issued before the slot scan; eight would not fit the
// register budget of four waves per SIMD with it)
constexpr int kDU = 4;

template <int U, bool TILED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void gate_up_direct(ExpertArgs a) {
  __shared__ int s_slot[kDirectMaxN];
  const int ntile = a.I / 64;
  const int wave = blockIdx.x % kSub, bq = blockIdx.x / kSub;
  const int e = bq / ntile, nt = bq - e * ntile;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 64 + wave * 16;
  const uint16_t* wg = TILED ? a.w_gate_up + (((size_t)e * (2 * I / 16) + n0 / 16) * (H / 32) * 64 + lane) * 8
                             : a.w_gate_up + ((size_t)e * 2 * I + n0 + r) * H + g * 8;
  const size_t wuo = TILED ? (size_t)(I / 16) * (H / 32) * 512 : (size_t)I * H;  // up rows after the gate rows
  const int wstep = TILED ? 512 : 32;
  // the first batch of weights depends on the expert only: it is in flight
  // during the slot scan (and dropped if the expert has no rows)
  u32x4_t pg[U], pu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    pg[u] = ld16_stream(wg + u * wstep);
    pu[u] = ld16_stream(wg + wuo + u * wstep);
  }
  const SlotList sl = scan_slots(a, e, lane, s_slot);
  if (nt == 0 && wave == 0) publish_slots(a, e, sl, lane, s_slot);
  if (sl.count <= kTile) {
    if (sl.count > 0) gate_up_pass<U, 1, true>(a, wg, wuo, wstep, sl, 0, s_slot, n0, lane, pg, pu);
    return;
  }
  for (int m0 = 0; m0 < sl.count; m0 += 2 * kTile) {
    if (sl.count - m0 > kTile)
      gate_up_pass<U / 2, 2>(a, wg, wuo, wstep, sl, m0, s_slot, n0, lane);
    else
      gate_up_pass<U, 1>(a, wg, wuo, wstep, sl, m0, s_slot, n0, lane);
  }
}

// rows m0 .. m0 + 16 RT - 1 of expert e's list through one pass over its
// down weights (w0: this lane's first chunk of the wave's first 16-column
// block; block b's chunks are wb elements further).  PRE: the first U
// k-steps of weights are already in pre.
template <int U, int RT, int CB, bool PRE = false>
__device__ __forceinline__ void down_pass(const ExpertArgs& a, const uint16_t* w0, size_t wb, int wstep,
                                          const SlotList& sl, int m0, const int* s_slot, int c0, int lane,
                                          const u32x4_t* pre = nullptr) {
  const int H = a.H, I = a.I, r = lane & 15, g = lane >> 4;
  bool rv[RT];
  const uint16_t* hr[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const int i = m0 + 16 * j + r;
    rv[j] = i < sl.count;
    hr[j] = a.h + (size_t)(sl.off + (rv[j] ? i : 0)) * I + g * 8;
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc[RT][CB];
#pragma unroll
  for (int j = 0; j < RT; ++j)
#pragma unroll
    for (int b = 0; b < CB; ++b) acc[j][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // wv[b * U + u]: block b, k-step u of the batch
  auto batch = [&](const u32x4_t* wv, int kk) {
    u32x4_t hb[RT][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < RT; ++j) hb[j][u] = rv[j] ? ld16(hr[j] + kk + u * 32) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < RT; ++j)
#pragma unroll
        for (int b = 0; b < CB; ++b) acc[j][b] = mfma16(wv[b * U + u], hb[j][u], acc[j][b]);
  };
  int kk0 = 0;
  if constexpr (PRE) {
    batch(pre, 0);
    __builtin_amdgcn_sched_barrier(0);
    kk0 = 32 * U;
  }
  for (int kk = kk0; kk < I; kk += 32 * U) {
    u32x4_t wv[CB * U];
    const size_t wo = (size_t)(kk / 32) * wstep;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < CB; ++b) wv[b * U + u] = ld16_stream(w0 + b * wb + wo + u * wstep);
    batch(wv, kk);
  }
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    if (rv[j]) {
      float* yrow = a.y + (size_t)s_slot[m0 + 16 * j + r] * H + c0 + 4 * g;
#pragma unroll
      for (int b = 0; b < CB; ++b) *reinterpret_cast<f32x4_t*>(yrow + 16 * b) = acc[j][b];
    }
  }
}

constexpr int kDnCB = 2;  // 16-column blocks of the output per wave (direct down)

// wave (e, cw) computes output columns cw * 16 CB .. + 16 CB - 1 of expert
// e's rows; U2: k-steps per batch of loads in the two-block pass
template <int U, int U2, int CB, bool TILED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void down_direct(ExpertArgs a) {
  __shared__ int s_slot[kDirectMaxN];
  const int ncw = a.H / (16 * CB);
  const int e = blockIdx.x / ncw, cw = blockIdx.x - e * ncw;
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = cw * 16 * CB;
  const uint16_t* w0 = TILED ? a.w_down + (((size_t)e * (H / 16) + c0 / 16) * (I / 32) * 64 + lane) * 8
                             : a.w_down + ((size_t)e * H + c0 + r) * I + g * 8;
  const size_t wb = TILED ? (size_t)(I / 32) * 512 : (size_t)16 * I;
  const int wstep = TILED ? 512 : 32;
  u32x4_t pre[CB * U];  // first batch, in flight during the slot scan
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int b = 0; b < CB; ++b) pre[b * U + u] = ld16_stream(w0 + b * wb + u * wstep);
  const SlotList sl = scan_slots(a, e, lane, s_slot);
  if (sl.count <= kTile) {
    if (sl.count > 0) down_pass<U, 1, CB, true>(a, w0, wb, wstep, sl, 0, s_slot, c0, lane, pre);
    return;
  }
  for (int m0 = 0; m0 < sl.count; m0 += 2 * kTile) {
    if (sl.count - m0 > kTile)
      down_pass<U2, 2, CB>(a, w0, wb, wstep, sl, m0, s_slot, c0, lane);
    else
      down_pass<U, 1, CB>(a, w0, wb, wstep, sl, m0, s_slot, c0, lane);
  }
}

// ------------------------------------------------------------------ 4-bit
// (the table and the code and scale loads are in nf4.hpp)

// one 128-k block of one weight tile: acc[q] += absmax_0 * P0[q] + absmax_1 * P1[q]
__device__ __forceinline__ f32x4_t block_mma(const u32x2_t* s_lutl, u32x4_t codes, const u32x4_t (&xb)[4],
                                             u32x2_t sc, f32x4_t acc) {
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  u32x4_t hi[4], lo[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) lut8(s_lutl, codes[st], hi[st], lo[st]);
  f32x4_t p0 = mfma16(xb[0], lo[0], zero);
  p0 = mfma16(xb[1], lo[1], p0);
  p0 = mfma16(xb[0], hi[0], p0);
  p0 = mfma16(xb[1], hi[1], p0);
  f32x4_t p1 = mfma16(xb[2], lo[2], zero);
  p1 = mfma16(xb[3], lo[3], p1);
  p1 = mfma16(xb[2], hi[2], p1);
  p1 = mfma16(xb[3], hi[3], p1);
  const float s0 = __uint_as_float(sc[0]), s1 = __uint_as_float(sc[1]);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = fmaf(s1, p1[q], fmaf(s0, p0[q], acc[q]));
  return acc;
}

// gate/up: a wave owns two 16-row tiles of gate rows and the matching up
// rows (32 n), so one token fragment feeds four weight tiles; the table is
// built once per 4-wave workgroup
template <int NB, bool TILED, bool LORA>  // NB: 128-k blocks per loop iteration (H % (128 * NB) == 0)
__global__ __launch_bounds__(kNf4Threads) void gate_up_nf4(ExpertArgs a) {
  __shared__ u32x2_t s_lut[256 * kLutRep];
  const int ntile = a.I / 128;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  Item it;
  if (!load_item(a, item, it)) return;
  build_lut(s_lut, a.codebook, threadIdx.x);
  __syncthreads();
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = nt * 128 + wave * 32;
  const u32x2_t* sl = lut_copy(s_lut, lane);
  const bool rv = r < it.M;
  const int tok = rv ? a.perm[it.base + r] / a.k : 0;
  const uint16_t* xr = a.x + (size_t)tok * H + 8 * g;
  const int nkb = H / 128;
  // tiles j = 0, 1: gate rows n0 + 16j; j = 2, 3: the matching up rows
  const uint8_t* q[4];
  const float* sp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t row0 = (size_t)it.e * 2 * I + (j >= 2 ? I : 0) + n0 + 16 * (j & 1);  // first row of the tile
    const size_t rt = row0 / 16;
    q[j] = TILED ? a.q_gate_up + (rt * nkb * 64 + lane) * 16 : a.q_gate_up + (row0 + r) * (H / 2);
    sp[j] = TILED ? a.s_gate_up + rt * nkb * 32 + 2 * r : a.s_gate_up + (row0 + r) * (H / 64);
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kb0 = 0; kb0 < nkb; kb0 += NB) {
    u32x4_t cd[NB][4], xb[NB][4];
    u32x2_t sc[NB][4];
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const int kb = kb0 + h;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cd[h][j] = load_codes<TILED>(q[j], kb, g);
        sc[h][j] = load_scales<TILED>(sp[j], kb);
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) xb[h][st] = rv ? ld16(xr + 128 * kb + 32 * st) : zero;
    }
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = block_mma(sl, cd[h][j], xb[h], sc[h][j], acc[j]);
  }
  // lane holds tokens 4g + q of rows n0 + 16j + r
  if constexpr (LORA) {  // tokens are the rows of these tiles: P = U, Q = the adapter's B rows
    const f32x4_t up = rv ? ld4f(a.u_gate_up + (size_t)(it.base + r) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* bg = a.lb_gate_up + ((size_t)it.e * 2 * I + n0 + r) * 16 + 4 * g;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      add_scaled(acc[j], lora_tile(up, ld4f(bg + 16 * 16 * j)), a.lora_scale);
      add_scaled(acc[j + 2], lora_tile(up, ld4f(bg + (size_t)I * 16 + 16 * 16 * j)), a.lora_scale);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 4 * g + q;
    if (m < it.M) {
      uint16_t* hrow = a.h + (size_t)(it.base + m) * I + n0 + r;
      if (a.gu) {  // training forward: keep the pre-activations the nonlinearity sees
        float* gp = a.gu + (size_t)(it.base + m) * 2 * I + n0 + r;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          gp[16 * j] = acc[j][q];
          gp[I + 16 * j] = acc[j + 2][q];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float hv = silu(acc[j][q]) * acc[j + 2][q];
        hrow[16 * j] = (uint16_t)(pack_bf16x2(hv, 0.f) & 0xffffu);
      }
    }
  }
}

// down: a wave owns two 16-row tiles of W_down (32 output columns)
template <int NB, bool TILED, bool LORA>  // NB: 128-k blocks per loop iteration (I % (128 * NB) == 0)
__global__ __launch_bounds__(kNf4Threads) void down_nf4(ExpertArgs a) {
  __shared__ u32x2_t s_lut[256 * kLutRep];
  const int ctile = a.H / 128;
  const int item = blockIdx.x / ctile, ct = blockIdx.x - item * ctile;
  Item it;
  if (!load_item(a, item, it)) return;
  build_lut(s_lut, a.codebook, threadIdx.x);
  __syncthreads();
  const int H = a.H, I = a.I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = ct * 128 + wave * 32;
  const u32x2_t* sl = lut_copy(s_lut, lane);
  const bool rv = r < it.M;
  const uint16_t* hr = a.h + (size_t)(it.base + (rv ? r : 0)) * I + 8 * g;
  const int nkb = I / 128;
  const uint8_t* q[2];
  const float* sp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const size_t row0 = (size_t)it.e * H + c0 + 16 * j;
    const size_t rt = row0 / 16;
    q[j] = TILED ? a.q_down + (rt * nkb * 64 + lane) * 16 : a.q_down + (row0 + r) * (I / 2);
    sp[j] = TILED ? a.s_down + rt * nkb * 32 + 2 * r : a.s_down + (row0 + r) * (I / 64);
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int kb0 = 0; kb0 < nkb; kb0 += NB) {
    u32x4_t cd[NB][2], hb[NB][4];
    u32x2_t sc[NB][2];
#pragma unroll
    for (int h = 0; h < NB; ++h) {
      const int kb = kb0 + h;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        cd[h][j] = load_codes<TILED>(q[j], kb, g);
        sc[h][j] = load_scales<TILED>(sp[j], kb);
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) hb[h][st] = rv ? ld16(hr + 128 * kb + 32 * st) : zero;
    }
#pragma unroll
    for (int h = 0; h < NB; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = block_mma(sl, cd[h][j], hb[h], sc[h][j], acc[j]);
  }
  // lane holds tokens 4g + q of output columns c0 + 16j + r
  if constexpr (LORA) {
    const f32x4_t up = rv ? ld4f(a.u_down + (size_t)(it.base + r) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float* b0 = a.lb_down + ((size_t)it.e * H + c0 + r) * 16 + 4 * g;
    add_scaled(acc[0], lora_tile(up, ld4f(b0)), a.lora_scale);
    add_scaled(acc[1], lora_tile(up, ld4f(b0 + 16 * 16)), a.lora_scale);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int m = 4 * g + q;
    if (m < it.M) {
      float* yrow = a.y + (size_t)a.perm[it.base + m] * H + c0 + r;
      yrow[0] = acc[0][q];
      yrow[16] = acc[1][q];
    }
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

// 4-bit down: a grid of at most kNf4DnSmallGrid workgroups (a few tokens)
// takes the largest count up to 3 of 128-k blocks per loop iteration that
// divides I / 128, which shortens each wave's chain of dependent loads; a
// larger grid takes one block per iteration, which keeps more waves resident
constexpr int kNf4DnSmallGrid = 1024;

template <bool LORA>
hipError_t launch_gate_up_t(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  if (nf4) {
    // one 128-k block per iteration (more only cost occupancy)
    const dim3 grid(a.max_items * (a.I / 128));  // 128 n per workgroup
    if (tiled)
      hipLaunchKernelGGL((gate_up_nf4<1, true, LORA>), grid, dim3(kNf4Threads), 0, s, a);
    else
      hipLaunchKernelGGL((gate_up_nf4<1, false, LORA>), grid, dim3(kNf4Threads), 0, s, a);
    return hipGetLastError();
  }
  const dim3 gw(a.max_items * (a.I / 64) * kSub);
  if (a.gu && tiled)  // training forward: keep the pre-activations
    return launch_u(a.H, gate_up_bf16<8, true, LORA, true>, gate_up_bf16<4, true, LORA, true>, gw, s, a, 64);
  return tiled ? launch_u(a.H, gate_up_bf16<8, true, LORA>, gate_up_bf16<4, true, LORA>, gw, s, a, 64)
               : launch_u(a.H, gate_up_bf16<8, false, LORA>, gate_up_bf16<4, false, LORA>, gw, s, a, 64);
}

template <bool TILED, bool LORA>
void launch_down_nf4(const ExpertArgs& a, hipStream_t s) {
  const dim3 grid(a.max_items * (a.H / 128));  // 128 output columns per workgroup
  const int nkb = a.I / 128;
  const bool small = (long)grid.x <= kNf4DnSmallGrid;
  if (small && nkb % 3 == 0)
    hipLaunchKernelGGL((down_nf4<3, TILED, LORA>), grid, dim3(kNf4Threads), 0, s, a);
  else if (small && nkb % 2 == 0)
    hipLaunchKernelGGL((down_nf4<2, TILED, LORA>), grid, dim3(kNf4Threads), 0, s, a);
  else
    hipLaunchKernelGGL((down_nf4<1, TILED, LORA>), grid, dim3(kNf4Threads), 0, s, a);
}

template <bool LORA>
hipError_t launch_down_t(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  if (nf4) {
    if (tiled)
      launch_down_nf4<true, LORA>(a, s);
    else
      launch_down_nf4<false, LORA>(a, s);
    return hipGetLastError();
  }
  const dim3 gw(a.max_items * (a.H / 128) * kSub);
  return tiled ? launch_u(a.I, down_bf16<8, true, LORA>, down_bf16<4, true, LORA>, gw, s, a, 64)
               : launch_u(a.I, down_bf16<8, false, LORA>, down_bf16<4, false, LORA>, gw, s, a, 64);
}

// the direct form covers bf16 weights without adapters or kept pre-activations
bool direct_ok(const ExpertArgs& a, bool nf4) {
  return !nf4 && !a.lora && !a.gu && a.N >= 1 && a.N <= kDirectMaxN && a.H % (32 * kDU) == 0 &&
         a.I % (32 * kDU) == 0;
}

hipError_t launch_gate_up(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  if (a.ids) {
    if (!direct_ok(a, nf4)) return hipErrorInvalidValue;
    const dim3 gw(a.E * (a.I / 64) * kSub);
    if (tiled)
      hipLaunchKernelGGL((gate_up_direct<kDU, true>), gw, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((gate_up_direct<kDU, false>), gw, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  return a.lora ? launch_gate_up_t<true>(a, nf4, tiled, s) : launch_gate_up_t<false>(a, nf4, tiled, s);
}

hipError_t launch_down(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s) {
  if (a.ids) {
    if (!direct_ok(a, nf4)) return hipErrorInvalidValue;
    const dim3 gw(a.E * (a.H / (16 * kDnCB)));
    if (tiled)
      hipLaunchKernelGGL((down_direct<kDU, kDU / 2, kDnCB, true>), gw, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((down_direct<kDU, kDU / 2, kDnCB, false>), gw, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  return a.lora ? launch_down_t<true>(a, nf4, tiled, s) : launch_down_t<false>(a, nf4, tiled, s);
}

}  // namespace moe
