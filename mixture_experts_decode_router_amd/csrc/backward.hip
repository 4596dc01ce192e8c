// Backward of the block for frozen weights and the forward's routing (the
// top-k choice is piecewise constant in x): given dL/dout, the gradients with
// respect to the input x and to the routing weights,
//   d_w[t][j] = <d_out[t], y[t*k+j]>
//   d_l[t][j] = w_j (d_w_j - sum_i w_i d_w_i)           (renormalised softmax)
//   d_h[p]    = W_d^T (w_p d_out[t_p]),  d_g = d_h u silu'(g),  d_u = d_h silu(g)
//               (g, u: the pre-activations a training forward kept)
//   d_x[t]    = sum_j d_l[t][j] Wr[id_j] + sum_j (W_g^T d_g + W_u^T d_u)[t*k+j]
// The grouped GEMM path these follow is the grouped_mm MoE of the unsloth
// commit 80aaf1121b page (third paragraph), whose training branch the GRPO
// runs of the 4f2bfe7f69 page use.
//
// Kernels: bwd_weights (one workgroup per token: d_w, d_l and the router's
// share of d_x), bwd_t<DOWN> and bwd_t<GATE_UP> (grouped transposed GEMVs over the tiled
// weight fragments, each 16 x 32 fragment pair turned through LDS into MFMA
// operands), bwd_combine (per-token sum over the k slots, j in order).  No
// float atomics: every output element is written once, sums run in a fixed
// order.
#include "common.hpp"
#include "kernels.hpp"
#include "nf4.hpp"

namespace moe {
namespace {

constexpr int kU = 8;  // 32-row steps of loads in flight per wave

// a one-wave workgroup's LDS writes are visible to all its lanes (no wait on
// global loads still in flight)
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Top-k weights without renormalisation: w_j = p[id_j], p the softmax over
// all E logits, so the logit gradient reaches every expert,
//   d_l[e] = [e chosen] w_e d_w_e - p_e sum_j w_j d_w_j,
// and the router's share of d_x is sum_e d_l[e] Wr[e] over all E.  p comes
// from the router's approximate logits (stored split partials summed in
// split order, plus the bias), which lie within ~1e-6 of the fp32 logits.
// Thread e < E handles expert e; sums over the workgroup run in wave order.
__device__ void router_share_all(const BwdArgs& a, int t, float swd, const float* s_dw) {
  __shared__ float s_dl[256];
  __shared__ float s_r[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, H = a.H, T = a.T, k = a.k;
  float lg = -INFINITY;
  if (tid < E) {
    float sum = 0.f;
    for (int sp = 0; sp < a.r_nst; ++sp) sum += a.r_part[((size_t)sp * T + t) * E + tid];
    lg = a.r_bias ? sum + a.r_bias[tid] : sum;
  }
  float m = lg;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) s_r[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]));
  __syncthreads();  // s_r is reused
  const float ex = tid < E ? __expf(lg - m) : 0.f;
  const float ws = wave_sum(ex);
  if (lane == 0) s_r[wave] = ws;
  __syncthreads();
  const float z = ((s_r[0] + s_r[1]) + s_r[2]) + s_r[3];
  if (tid < E) {
    float dl = -(ex / z) * swd;
    for (int j = 0; j < k; ++j)
      if (a.ids[(size_t)t * k + j] == tid) dl = fmaf(a.wts[(size_t)t * k + j], s_dw[j], dl);
    s_dl[tid] = dl;
  }
  __syncthreads();
  // sum_e d_l[e] Wr[e] per column chunk of 4, e in order
  for (int c4 = tid; c4 < H / 4; c4 += 256) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int e = 0; e < E; ++e) {
      const u32x2_t wv = *reinterpret_cast<const u32x2_t*>(a.w_router + (size_t)e * H + 4 * c4);
      const float dl = s_dl[e];
      acc[0] = fmaf(dl, bf16lo(wv[0]), acc[0]);
      acc[1] = fmaf(dl, bf16hi(wv[0]), acc[1]);
      acc[2] = fmaf(dl, bf16lo(wv[1]), acc[2]);
      acc[3] = fmaf(dl, bf16hi(wv[1]), acc[3]);
    }
    *reinterpret_cast<f32x4_t*>(a.d_x + (size_t)t * H + 4 * c4) = acc;
  }
}

// ---------------------------------------------------------------- weights
// One 256-thread workgroup per token; thread i holds the float4 column
// chunks i, i + 256, ... (at most 4: H <= 4096).  For each chunk the y rows
// of all k slots are loaded together, so a token costs one load round trip
// per chunk, not one per slot (KS: the slot count where it is known at
// compile time, whose two chunks' loads are then in flight together).  Per
// slot: the thread's partial dot, a butterfly over the wave, the four wave
// sums added in wave order.
template <int KS>
__global__ __launch_bounds__(256) void bwd_weights_kernel(BwdArgs a) {
  __shared__ float s_part[16][4];
  __shared__ float s_dw[16];
  constexpr int kMaxKs = KS > 0 ? KS : 16;
  constexpr int kPair = KS > 0 && KS <= 8 ? 2 : 1;  // chunks whose loads issue together
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, k = KS > 0 ? KS : a.k, n4 = H / 4;
  const float* dout = a.d_out + (size_t)t * H;
  const float* ybase = a.y + (size_t)t * k * H;
  float part[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) part[j] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < 4; i0 += kPair) {
    f32x4_t dv[kPair], yv[kPair][kMaxKs];
#pragma unroll
    for (int u = 0; u < kPair; ++u) {
      const int c4 = tid + 256 * (i0 + u);
      if (c4 < n4) {
        dv[u] = *reinterpret_cast<const f32x4_t*>(dout + 4 * c4);
#pragma unroll
        for (int j = 0; j < kMaxKs; ++j)
          if (j < k) yv[u][j] = *reinterpret_cast<const f32x4_t*>(ybase + (size_t)j * H + 4 * c4);
      }
    }
#pragma unroll
    for (int u = 0; u < kPair; ++u) {
      if (tid + 256 * (i0 + u) < n4) {
#pragma unroll
        for (int j = 0; j < kMaxKs; ++j)
          if (j < k)
#pragma unroll
            for (int q = 0; q < 4; ++q) part[j] = fmaf(dv[u][q], yv[u][j][q], part[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      const float v = wave_sum(part[j]);
      if (lane == 0) s_part[j][wave] = v;
    }
  }
  __syncthreads();
  if (tid < k) s_dw[tid] = ((s_part[tid][0] + s_part[tid][1]) + s_part[tid][2]) + s_part[tid][3];
  __syncthreads();
  float swd = 0.f;
  for (int j = 0; j < k; ++j) swd = fmaf(a.wts[(size_t)t * k + j], s_dw[j], swd);
  if (a.d_w && tid < k) a.d_w[(size_t)t * k + tid] = s_dw[tid];
  if (a.unrenorm) {
    router_share_all(a, t, swd, s_dw);
    return;
  }
  // the router's share: sum_j d_l_j Wr[id_j], j in order, d_l_j = w_j (d_w_j - swd)
  float dl[16];
  int ids[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    dl[j] = j < k ? a.wts[(size_t)t * k + j] * (s_dw[j] - swd) : 0.f;
    ids[j] = j < k ? a.ids[(size_t)t * k + j] : 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c4 = tid + 256 * i;
    if (c4 >= n4) break;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      const u32x2_t wv = *reinterpret_cast<const u32x2_t*>(a.w_router + (size_t)ids[j] * H + 4 * c4);
      acc[0] = fmaf(dl[j], bf16lo(wv[0]), acc[0]);
      acc[1] = fmaf(dl[j], bf16hi(wv[0]), acc[1]);
      acc[2] = fmaf(dl[j], bf16lo(wv[1]), acc[2]);
      acc[3] = fmaf(dl[j], bf16hi(wv[1]), acc[3]);
    }
    *reinterpret_cast<f32x4_t*>(a.d_x + (size_t)t * H + 4 * c4) = acc;
  }
}

// ---------------------------------------------------------------- transposed GEMVs
// out[p][n] = sum_m W[e][m][n] v[p][m] for the routed rows p of a work item
// (<= 16) and one 32-column tile n0 = 32 ks of W (tiled: fragment (rt, ks) is
// W[16rt .. +16][32ks .. +32], lane (g, r) holding row r, columns 8g .. 8g+7).
// The rows are the MFMA A operand (lane (r, g): row r, m = 8g .. 8g+7 of a
// 32-m step).  Each fragment pair (rt = 2s, 2s+1) is written to LDS row-major
// (one 16-byte write per lane and fragment: rows m = 0..31, 32 columns, rows
// kRowStride elements apart) and a lane's B operand (column r or 16 + r, m =
// 8g .. 8g+7) is read back with two transposing reads (ds_read_b64_tr_b16:
// within each 16-lane group, lane j's value q comes from the address lane
// 4q + (j >> 2) supplies, plus j & 3 elements; so lane (r, g) supplies row
// 8g + (r >> 2) (+ 4 for the second read), column 16 nh + 4 (r & 3)).  v
// enters the MFMA rounded to bf16, except in the DOWN pass
// when adapter or weight gradients are formed (HILO), where it enters as two
// bf16 parts, hi = RNE(v) and lo = RNE(v - hi), in two MFMAs into the same
// accumulator, so that d_h carries about 16 bits of v (the weights are exact
// in bf16): those gradients are outer products of d_g, d_u with U, x or of
// B^T (d_g, d_u) with x, which pass each element's rounding error through
// unsmoothed.  (d_x, a sum over many terms, meets the bf16 tolerance either
// way.)
//   DOWN:    W = W_d [H][I], v = w_p d_out[t_p], epilogue: SiLU backward,
//            gu[p] (g, u) -> (d_g, d_u) in place.
//   GATE_UP: W = W_gu [2I][H], v = (d_g, d_u)[p], epilogue: d_xs[slot(p)].
enum { kDown = 0, kGateUp = 1 };

constexpr int kRowStride = 40;  // elements per staged row: 32 columns + padding (rows stay 16-byte aligned)
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

// 4 bf16 of the transposing read at element offset off of the LDS array
__device__ __forceinline__ uint2 read_tr4(const uint16_t* base, int off) {
  const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off));
  return uint2{(uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16),
               (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16)};
}

// LoRA (LORA true): s * sum_j A[e][j][n] z[p][j] joins each output first
// (z = B^T v from lora_bt; A = A_d for DOWN, A_gu for GATE_UP), the chain
// rule through W + s B A.
// NF4: tiled 4-bit weights, W[m][n] = codebook[code] * absmax[m][n / 64].
// The lane's 8 codes of row r, columns 8g .. 8g+7 of the strip are dword
// (ks & 3) of its 16-byte code chunk in 128-column block ks >> 2.  The strip
// lies in one 64-column scale block, so the absmax depends on the row m
// only and is folded into v: the MFMA multiplies (v[p][m] * absmax[m]) by
// the codebook entries.  Each fp32 entry enters as two bf16 parts, hi =
// RNE(cb) and lo = RNE(cb - hi), staged as two fragments and multiplied in
// two MFMAs into the same accumulator (lo first), so the weights carry the
// entry to within 2^-18 of its magnitude, as in the forward.
// RT: 16-row tiles per work item (RT > 1 after an MFMA forward, whose rows
// are re-bucketed into items of 16 RT rows): each staged weight fragment
// then serves RT MFMAs, so the weights are streamed once per 16 RT rows.
// NS: 32-column strips per work unit (NS > 1 with RT > 1): the rows' v,
// read once per step for all NS strips, is read once per 32 NS columns.
template <int MODE, bool LORA, bool HILO, bool NF4 = false, int RT = 1, int NS = 1>
__global__ __launch_bounds__(64) void bwd_t_kernel(BwdArgs a) {
  static_assert(RT == 1 || (!LORA && !NF4), "adapters and 4-bit bases take 16-row items");
  static_assert(NS == 1 || RT > 1, "several strips per unit go with several row tiles");
  constexpr bool kHiLo = HILO && MODE == kDown;
  constexpr int kUr = RT == 1 ? kU : (kU / RT > 1 ? kU / RT : 1);  // steps of loads in flight
  constexpr int kStage = NF4 ? 2 : NS;  // staged fragments per step: the strips, or the hi and lo parts
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kStage][32 * kRowStride];
  // code byte -> the hi and the lo bf16 parts of (cb[low nibble], cb[high nibble])
  __shared__ u32x2_t s_lut[NF4 ? 256 : 1];
  const int I = a.I, H = a.H;
  const int ncols = MODE == kDown ? I : H;      // n
  const int nrows = MODE == kDown ? H : 2 * I;  // m
  const int nfr = ncols / 32;                   // 32-column fragments per row tile
  const int ntile = nfr / NS;
  const int item = blockIdx.x / ntile, ks = (blockIdx.x - item * ntile) * NS;  // first strip
  if (item >= *a.n_items) return;
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int c = a.counts[e] - m0;
  const int M = c < 16 * RT ? c : 16 * RT, base = a.offsets[e] + m0;
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  bool rv[RT];
  const float* vrow[RT];
  float vs[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * rt + r;
    rv[rt] = row < M;
    vs[rt] = 1.f;
    if (MODE == kDown) {
      const int slot = rv[rt] ? a.perm[base + row] : 0;
      vrow[rt] = a.d_out + (size_t)(slot / a.k) * H;
      vs[rt] = rv[rt] ? a.wts[slot] : 0.f;
    } else {
      vrow[rt] = a.gu + (size_t)(rv[rt] ? base + row : 0) * 2 * I;
    }
  }
  const uint16_t* W = MODE == kDown ? a.w_down : a.w_gate_up;
  const size_t rt0 = (size_t)e * (nrows / 16);
  const int nsteps = nrows / 32;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  // NF4: byte offset of this lane's code dword in row tile rt's chunk, and
  // the index of its row's absmax, as functions of rt
  const int nkb = ncols / 128;
  const uint8_t* Q = MODE == kDown ? a.q_down : a.q_gate_up;
  const float* SC = MODE == kDown ? a.s_down : a.s_gate_up;
  auto code_off = [&](size_t rt) { return ((rt * nkb + (ks >> 2)) * 64 + lane) * 16 + 4 * (ks & 3); };
  // the absmax of rows m = 8g .. 8g+7 of a 32-row step (row tile 2s + (g >> 1),
  // rows 8 (g & 1) + i) lie at floats 2i + h of the 16 from this base
  const int sh = (ks >> 1) & 1;
  auto scale_base = [&](size_t rt) { return (rt * nkb + (ks >> 2)) * 32 + 16 * (g & 1); };
  if constexpr (NF4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = lane + 64 * i;
      const float cl = a.codebook[b & 15], ch = a.codebook[b >> 4];
      const uint32_t hi = pack_bf16x2(cl, ch);
      s_lut[b] = u32x2_t{hi, pack_bf16x2(cl - bf16lo(hi), ch - bf16hi(hi))};
    }
    wave_sync_lds();
  }
  // 8 codes (element 2i in the low nibble of byte i) -> the hi and lo parts
  // of their 8 codebook entries as bf16 pairs
  auto decode8 = [&](uint32_t w, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x2_t v = s_lut[(w >> (8 * i)) & 0xffu];
      hi[i] = v[0];
      lo[i] = v[1];
    }
  };
  f32x4_t acc[RT][NS][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[rt][j][0] = acc[rt][j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // this lane's fragment rows go to rows r and 16 + r, columns 8g .. 8g+7;
  // its transposing reads start at row 8g + (r >> 2), column 4 (r & 3)
  const int w_off0 = r * kRowStride + 8 * g, w_off1 = (16 + r) * kRowStride + 8 * g;
  const int tr_off = (8 * g + (r >> 2)) * kRowStride + 4 * (r & 3);
  for (int s0 = 0; s0 < nsteps; s0 += kUr) {
    // kUr steps of loads in flight: two weight fragments and the rows' v
    u32x4_t f0[kUr][NS], f1[kUr][NS], va[kUr][RT], vl[kUr][RT];
    uint32_t c0[NF4 ? kUr : 1], c1[NF4 ? kUr : 1];
#pragma unroll
    for (int u = 0; u < kUr; ++u) {
      const int s = s0 + u;
#pragma unroll
      for (int j = 0; j < NS; ++j) f0[u][j] = f1[u][j] = zero;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) va[u][rt] = vl[u][rt] = zero;
      if constexpr (NF4) c0[u] = c1[u] = 0u;
      if (s < nsteps) {
        float sm[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};  // absmax of the lane's rows m (NF4)
        if constexpr (NF4) {
          c0[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(Q + code_off(rt0 + 2 * s)));
          c1[u] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(Q + code_off(rt0 + 2 * s + 1)));
          const float* sp = SC + scale_base(rt0 + 2 * s + (g >> 1));
          f32x4_t s4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) s4[j] = *reinterpret_cast<const f32x4_t*>(sp + 4 * j);
#pragma unroll
          for (int i = 0; i < 8; ++i) sm[i] = sh ? s4[i >> 1][2 * (i & 1) + 1] : s4[i >> 1][2 * (i & 1)];
        } else {
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            f0[u][j] = ld16_stream(W + (((rt0 + 2 * s) * nfr + ks + j) * 64 + lane) * 8);
            f1[u][j] = ld16_stream(W + (((rt0 + 2 * s + 1) * nfr + ks + j) * 64 + lane) * 8);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (rv[rt]) {
            const float* vr = vrow[rt];
            const float w = vs[rt];
            const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(vr + 32 * s + 8 * g);
            const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(vr + 32 * s + 8 * g + 4);
            const float t[8] = {w * v0[0] * sm[0], w * v0[1] * sm[1], w * v0[2] * sm[2], w * v0[3] * sm[3],
                                w * v1[0] * sm[4], w * v1[1] * sm[5], w * v1[2] * sm[6], w * v1[3] * sm[7]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t hi = pack_bf16x2(t[2 * i], t[2 * i + 1]);
              va[u][rt][i] = hi;
              if constexpr (kHiLo) vl[u][rt][i] = pack_bf16x2(t[2 * i] - bf16lo(hi), t[2 * i + 1] - bf16hi(hi));
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUr; ++u) {
      if (s0 + u >= nsteps) break;
      u32x4_t f0l = zero, f1l = zero;  // NF4: the lo parts
      if constexpr (NF4) {
        decode8(c0[u], f0[u][0], f0l);
        decode8(c1[u], f1[u][0], f1l);
      }
      wave_sync_lds();  // the previous step's reads are done
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        *reinterpret_cast<u32x4_t*>(s_w[j] + w_off0) = f0[u][j];
        *reinterpret_cast<u32x4_t*>(s_w[j] + w_off1) = f1[u][j];
      }
      if constexpr (NF4) {
        *reinterpret_cast<u32x4_t*>(s_w[1] + w_off0) = f0l;
        *reinterpret_cast<u32x4_t*>(s_w[1] + w_off1) = f1l;
      }
      wave_sync_lds();
#pragma unroll
      for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) {
          const uint2 lo = read_tr4(s_w[j], tr_off + 16 * nh);                   // m = 8g .. 8g+3
          const uint2 hi = read_tr4(s_w[j], tr_off + 4 * kRowStride + 16 * nh);  // m = 8g+4 .. 8g+7
          const u32x4_t b = {lo.x, lo.y, hi.x, hi.y};
          if constexpr (NF4) {  // the codebook entries' lo parts
            const uint2 llo = read_tr4(s_w[1], tr_off + 16 * nh);
            const uint2 lhi = read_tr4(s_w[1], tr_off + 4 * kRowStride + 16 * nh);
            const u32x4_t bl = {llo.x, llo.y, lhi.x, lhi.y};
            acc[0][j][nh] = mfma16(va[u][0], bl, acc[0][j][nh]);
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            acc[rt][j][nh] = mfma16(va[u][rt], b, acc[rt][j][nh]);
            if constexpr (kHiLo) acc[rt][j][nh] = mfma16(vl[u][rt], b, acc[rt][j][nh]);
          }
        }
      }
    }
  }
  // lane holds D[row 4g + q][column 32 ks + 16 nh + r]
  if constexpr (LORA) {  // s A^T z: rows p (P = z), columns n (Q[n][j] = A[e][j][n])
    const float* la = (MODE == kDown ? a.la_down + (size_t)e * 16 * I : a.la_gate_up + (size_t)e * 16 * H) +
                      32 * ks + r;
    const float* zb = MODE == kDown ? a.z_down : a.z_gate_up;
    const f32x4_t zp = r < M ? ld4f(zb + (size_t)(base + r) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nh = 0; nh < 2; ++nh) {
      f32x4_t aq;
#pragma unroll
      for (int c = 0; c < 4; ++c) aq[c] = la[(size_t)(4 * g + c) * ncols + 16 * nh];
      add_scaled(acc[0][0][nh], lora_tile(zp, aq), a.lora_scale);
    }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 16 * rt + 4 * g + q;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) {
          const int n = 32 * (ks + j) + 16 * nh + r;
          if (MODE == kDown) {
            float* gp = a.gu + (size_t)(base + m) * 2 * I;
            const float gv = gp[n], uv = gp[I + n];
            const float sg = 1.0f / (1.0f + __expf(-gv));
            const float dh = acc[rt][j][nh][q];
            gp[n] = dh * uv * (sg * (1.0f + gv * (1.0f - sg)));
            gp[I + n] = dh * (gv * sg);
          } else {
            a.d_xs[(size_t)a.perm[base + m] * H + n] = acc[rt][j][nh][q];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- transposed GEMMs
// The same products as bwd_t_kernel, out[p][n] = sum_m W[e][m][n] v[p][m],
// over the 128-row items of the MFMA forward's work list, as LDS-tiled MFMA
// GEMMs: a 512-thread workgroup owns an item's 128 rows x 256 columns n; 8
// waves, each 64 rows x 64 columns as 4 x 4 MFMA 16x16x32 tiles.  Per 32-m
// stage the waves copy global -> LDS (the load unit's LDS path, no
// registers) the stage's weight fragments (2 row tiles x 8 column blocks,
// each one contiguous kilobyte of the tiled layout) into a 3-stage ring,
// two stages ahead, and the rows' fp32 v into a 2-stage ring, one stage
// ahead; a lane's A operand is its row's v, scaled and rounded to bf16 as it
// is read (hi, and lo = v - hi where HILO), its B operand (column n, m = 8g
// .. 8g+7) is read straight out of the weight fragments with transposing LDS
// reads.  The loop's LDS reads and waits are explicit (asm): the compiler
// would otherwise wait for every copy in flight before each read.  The
// operands, the lanes' m assignment and the m order are those of
// bwd_t_kernel, so every output is the same bits as there: a row's gradient
// does not depend on the batch.  Epilogues as in bwd_t_kernel.
constexpr int kBgBN = 256;                       // output columns per workgroup
constexpr int kBgWaves = 8;
constexpr int kBgThreads = 64 * kBgWaves;
constexpr int kBgWFrags = 2 * (kBgBN / 32);      // weight fragments per stage
constexpr int kBgVFrags = kMfmaTile / 16;        // v fragments per stage (hi or lo)
constexpr int kBgWLoads = kBgWFrags / kBgWaves;  // weight fragments per wave per stage
static_assert(kMfmaTile == 128 && kBgWFrags % kBgWaves == 0, "transposed GEMM tiles");

constexpr int kBgWRing = 3;                      // weight stages in LDS (two in flight)
constexpr int kBgWStage = kBgWFrags * 1024;      // weight bytes per stage
constexpr int kBgVStage = kMfmaTile * 32 * 4;    // v bytes per stage: 128 rows x 32 m, fp32
constexpr int kBgLds = kBgWRing * kBgWStage + 2 * kBgVStage;  // two v stages (one in flight)
constexpr int kBgVLoads = kBgVStage / 1024 / kBgWaves;        // v copies per wave per stage
typedef __attribute__((address_space(3))) void bg_lds_t;
// s_waitcnt vmcnt(n) with the other counters left free (vmcnt[3:0] |
// expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
#define BG_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// LDS accesses of the transposed GEMM's loop, in asm: the compiler cannot
// tell which LDS bytes the LDS-DMA copies in flight write, and waits for all
// of them before any LDS access it emits itself.  Ordering comes from the
// explicit waits and barriers of the loop.
__device__ __forceinline__ uint32_t bg_lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
// the four transposed B operands of a stage (two 8-byte transposing reads
// each, 64 bytes apart), waited for in the same asm block
__device__ __forceinline__ void bg_read_tr(const unsigned char* wb, const int (&tr)[4], u32x4_t (&bop)[4]) {
  u32x2_t r[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:64\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(bg_lds_addr(wb + tr[0])), "v"(bg_lds_addr(wb + tr[1])), "v"(bg_lds_addr(wb + tr[2])),
        "v"(bg_lds_addr(wb + tr[3]))
      : "memory");
#pragma unroll
  for (int t = 0; t < 4; ++t) bop[t] = u32x4_t{r[2 * t][0], r[2 * t][1], r[2 * t + 1][0], r[2 * t + 1][1]};
}

template <int MODE, bool LORA, bool HILO>
__global__ __launch_bounds__(kBgThreads) void bwd_gemm_kernel(BwdArgs a) {
  constexpr bool kHiLo = HILO && MODE == kDown;
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_dyn[];
  const int I = a.I, H = a.H;
  const int ncols = MODE == kDown ? I : H;      // n
  const int nrows = MODE == kDown ? H : 2 * I;  // m
  const int nkb = ncols / 32;                   // 32-column blocks of a row tile
  const int ntile = (ncols + kBgBN - 1) / kBgBN;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  if (item >= *a.n_items) return;
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int cnt = a.counts[e] - m0;
  const int M = cnt < kMfmaTile ? cnt : kMfmaTile, base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // the wave's 64 rows x 64 columns
  const int nsteps = nrows / 32;
  const int n0 = nt * kBgBN;
  const uint16_t* W = MODE == kDown ? a.w_down : a.w_gate_up;
  const size_t rt0 = (size_t)e * (nrows / 16);

  // weights: this wave's fragments f = kBgWLoads * wave + i of a stage (row
  // tile f / 8 of the stage, column block f % 8 of the window; blocks past
  // ncols load the last valid block, whose columns are never stored), copied
  // global -> LDS by the load unit (lane j's 16 bytes to fragment byte 16 j)
  const uint16_t* wsrc[kBgWLoads];
#pragma unroll
  for (int i = 0; i < kBgWLoads; ++i) {
    const int f = kBgWLoads * wave + i;
    const int kb = min(n0 / 32 + (f & 7), nkb - 1);
    wsrc[i] = W + ((rt0 + (f >> 3)) * nkb + kb) * 512 + lane * 8;
  }
  const size_t wstep = (size_t)2 * nkb * 512;  // elements per 32-m stage (two row tiles)
  auto wring = [&](int st) { return s_dyn + (st % kBgWRing) * kBgWStage; };
  auto vbuf = [&](int st) { return s_dyn + kBgWRing * kBgWStage + (st & 1) * kBgVStage; };
  // the copies of stage st into its ring slot; past the last stage, the last
  // stage's weights again into the slot of stage st, which no later stage reads
  // (so every stage issues the same number of copies and the counts stay exact)
  auto issue_w = [&](int st) {
    const int src = min(st, nsteps - 1);
#pragma unroll
    for (int i = 0; i < kBgWLoads; ++i)
      __builtin_amdgcn_global_load_lds(wsrc[i] + src * wstep, (bg_lds_t*)(wring(st) + (kBgWLoads * wave + i) * 1024),
                                       16, 0, 0);
  };
  // v rows (fp32: w d_out[token] or (d_g, d_u)), copied global -> LDS like the
  // weights: 16-byte slot s of a stage holds chunk (s & 7) ^ sw(row) of row
  // s >> 3 (m = 4 chunk .. +3), sw(row) = bits 1-2 of the row, so a lane's
  // two 16-byte reads of one row (row r of a tile, chunks 2g, 2g + 1) meet
  // no bank conflicts over 8 consecutive rows.  Rows past the item copy row
  // 0 and are scaled by 0.
  // The gate/up pass instead copies (d_g, d_u) as the down pass rounded
  // them to bf16 (the operand it would form, so the same bits): 64 bytes
  // per row and stage, slot 4 row + c holding chunk xchunk(row, c), the
  // MFMA operand order of the prefill GEMMs' token tiles, read at xslot.
  constexpr bool kVb = MODE == kGateUp;
  constexpr int kVLoads = kVb ? kBgVStage / 2 / 1024 / kBgWaves : kBgVLoads;  // v copies per wave per stage
  const void* vsrc[kVLoads];
#pragma unroll
  for (int j = 0; j < kVLoads; ++j) {
    const int slot = (kVLoads * wave + j) * 64 + lane;
    if constexpr (kVb) {
      const int row = slot >> 2, ch = xchunk(row & 15, slot & 3);
      const int rc = row < M ? row : 0;
      vsrc[j] = a.gub + (size_t)(base + rc) * 2 * I + 8 * ch;
    } else {
      const int row = slot >> 3, ch = (slot & 7) ^ ((row >> 1) & 3);
      const int rc = row < M ? row : 0;
      const float* rp;
      if (MODE == kDown)
        rp = a.d_out + (size_t)(a.perm[base + rc] / a.k) * H;
      else
        rp = a.gu + (size_t)(base + rc) * 2 * I;
      vsrc[j] = rp + 4 * ch;
    }
  }
  auto issue_v = [&](int st) {
    const int src = min(st, nsteps - 1);
#pragma unroll
    for (int j = 0; j < kVLoads; ++j) {
      const void* gsrc = kVb ? (const void*)(static_cast<const uint16_t*>(vsrc[j]) + 32 * src)
                             : (const void*)(static_cast<const float*>(vsrc[j]) + 32 * src);
      __builtin_amdgcn_global_load_lds(gsrc, (bg_lds_t*)(vbuf(st) + (kVLoads * wave + j) * 1024), 16, 0, 0);
    }
  };
  // the scale of this lane's A-operand row in each of the wave's row tiles
  const int r_ = lane & 15, g_ = lane >> 4;
  float vw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 64 + 16 * i + r_;
    vw[i] = row < M ? (MODE == kDown ? a.wts[a.perm[base + row]] : 1.f) : 0.f;
  }
  // byte offsets of the lane's two chunks of row 16 i + r_ (of the wave's 64)
  int voff[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 64 + 16 * i + r_;
#pragma unroll
    for (int c = 0; c < 2; ++c) voff[i][c] = (row * 8 + ((2 * g_ + c) ^ ((row >> 1) & 3))) * 16;
  }
  // transposing reads of the weight fragments: lane (s, G) supplies row
  // 8G + (s >> 2) (row tile G >> 1 of the stage, row (8G + (s >> 2)) & 15 in
  // it) and 4 columns from 16 (t & 1) + 4 (s & 3) of column block t >> 1 of
  // the wave's window (element (16 g' + r') * 8 + 4 h of the fragment)
  const int s_ = lane & 15, G = lane >> 4;
  const int rloc = (8 * G + (s_ >> 2)) & 15, rtl = G >> 1;
  int tr_byte[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kbw = 2 * wn + (t >> 1);  // column block within the window
    const int gq = 2 * (t & 1) + ((s_ & 3) >> 1), h = s_ & 1;
    tr_byte[t] = (rtl * 8 + kbw) * 1024 + (16 * gq + rloc) * 16 + 8 * h;
  }
  const int nj = min(max((M - wm * 64 + 15) / 16, 0), 4);  // the wave's row tiles holding rows of the item
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // issue order W(0), v(0), W(1), then per stage v(st + 1), W(st + 2): at the
  // top of stage st only W(st + 1)'s copies may still be in flight
  issue_w(0);
  issue_v(0);
  issue_w(1);
  for (int st = 0; st < nsteps; ++st) {
    __builtin_amdgcn_s_waitcnt(BG_VMCNT(kBgWLoads));
    // every wave's copies of stage st are in LDS, and every wave is done with
    // stage st - 1 (whose v buffer v(st + 1) and weight slot W(st + 2) reuse)
    asm volatile("s_barrier" ::: "memory");
    issue_v(st + 1);
    issue_w(st + 2);
    if (nj > 0) {
      const unsigned char* wb = wring(st);
      const unsigned char* vb = vbuf(st);
      u32x4_t bop[4];
      bg_read_tr(wb, tr_byte, bop);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nj) break;
        u32x4_t ah, al;
        if constexpr (kVb) {
          ah = *reinterpret_cast<const u32x4_t*>(vb + (wm * 4 + i) * 1024 + xslot(lane) * 16);
        } else {
          // the A operand: w v rounded to bf16 (hi, and lo = w v - hi)
          const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(vb + voff[i][0]);
          const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(vb + voff[i][1]);
          const float t[8] = {vw[i] * v0[0], vw[i] * v0[1], vw[i] * v0[2], vw[i] * v0[3],
                              vw[i] * v1[0], vw[i] * v1[1], vw[i] * v1[2], vw[i] * v1[3]};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ah[q] = pack_bf16x2(t[2 * q], t[2 * q + 1]);
            if constexpr (kHiLo) al[q] = pack_bf16x2(t[2 * q] - bf16lo(ah[q]), t[2 * q + 1] - bf16hi(ah[q]));
          }
        }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          acc[i][t4] = mfma16(ah, bop[t4], acc[i][t4]);
          if constexpr (kHiLo) acc[i][t4] = mfma16(al, bop[t4], acc[i][t4]);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's LDS reads are done before the next barrier
  }
  __builtin_amdgcn_s_waitcnt(BG_VMCNT(0));  // no copy into LDS outlives the workgroup
  // lane (r, g) holds D[row 4g + q][column r] of tile (i, t): row
  // wm * 64 + 16 i + 4g + q of the item, column n0 + wn * 64 + 16 t + r
  const int r = lane & 15, g = lane >> 4;
  if constexpr (LORA) {  // s A^T z, as in bwd_t_kernel
    const float* la = (MODE == kDown ? a.la_down + (size_t)e * 16 * I : a.la_gate_up + (size_t)e * 16 * H);
    const float* zb = MODE == kDown ? a.z_down : a.z_gate_up;
    f32x4_t aq[4], zq[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = min(n0 + wn * 64 + 16 * t + r, ncols - 1);  // columns past ncols are never stored
#pragma unroll
      for (int c = 0; c < 4; ++c) aq[t][c] = la[(size_t)(4 * g + c) * ncols + n];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int prow = wm * 64 + 16 * i + r;
      zq[i] = prow < M ? ld4f(zb + (size_t)(base + prow) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // each sum is formed here, one tile at a time (the empty asm keeps the
    // compiler from sinking the adds into the conditional stores below, which
    // would hold all sixteen rank-16 tiles beside the accumulators)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        add_scaled(acc[i][t], lora_tile(zq[i], aq[t]), a.lora_scale);
        asm volatile("" : "+v"(acc[i][t]));
        __builtin_amdgcn_sched_barrier(0);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = wm * 64 + 16 * i + 4 * g + q;
      if (m >= M) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + wn * 64 + 16 * t + r;
        if (n >= ncols) continue;
        if (MODE == kDown) {
          float* gp = a.gu + (size_t)(base + m) * 2 * I;
          const float gv = gp[n], uv = gp[I + n];
          const float sg = 1.0f / (1.0f + __expf(-gv));
          const float dh = acc[i][t][q];
          const float dg = dh * uv * (sg * (1.0f + gv * (1.0f - sg))), du = dh * (gv * sg);
          gp[n] = dg;
          gp[I + n] = du;
          // the gate/up pass's A operand, rounded once here
          uint16_t* gb = a.gub + (size_t)(base + m) * 2 * I;
          gb[n] = (uint16_t)pack_bf16x2(dg, 0.f);
          gb[I + n] = (uint16_t)pack_bf16x2(du, 0.f);
        } else {
          a.d_xs[(size_t)a.perm[base + m] * H + n] = acc[i][t][q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- 4-bit transposed GEMMs
// bwd_gemm_kernel for tiled 4-bit weights, over the 128-row items of the
// 4-bit MFMA forward: the same workgroup tile (an item's 128 rows x 256
// columns n, 8 waves of 64 x 64) and the same arithmetic as bwd_t_kernel's
// 4-bit form.  Per 32-m stage the workgroup's four 16-byte code chunks (two
// row tiles x two 128-column blocks of the window) are turned into the hi
// and lo bf16 parts of their codebook entries and written to LDS as the
// weight fragments the bf16 kernel stages (the code chunk's lane order is
// the fragments' lane order), so the transposing reads are the same; the
// rows' v (w d_out or (d_g, d_u), fp32) is staged as fp32.  Each wave's 64
// columns lie in one 64-column absmax block, so its A operand is v[p][m]
// times absmax[m] of that block, rounded to bf16 (hi, and lo with HILO) by
// the wave itself, and per step the MFMAs run lo-part weights, then hi-part
// weights, then (HILO) v's lo part with the hi-part weights, into one
// accumulator: bwd_t_kernel's sequence, so a row's gradient is the same
// bits from either kernel.  Two 50 KiB stages and the code-pair table's
// copies: one workgroup per CU.
constexpr int kBqVStride = 36;                        // floats per staged v row (32 m + padding)
constexpr int kBqWBytes = kBgWFrags * 1024;           // one part (hi or lo) of a stage's weight fragments
constexpr int kBqVBytes = kMfmaTile * kBqVStride * 4;
constexpr int kBqStage = 2 * kBqWBytes + kBqVBytes;
constexpr int kBqLds = 2 * kBqStage + 256 * kLutRep * 8;

template <int MODE, bool LORA, bool HILO>
__global__ __launch_bounds__(kBgThreads) void bwd_gemm_nf4_kernel(BwdArgs a) {
  constexpr bool kHiLo = HILO && MODE == kDown;
  extern __shared__ __attribute__((aligned(1024))) unsigned char s_dyn[];
  u32x2_t* s_lut = reinterpret_cast<u32x2_t*>(s_dyn + 2 * kBqStage);
  const int I = a.I, H = a.H;
  const int ncols = MODE == kDown ? I : H;      // n
  const int nrows = MODE == kDown ? H : 2 * I;  // m
  const int nkb = ncols / 128;                  // 128-column code blocks of a row tile
  const int ntile = (ncols + kBgBN - 1) / kBgBN;
  const int item = blockIdx.x / ntile, nt = blockIdx.x - item * ntile;
  if (item >= *a.n_items) return;
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int cnt = a.counts[e] - m0;
  const int M = cnt < kMfmaTile ? cnt : kMfmaTile, base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // the wave's 64 rows x 64 columns
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = nrows / 32;
  const int n0 = nt * kBgBN;
  const size_t rt0 = (size_t)e * (nrows / 16);
  const uint8_t* Q = MODE == kDown ? a.q_down : a.q_gate_up;
  const float* SC = MODE == kDown ? a.s_down : a.s_gate_up;
  build_lut(s_lut, a.codebook, tid);
  const u32x2_t* s_lutl = lut_copy(s_lut, lane);

  // codes: wave w decodes dwords 2 (w & 1), +1 of chunk w >> 1, which is
  // row tile (w >> 1) >> 1 of the stage and 128-column block (w >> 1) & 1 of
  // the window (blocks past ncols decode the last valid block, whose columns
  // are never stored); dword st of a chunk is the fragment of 32-column
  // block 4 kb + st
  const int cw = wave >> 1, dh = wave & 1;
  const int c_rtl = cw >> 1, c_kbw = cw & 1;
  const int c_kb = min(n0 / 128 + c_kbw, nkb - 1);
  const uint8_t* csrc = Q + ((rt0 + c_rtl) * nkb + c_kb) * 1024 + lane * 16 + 8 * dh;
  const size_t cstep = (size_t)2 * nkb * 1024;  // bytes per 32-m stage (two row tiles)
  // v rows: thread t brings row p = t / 4, m = 8 (t % 4) .. +7 of each stage
  const int vp = tid >> 2, vg = tid & 3;
  const int vpc = vp < M ? vp : 0;
  const float* vrow;
  float vw;
  if (MODE == kDown) {
    const int slot = a.perm[base + vpc];
    vrow = a.d_out + (size_t)(slot / a.k) * H + 8 * vg;
    vw = vp < M ? a.wts[slot] : 0.f;
  } else {
    vrow = a.gu + (size_t)(base + vpc) * 2 * I + 8 * vg;
    vw = vp < M ? 1.f : 0.f;
  }
  // absmax of this lane's rows m = 8g .. 8g+7 of a stage for the wave's
  // column block: row tile 2s + (g >> 1), rows 8 (g & 1) + i, floats 2i + h
  const int wblk = min((n0 + wn * 64) / 64, 2 * nkb - 1);  // blocks past ncols: never stored
  const int w_kb = wblk >> 1, w_h = wblk & 1;
  const float* ssrc = SC + ((rt0 + (g >> 1)) * nkb + w_kb) * 32 + 16 * (g & 1);
  const size_t sstep = (size_t)2 * nkb * 32;

  u32x2_t cd;
  f32x4_t v0, v1, s4[4];
  auto load = [&](int st) {
    cd = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(csrc + st * cstep));
    v0 = *reinterpret_cast<const f32x4_t*>(vrow + 32 * st);
    v1 = *reinterpret_cast<const f32x4_t*>(vrow + 32 * st + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) s4[j] = *reinterpret_cast<const f32x4_t*>(ssrc + st * sstep + 4 * j);
  };
  auto store = [&](int buf) {
    unsigned char* sb = s_dyn + buf * kBqStage;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      u32x4_t hi, lo;
      lut8(s_lutl, cd[d], hi, lo);
      const int f = c_rtl * 8 + 4 * c_kbw + 2 * dh + d;  // fragment (row tile, column block) of the stage
      *reinterpret_cast<u32x4_t*>(sb + f * 1024 + lane * 16) = hi;
      *reinterpret_cast<u32x4_t*>(sb + kBqWBytes + f * 1024 + lane * 16) = lo;
    }
    float* vs = reinterpret_cast<float*>(sb + 2 * kBqWBytes) + vp * kBqVStride + 8 * vg;
    *reinterpret_cast<f32x4_t*>(vs) = f32x4_t{vw * v0[0], vw * v0[1], vw * v0[2], vw * v0[3]};
    *reinterpret_cast<f32x4_t*>(vs + 4) = f32x4_t{vw * v1[0], vw * v1[1], vw * v1[2], vw * v1[3]};
  };
  // transposing reads of the weight fragments, as in bwd_gemm_kernel
  const int s_ = lane & 15, G = lane >> 4;
  const int rloc = (8 * G + (s_ >> 2)) & 15, rtl = G >> 1;
  int tr_byte[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int kbw = 2 * wn + (t >> 1);
    const int gq = 2 * (t & 1) + ((s_ & 3) >> 1), h = s_ & 1;
    tr_byte[t] = (rtl * 8 + kbw) * 1024 + (16 * gq + rloc) * 16 + 8 * h;
  }
  const int nj = min(max((M - wm * 64 + 15) / 16, 0), 4);
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto bop = [&](const unsigned char* p) {
    const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 64));
    return u32x4_t{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                   (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                   (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                   (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
  };

  __syncthreads();  // the table is built
  load(0);
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    float smc[8];  // absmax of the lane's rows m for the wave's column block
#pragma unroll
    for (int i = 0; i < 8; ++i) smc[i] = w_h ? s4[i >> 1][2 * (i & 1) + 1] : s4[i >> 1][2 * (i & 1)];
    store(buf);
    __syncthreads();  // stage st in LDS; every wave is done with stage st - 1's buffer
    if (st + 1 < nsteps) load(st + 1);  // in flight during this stage's MFMAs
    if (nj > 0) {
      const unsigned char* sb = s_dyn + buf * kBqStage;
      u32x4_t bh[4], bl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bh[t] = bop(sb + tr_byte[t]);
        bl[t] = bop(sb + kBqWBytes + tr_byte[t]);
      }
      const float* vs = reinterpret_cast<const float*>(sb + 2 * kBqWBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nj) break;
        // A operand: row p = wm * 64 + 16 i + r, m = 8g .. 8g+7, times the absmax of m
        const float* vr = vs + (wm * 64 + 16 * i + r) * kBqVStride + 8 * g;
        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(vr);
        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(vr + 4);
        const float t8[8] = {x0[0] * smc[0], x0[1] * smc[1], x0[2] * smc[2], x0[3] * smc[3],
                             x1[0] * smc[4], x1[1] * smc[5], x1[2] * smc[6], x1[3] * smc[7]};
        u32x4_t ah, al;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ah[q] = pack_bf16x2(t8[2 * q], t8[2 * q + 1]);
          if constexpr (kHiLo) al[q] = pack_bf16x2(t8[2 * q] - bf16lo(ah[q]), t8[2 * q + 1] - bf16hi(ah[q]));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[i][t] = mfma16(ah, bl[t], acc[i][t]);
          acc[i][t] = mfma16(ah, bh[t], acc[i][t]);
          if constexpr (kHiLo) acc[i][t] = mfma16(al, bh[t], acc[i][t]);
        }
      }
    }
  }
  if constexpr (LORA) {  // s A^T z, as in bwd_t_kernel
    const float* la = (MODE == kDown ? a.la_down + (size_t)e * 16 * I : a.la_gate_up + (size_t)e * 16 * H);
    const float* zb = MODE == kDown ? a.z_down : a.z_gate_up;
    f32x4_t aq[4], zq[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = min(n0 + wn * 64 + 16 * t + r, ncols - 1);  // columns past ncols are never stored
#pragma unroll
      for (int c = 0; c < 4; ++c) aq[t][c] = la[(size_t)(4 * g + c) * ncols + n];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int prow = wm * 64 + 16 * i + r;
      zq[i] = prow < M ? ld4f(zb + (size_t)(base + prow) * 16 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // each sum is formed here, one tile at a time (the empty asm keeps the
    // compiler from sinking the adds into the conditional stores below, which
    // would hold all sixteen rank-16 tiles beside the accumulators)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        add_scaled(acc[i][t], lora_tile(zq[i], aq[t]), a.lora_scale);
        asm volatile("" : "+v"(acc[i][t]));
        __builtin_amdgcn_sched_barrier(0);
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = wm * 64 + 16 * i + 4 * g + q;
      if (m >= M) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + wn * 64 + 16 * t + r;
        if (n >= ncols) continue;
        if (MODE == kDown) {
          float* gp = a.gu + (size_t)(base + m) * 2 * I;
          const float gv = gp[n], uv = gp[I + n];
          const float sg = 1.0f / (1.0f + __expf(-gv));
          const float dh = acc[i][t][q];
          gp[n] = dh * uv * (sg * (1.0f + gv * (1.0f - sg)));
          gp[I + n] = dh * (gv * sg);
        } else {
          a.d_xs[(size_t)a.perm[base + m] * H + n] = acc[i][t][q];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- weight gradients
// d_W[e][r][c] = sum_p A[p][r] B[p][c] over expert e's routed rows p in slot
// order (no atomics; zero for an expert no row reached):
//   down (before the down pass turns g, u into d_g, d_u):
//     A = d_y = w_p d_out[t_p] (r < H),  B = h = silu(g) u in fp32 (c < I)
//   gate/up (after it): A = (d_g, d_u)[p] (r < 2I),  B = x[t_p] (c < H)
// On the matrix cores: a 256-thread workgroup owns a 64 x 64 tile of one
// expert's d_W and walks the expert's rows 32 at a time (one MFMA k-step).
// Each chunk of A and B is written to LDS as [p][column] bf16 tiles and read
// back transposed (ds_read_b64_tr_b16, as in the transposed GEMVs above), so
// a lane gets 8 consecutive p of one column.  fp32 operands enter as two
// bf16 parts, hi = RNE(v) and lo = RNE(v - hi) (about 16 bits of v); x is
// bf16 and enters whole.  Products: A_lo B_hi (+ A_hi B_lo for the down
// part), then A_hi B_hi, into one fp32 accumulator per output element.  The
// next chunk's global loads are issued before this chunk's MFMAs.  The
// output is write-bound: fp32 gradients the size of all experts' weights.
constexpr int kWmR = 64, kWmC = 64, kWmP = 32;
constexpr int kWmS = 72;  // LDS row stride in elements (64 columns + padding; rows stay 16-byte aligned)

// h = silu(g) u in fp32 for every routed row (sorted-slot order), formed
// once for the down weight gradient instead of once per output tile
__global__ __launch_bounds__(256) void h_kernel(BwdArgs a, float* hf) {
  const int I = a.I;
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
  if (i4 >= (size_t)a.T * a.k * (I / 4)) return;
  const size_t p = i4 / (I / 4);
  const int n = (int)(i4 - p * (I / 4)) * 4;
  const f32x4_t gv = *reinterpret_cast<const f32x4_t*>(a.gu + p * 2 * I + n);
  const f32x4_t uv = *reinterpret_cast<const f32x4_t*>(a.gu + p * 2 * I + I + n);
  f32x4_t h;
#pragma unroll
  for (int q = 0; q < 4; ++q) h[q] = silu(gv[q]) * uv[q];
  *reinterpret_cast<f32x4_t*>(hf + p * I + n) = h;
}

// 8 fp32 -> their hi and lo bf16 parts, packed in pairs
__device__ __forceinline__ void split8(const float (&v)[8], u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    lo[i] = pack_bf16x2(v[2 * i] - bf16lo(hi[i]), v[2 * i + 1] - bf16hi(hi[i]));
  }
}

// the MFMA operand of 16 columns starting at col0: lane (r, g) gets column
// col0 + r, rows p = 8g .. 8g+7 of a [32 p][kWmS] tile
__device__ __forceinline__ u32x4_t wm_operand(const uint16_t* tile, int tr_off, int col0) {
  const uint2 lo = read_tr4(tile, tr_off + col0);
  const uint2 hi = read_tr4(tile, tr_off + 4 * kWmS + col0);
  return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

template <int PART>  // 0: down, 1: gate/up
__global__ __launch_bounds__(256) void wgrad_mfma_kernel(BwdArgs a) {
  constexpr bool kBLo = PART == 0;  // B in two parts (h fp32); x is bf16
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kWmP * kWmS];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kBLo ? 2 : 1][kWmP * kWmS];
  const int H = a.H, I = a.I;
  const int R = PART == 0 ? H : 2 * I, C = PART == 0 ? I : H;
  const int e = blockIdx.z;
  const int r0 = blockIdx.y * kWmR, c0 = blockIdx.x * kWmC;
  const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;  // the wave's 32 x 32 sub-tile
  const int rr = lane & 15, g = lane >> 4;
  const int tr_off = (8 * g + (rr >> 2)) * kWmS + 4 * (rr & 3);
  // chunk fill: thread t brings row p = chunk start + (t >> 3), columns 8 (t & 7) .. +7
  const int pl = tid >> 3, col = (tid & 7) * 8;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the chunk's raw values for this thread: A (8 fp32), B (8 fp32, or 8 bf16)
  f32x4_t ra0, ra1, rb0, rb1, rg0, rg1;
  u32x4_t rx;
  float rw = 0.f;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto fetch = [&](int pc) {
    const int p = pc + pl;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    ra0 = ra1 = rb0 = rb1 = rg0 = rg1 = z;
    rx = zero;
    rw = 0.f;
    if (p < p1) {
      if (PART == 0) {
        const int slot = a.perm[p];
        rw = a.wts[slot];
        const float* dr = a.d_out + (size_t)(slot / a.k) * H + r0 + col;
        ra0 = *reinterpret_cast<const f32x4_t*>(dr);
        ra1 = *reinterpret_cast<const f32x4_t*>(dr + 4);
        if (a.hf) {
          const float* hr = a.hf + (size_t)p * I + c0 + col;
          rb0 = *reinterpret_cast<const f32x4_t*>(hr);
          rb1 = *reinterpret_cast<const f32x4_t*>(hr + 4);
        } else {
          const float* gp = a.gu + (size_t)p * 2 * I + c0 + col;
          rb0 = *reinterpret_cast<const f32x4_t*>(gp);
          rb1 = *reinterpret_cast<const f32x4_t*>(gp + 4);
          rg0 = *reinterpret_cast<const f32x4_t*>(gp + I);
          rg1 = *reinterpret_cast<const f32x4_t*>(gp + I + 4);
        }
      } else {
        const float* gr = a.gu + (size_t)p * 2 * I + r0 + col;
        ra0 = *reinterpret_cast<const f32x4_t*>(gr);
        ra1 = *reinterpret_cast<const f32x4_t*>(gr + 4);
        rx = ld16(a.x + (size_t)(a.perm[p] / a.k) * H + c0 + col);
      }
    }
  };
  if (p0 < p1) fetch(p0);
  for (int pc = p0; pc < p1; pc += kWmP) {
    float av[8], bv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      av[q] = PART == 0 ? rw * ra0[q] : ra0[q];
      av[4 + q] = PART == 0 ? rw * ra1[q] : ra1[q];
    }
    u32x4_t ahi, alo, bhi, blo;
    split8(av, ahi, alo);
    if constexpr (PART == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bv[q] = a.hf ? rb0[q] : silu(rb0[q]) * rg0[q];
        bv[4 + q] = a.hf ? rb1[q] : silu(rb1[q]) * rg1[q];
      }
      split8(bv, bhi, blo);
    } else {
      bhi = rx;
      blo = zero;
    }
    __syncthreads();  // the previous chunk's LDS reads are done
    *reinterpret_cast<u32x4_t*>(s_a[0] + pl * kWmS + col) = ahi;
    *reinterpret_cast<u32x4_t*>(s_a[1] + pl * kWmS + col) = alo;
    *reinterpret_cast<u32x4_t*>(s_b[0] + pl * kWmS + col) = bhi;
    if constexpr (kBLo) *reinterpret_cast<u32x4_t*>(s_b[kBLo ? 1 : 0] + pl * kWmS + col) = blo;
    __syncthreads();
    if (pc + kWmP < p1) fetch(pc + kWmP);  // in flight during the MFMAs
    u32x4_t oa[2][2], ob[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      oa[i][0] = wm_operand(s_a[0], tr_off, 32 * wr + 16 * i);
      oa[i][1] = wm_operand(s_a[1], tr_off, 32 * wr + 16 * i);
      ob[i][0] = wm_operand(s_b[0], tr_off, 32 * wc + 16 * i);
      if constexpr (kBLo) ob[i][1] = wm_operand(s_b[kBLo ? 1 : 0], tr_off, 32 * wc + 16 * i);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma16(oa[i][1], ob[j][0], acc[i][j]);
        if constexpr (kBLo) acc[i][j] = mfma16(oa[i][0], ob[j][1], acc[i][j]);
        acc[i][j] = mfma16(oa[i][0], ob[j][0], acc[i][j]);
      }
  }
  // lane holds D[4g + q][r] of sub-tile (i, j): row r0 + 32 wr + 16 i + 4g + q, column c0 + 32 wc + 16 j + r
  float* o = (PART == 0 ? a.g_w_down : a.g_w_gate_up) + (size_t)e * R * C;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t row = (size_t)(r0 + 32 * wr + 16 * i + 4 * g + q);
#pragma unroll
      for (int j = 0; j < 2; ++j) o[row * C + c0 + 32 * wc + 16 * j + rr] = acc[i][j][q];
    }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdArgs a) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= a.H) return;
  float* dx = a.d_x + (size_t)t * a.H + c;
  // all k slot rows are loaded before the first add (one round trip), then
  // added in slot order
  f32x4_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < a.k) v[j] = *reinterpret_cast<const f32x4_t*>(a.d_xs + ((size_t)t * a.k + j) * a.H + c);
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(dx);
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < a.k)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += v[j][q];
  *reinterpret_cast<f32x4_t*>(dx) = acc;
}

// dynamic LDS beyond 64 KiB needs the per-function limit raised, once per device
template <int MODE, bool LORA, bool HILO>
hipError_t launch_bg(const BwdArgs& a, dim3 grid, hipStream_t s) {
  constexpr int lds = kBgLds;
  static bool done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_gemm_kernel<MODE, LORA, HILO>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    done[dev] = true;
  }
  hipLaunchKernelGGL((bwd_gemm_kernel<MODE, LORA, HILO>), grid, dim3(kBgThreads), lds, s, a);
  return hipGetLastError();
}

// dynamic LDS beyond 64 KiB needs the per-function limit raised, once per device
template <int MODE, bool LORA, bool HILO>
hipError_t launch_bq(const BwdArgs& a, dim3 grid, hipStream_t s) {
  static bool done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!done[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_gemm_nf4_kernel<MODE, LORA, HILO>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kBqLds);
    if (e != hipSuccess) return e;
    done[dev] = true;
  }
  hipLaunchKernelGGL((bwd_gemm_nf4_kernel<MODE, LORA, HILO>), grid, dim3(kBgThreads), kBqLds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_weights(const BwdArgs& a, hipStream_t s) {
  if (a.k == 8)
    hipLaunchKernelGGL(bwd_weights_kernel<8>, dim3(a.T), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bwd_weights_kernel<0>, dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_t(const BwdArgs& a, bool down, hipStream_t s) {
  const dim3 grid(a.max_items * ((down ? a.I : a.H) / 32));
  if (a.nf4) {  // frozen 4-bit base: no weight gradients
    if (a.wgrad) return hipErrorInvalidValue;
    if (a.row_tiles == kMfmaTile / 16) {  // the 4-bit MFMA forward's 128-row items
      const dim3 gg(a.max_items * (((down ? a.I : a.H) + kBgBN - 1) / kBgBN));
      if (down && a.lora) return launch_bq<kDown, true, true>(a, gg, s);
      if (down) return launch_bq<kDown, false, false>(a, gg, s);
      if (a.lora) return launch_bq<kGateUp, true, false>(a, gg, s);
      return launch_bq<kGateUp, false, false>(a, gg, s);
    }
    if (a.row_tiles != 1) return hipErrorInvalidValue;
    if (down) {
      if (a.lora)
        hipLaunchKernelGGL((bwd_t_kernel<kDown, true, true, true>), grid, dim3(64), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_t_kernel<kDown, false, false, true>), grid, dim3(64), 0, s, a);
    } else {
      if (a.lora)
        hipLaunchKernelGGL((bwd_t_kernel<kGateUp, true, false, true>), grid, dim3(64), 0, s, a);
      else
        hipLaunchKernelGGL((bwd_t_kernel<kGateUp, false, false, true>), grid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
  }
  if (a.row_tiles == kMfmaTile / 16) {  // the MFMA forward's 128-row items
    const dim3 gg(a.max_items * (((down ? a.I : a.H) + kBgBN - 1) / kBgBN));
    const bool hl = down && (a.lora || a.wgrad);
    hipError_t e;
    if (down && a.lora) e = launch_bg<kDown, true, true>(a, gg, s);
    else if (down && hl) e = launch_bg<kDown, false, true>(a, gg, s);
    else if (down) e = launch_bg<kDown, false, false>(a, gg, s);
    else if (a.lora) e = launch_bg<kGateUp, true, false>(a, gg, s);
    else e = launch_bg<kGateUp, false, false>(a, gg, s);
    return e;
  }
  if (a.row_tiles != 1) return hipErrorInvalidValue;
  if (down) {
    if (a.lora)
      hipLaunchKernelGGL((bwd_t_kernel<kDown, true, true>), grid, dim3(64), 0, s, a);
    else if (a.wgrad)
      hipLaunchKernelGGL((bwd_t_kernel<kDown, false, true>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_t_kernel<kDown, false, false>), grid, dim3(64), 0, s, a);
  } else {
    if (a.lora)
      hipLaunchKernelGGL((bwd_t_kernel<kGateUp, true, false>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_t_kernel<kGateUp, false, false>), grid, dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_h(const BwdArgs& a, float* hf, hipStream_t s) {
  const size_t n4 = (size_t)a.T * a.k * (a.I / 4);
  hipLaunchKernelGGL(h_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a, hf);
  return hipGetLastError();
}

hipError_t launch_wgrad(const BwdArgs& a, bool down, hipStream_t s) {
  const int R = down ? a.H : 2 * a.I, C = down ? a.I : a.H;
  if (R % kWmR || C % kWmC) return hipErrorInvalidValue;
  const dim3 grid(C / kWmC, R / kWmR, a.E);
  if (down)
    hipLaunchKernelGGL(wgrad_mfma_kernel<0>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(wgrad_mfma_kernel<1>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_combine(const BwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(a.T, (a.H + 1023) / 1024), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
