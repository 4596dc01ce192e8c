// Router for gfx950: logits -> top-k (ties to the lower expert index) ->
// renormalised softmax weights.
//
// The block's router is a linear map to fp32 logits followed by softmax,
// top-k and renormalisation; its pointwise tail is what the compiled walker
// fused (unsloth commit a1bc5cbd page, first paragraph).  The decision (which
// k experts, in which order) is taken on the correctly rounded fp32 logit of
// each expert, so that it is reproducible bit for bit.  Two kernels:
//
//   route_partial  bf16 MFMA (fp32 accumulate) over a K slice: partial
//            approximate logits a and, from the same operands with the sign
//            bits cleared, partial S = sum_h |x_h * w_h|.  The grid is
//            (16-token tiles) x (K splits), so at decode sizes the router
//            weights are read by many CUs in parallel instead of by a few.
//   route_select  one wave per token.  Partials are summed in split order.
//            An fp32 sum along a chain of d additions errs by at most
//            d * 2^-24 * S, so |a - l| <= beta = gamma * S + (rounding of the
//            fp32 result and of the bias add), gamma covering the longest
//            chain with a factor-2 margin.  L = k-th largest lower bound
//            a - beta (a ballot radix select over order-preserving keys).
//            Any expert with a + beta < L is beaten strictly by k others, so
//            the true top-k lies within C = {e : a + beta >= L}.  A candidate
//            whose interval [a - beta, a + beta] meets no other candidate's
//            is ordered against every other one by its approximate value; the
//            dot products of the candidates whose intervals overlap are
//            re-formed in fp64 from the exact bf16 products, rounded to fp32
//            (plus the fp32 bias).  The top-k of C by (value desc, index asc)
//            over these values is the top-k of all experts.
//
// Softmax weights w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), fp32, j in
// selection order (equal to the full softmax renormalised over the top k);
// or, for the un-renormalised form, the same numerators over the sum across
// all E experts.
#include <float.h>
#include <limits.h>

#include <cstring>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kTok = 16;        // MFMA column block = tokens per partial tile
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kMaxCand = 64;    // candidates held one per lane; more -> all-expert path
constexpr int kMaxSplit = 16;   // K splits of the partial pass

// ------------------------------------------------------------------ partials
struct PartParams {
  const uint16_t* x;
  const uint16_t* wr;
  int T, H, E, ks;
  int per_wg;    // K splits summed inside one workgroup (1, or ks at large T)
  float* part;   // [ks / per_wg][T][E] partial logits
  float* pabs;   // [ks / per_wg][T][E] partial sums of |x*w|
  // pre-block step (PN kernels only): the token operand is formed on the fly
  // as x = bf16(r * scale * gamma), r = bf16(res + delta), and written out
  const uint16_t* res;    // bf16 [T][H]
  const uint16_t* delta;  // bf16 [T][H], or null (r = res)
  const uint16_t* gamma;  // bf16 [H]
  float eps;
  uint16_t* res_out;      // bf16 [T][H] (r), or null
  uint16_t* x_out;        // bf16 [T][H] (x)
  // graph replays: the live row count.  Rows >= live_rows are not written
  // (PN); workgroup (0, 0) stores live_rows to *live_out, where the later
  // kernels of the step read it.  Eager calls: live_out null, live_rows = T.
  int live_rows;
  int32_t* live_out;
};

__device__ __forceinline__ float round_bf16(float v) { return bf16lo(pack_bf16x2(v, 0.f)); }

// r = bf16(res + delta) for the 8 elements of one chunk (the fp32 sum of two
// bf16 values rounds to bf16 exactly as their exact sum does)
__device__ __forceinline__ void residual8(u32x4_t rv, u32x4_t dv, float (&r)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[2 * q] = round_bf16(bf16lo(rv[q]) + bf16lo(dv[q]));
    r[2 * q + 1] = round_bf16(bf16hi(rv[q]) + bf16hi(dv[q]));
  }
}

// Pre-block step, first part: 1 / sqrt(mean_h r^2 + eps) of the workgroup's
// 16 rows into s_scale.  16 threads per row; thread i of a row sums r^2 over
// chunks i, i + 16, ... (8 elements each, in order, fp32 fma), then a
// butterfly over the 16 adds the partial sums.  Every workgroup that covers a
// row gets the same bits.  Rows past T get 0.
__device__ __forceinline__ void prenorm_scales(const PartParams& p, int t0, float* s_scale) {
  constexpr int kPass = 16;  // chunks per thread per pass (one load round trip)
  const int tid = threadIdx.x, rl = tid >> 4, sub = tid & 15;
  const int row = t0 + rl;
  const int nch = p.H >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  float ss = 0.f;
  if (row < p.T) {
    const uint16_t* rr = p.res + (size_t)row * p.H;
    const uint16_t* dr = p.delta ? p.delta + (size_t)row * p.H : nullptr;
    for (int c0 = 0; c0 < nch; c0 += 16 * kPass) {
      u32x4_t rv[kPass], dv[kPass];
#pragma unroll
      for (int j = 0; j < kPass; ++j) {
        const int c = c0 + sub + 16 * j;
        rv[j] = c < nch ? ld16(rr + 8 * c) : zero;
        dv[j] = (dr && c < nch) ? ld16(dr + 8 * c) : zero;
      }
#pragma unroll
      for (int j = 0; j < kPass; ++j) {
        float r[8];
        residual8(rv[j], dv[j], r);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(r[i], r[i], ss);
      }
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (sub == 0) s_scale[rl] = row < p.T ? 1.0f / sqrtf(ss / (float)p.H + p.eps) : 0.f;
  __syncthreads();
}

// Pre-block step, second part: one token fragment (8 elements of row r of
// the tile at k = kk + 8g) -> x fragment, r returned in rout.
__device__ __forceinline__ u32x4_t prenorm_x8(u32x4_t rv, u32x4_t dv, u32x4_t gv, float sc, u32x4_t& rout) {
  float r[8];
  residual8(rv, dv, r);
  u32x4_t xo;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    xo[q] = pack_bf16x2(r[2 * q] * sc * bf16lo(gv[q]), r[2 * q + 1] * sc * bf16hi(gv[q]));
    rout[q] = pack_bf16x2(r[2 * q], r[2 * q + 1]);
  }
  return xo;
}

// Wave w owns expert tiles w, w+4, ...; every wave walks the workgroup's
// whole K range, so no cross-wave reduction is needed.  U k-steps of loads
// are in flight before the MFMAs consume them.  A workgroup covers per_wg
// consecutive K splits: each split is its own MFMA accumulation chain and
// the split sums are added in split order, exactly as route_select adds
// stored split partials, so both forms give the same bits.  PN: the token
// operand comes from the pre-block step (prenorm_scales / prenorm_x8); wave
// 0 writes the fragments it forms to x_out and res_out, so every element of
// a live row is written by exactly one workgroup.
template <int NT, int U, bool PN>  // NT: expert tiles per wave (>= ceil(E/64)); U: k-steps per batch
__global__ __launch_bounds__(256) void route_partial(PartParams p) {
  __shared__ float s_scale[PN ? kTok : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kTok;
  const int H = p.H, E = p.E, T = p.T;
  const int n_et = E >> 4;
  const int klen = H / p.ks;
  const int trow = t0 + r;
  const bool tv = trow < T;
  const uint16_t* pb0 = (PN ? p.res : p.x) + (size_t)(tv ? trow : 0) * H + g * 8;
  const uint16_t* pd0 = PN && p.delta ? p.delta + (size_t)(tv ? trow : 0) * H + g * 8 : nullptr;
  const uint16_t* pg0 = PN ? p.gamma + g * 8 : nullptr;
  float sc = 0.f;
  bool wr_out = false;
  if constexpr (PN) {
    prenorm_scales(p, t0, s_scale);
    sc = s_scale[r];
    wr_out = wave == 0 && tv && trow < p.live_rows;
  }
  if (p.live_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.live_out = p.live_rows;
  const uint16_t* pa0 = p.wr + (size_t)(wave * 16 + r) * H + g * 8;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  const uint32_t absm = 0x7fff7fffu;
  f32x4_t lsum[NT], ssum[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    lsum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ssum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // the workgroup's K range is per_wg consecutive splits; batches of U
  // k-steps are software-pipelined (the next batch's loads are in flight
  // while this batch is multiplied), and at the end of each split its
  // accumulators are added to the running sums
  const int kbase = blockIdx.y * p.per_wg * klen;
  const int nbatch = p.per_wg * klen / (32 * U);
  const int bps = klen / (32 * U);  // batches per split
  const uint16_t* pb = pb0 + kbase;
  const uint16_t* pd = pd0 ? pd0 + kbase : nullptr;
  const uint16_t* pg = PN ? pg0 + kbase : nullptr;
  const uint16_t* pa = pa0 + kbase;
  f32x4_t acc[NT], aab[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    aab[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  u32x4_t b[U], av[U][NT];
  u32x4_t db[PN ? U : 1], gb[PN ? U : 1];
  auto load = [&](int j) {
    const int kk = j * 32 * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      b[u] = tv ? ld16(pb + kk + 32 * u) : zero;
      if constexpr (PN) {
        db[u] = (tv && pd) ? ld16(pd + kk + 32 * u) : zero;
        gb[u] = ld16(pg + kk + 32 * u);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i)
        av[u][i] = (wave + 4 * i < n_et) ? ld16(pa + (size_t)i * 64 * H + kk + 32 * u) : zero;
    }
  };
  load(0);
  for (int j = 0; j < nbatch; ++j) {
    u32x4_t bc[U], ac[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (PN) {
        u32x4_t rr;
        bc[u] = prenorm_x8(b[u], db[u], gb[u], sc, rr);
        if (wr_out) {
          const size_t o = (size_t)trow * H + g * 8 + kbase + j * 32 * U + 32 * u;
          *reinterpret_cast<u32x4_t*>(p.x_out + o) = bc[u];
          if (p.res_out) *reinterpret_cast<u32x4_t*>(p.res_out + o) = rr;
        }
      } else {
        bc[u] = b[u];
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) ac[u][i] = av[u][i];
    }
    if (j + 1 < nbatch) load(j + 1);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4_t babs = bc[u] & absm;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        acc[i] = mfma16(ac[u][i], bc[u], acc[i]);
        aab[i] = mfma16(ac[u][i] & absm, babs, aab[i]);
      }
    }
    if ((j + 1) % bps == 0) {  // end of a split
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        lsum[i] += acc[i];
        ssum[i] += aab[i];
        acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        aab[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // lane holds D[4g+q][r]: expert 16*(wave + 4i) + 4g + q, token r
  if (tv) {
    float* dl = p.part + ((size_t)blockIdx.y * T + trow) * E;
    float* ds = p.pabs + ((size_t)blockIdx.y * T + trow) * E;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (wave + 4 * i < n_et) {
        const int e0 = 16 * (wave + 4 * i) + 4 * g;
        *reinterpret_cast<f32x4_t*>(dl + e0) = lsum[i];
        *reinterpret_cast<f32x4_t*>(ds + e0) = ssum[i];
      }
  }
}

// The same partials with the operands staged through LDS (plain token
// rows, no pre-block step): each wave copies, per 32-k step, its token tile
// and its NT expert tiles (16 rows x 64 bytes each) global -> LDS with
// global_load_lds_dwordx4, four lanes per 64-byte row segment (xchunk
// order), into a private ring of RS steps, RS - 1 of them in flight; then
// reads its MFMA operands from the xslot positions.  Loaded directly, each
// lane's 16 bytes come from another row, a pattern the load unit serves
// about half as fast.  The operands each lane receives, the MFMA sequence and
// the split sums are those of route_partial, so the partials are the same
// bits.  Tiles past E copy tile 0 and are never stored.
typedef __attribute__((address_space(3))) char lds_char_t;
#define MOE_R_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

template <int L, int RS>
__device__ __forceinline__ void route_wait(int later) {  // at most `later` steps of L loads still in flight
  static_assert(RS <= 8 && L * (RS - 2) < 64, "wait counts");
  switch (later) {
    case 0: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(L)); break;
    case 2: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(2 * L)); break;
    case 3: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(3 * L)); break;
    case 4: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(4 * L)); break;
    case 5: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(5 * L)); break;
    default: __builtin_amdgcn_s_waitcnt(MOE_R_VMCNT(6 * L)); break;
  }
  asm volatile("" ::: "memory");  // the LDS reads of the step stay below
}

// W waves per workgroup (4, or 8 where one workgroup sums all K splits of
// its tokens and the token tiles alone give one workgroup per CU); wave w
// owns expert tiles w, w + W, ...
template <int W, int NT>
constexpr int route_ring() {
  return W == 4 ? (NT == 1 ? 6 : (NT == 2 ? 5 : 3)) : (NT == 1 ? 3 : 2);  // within 60 KiB of static LDS
}

template <int NT, int W = 4>
__global__ __launch_bounds__(64 * W) void route_partial_lds(PartParams p) {
  constexpr int L = 1 + NT;  // copies per wave per step: the token tile, then its expert tiles
  constexpr int RS = route_ring<W, NT>();  // ring steps
  static_assert(W * RS * L <= 60, "static LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char s_ring[W][RS][L][1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int t0 = blockIdx.x * kTok;
  const int H = p.H, E = p.E, T = p.T;
  const int n_et = E >> 4;
  const int klen = H / p.ks;
  const int trow = t0 + r;
  const bool tv = trow < T;
  if (p.live_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *p.live_out = p.live_rows;
  // copy lanes: lane 4q + c brings row q of a tile, k chunk xchunk(q, c) of each step
  const int q = lane >> 2, cc = xchunk(q, lane & 3);
  const int kbase = blockIdx.y * p.per_wg * klen;
  const uint16_t* xs = p.x + (size_t)min(t0 + q, T - 1) * H + kbase + cc * 8;  // rows past T: never stored
  const uint16_t* ws = p.wr + (size_t)q * H + kbase + cc * 8;  // row q of expert tile 0
  const int nsteps = p.per_wg * klen / 32;
  const int sps = klen / 32;  // steps per split
  auto issue = [&](int st) {
    lds_char_t* sb = (lds_char_t*)&s_ring[wave][st % RS][0][0];
    __builtin_amdgcn_global_load_lds(xs + st * 32, sb, 16, 0, 0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int et = wave + W * i < n_et ? wave + W * i : 0;
      __builtin_amdgcn_global_load_lds(ws + (size_t)et * 16 * H + st * 32, sb + (1 + i) * 1024, 16, 0, 0);
    }
  };
  const int xo = xslot(lane) * 16;
  const uint32_t absm = 0x7fff7fffu;
  f32x4_t lsum[NT], ssum[NT], acc[NT], aab[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) lsum[i] = ssum[i] = acc[i] = aab[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < RS - 1; ++st)
    if (st < nsteps) issue(st);
  for (int st = 0; st < nsteps; ++st) {
    route_wait<L, RS>(min(RS - 2, nsteps - 1 - st));  // step st has landed
    if (st + RS - 1 < nsteps) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads of the buffer it overwrites are done
      issue(st + RS - 1);
    }
    // tiles past E (copies of tile 0) are multiplied too and never stored
    const unsigned char* sb = &s_ring[wave][st % RS][0][0];
    u32x4_t av[NT];
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(sb + xo);
#pragma unroll
    for (int i = 0; i < NT; ++i) av[i] = *reinterpret_cast<const u32x4_t*>(sb + (1 + i) * 1024 + xo);
    const u32x4_t babs = b & absm;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      acc[i] = mfma16(av[i], b, acc[i]);
      aab[i] = mfma16(av[i] & absm, babs, aab[i]);
    }
    if ((st + 1) % sps == 0) {  // end of a split
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        lsum[i] += acc[i];
        ssum[i] += aab[i];
        acc[i] = aab[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  // lane holds D[4g+q][r]: expert 16*(wave + W i) + 4g + q, token r
  if (tv) {
    const int g = lane >> 4;
    float* dl = p.part + ((size_t)blockIdx.y * T + trow) * E;
    float* ds = p.pabs + ((size_t)blockIdx.y * T + trow) * E;
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (wave + W * i < n_et) {
        const int e0 = 16 * (wave + W * i) + 4 * g;
        *reinterpret_cast<f32x4_t*>(dl + e0) = lsum[i];
        *reinterpret_cast<f32x4_t*>(ds + e0) = ssum[i];
      }
  }
}

// ------------------------------------------------------------------ select
struct SelParams {
  RouteArgs a;
  const float* part;
  const float* pabs;
  int ks;
  float gamma;
  PermuteArgs pa;  // the fused bucketing of small batches (route_select<..., true>)
};

// Butterfly sum: partners add the same two values, so every lane ends with
// the bit-identical total.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ double dot8_f64(u32x4_t xa, u32x4_t wa, double s) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s = fma((double)bf16lo(xa[q]), (double)bf16lo(wa[q]), s);
    s = fma((double)bf16hi(xa[q]), (double)bf16hi(wa[q]), s);
  }
  return s;
}

__device__ __forceinline__ float readlane_f(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// key f beats key e: larger value, or equal value and lower index
__device__ __forceinline__ int beats(float vf, int f, float ve, int e) {
  return (vf > ve || (vf == ve && f < e)) ? 1 : 0;
}

// order-preserving map float -> uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float okey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// exact (fp64-formed, fp32-rounded, + fp32 bias) logit of expert e for x row xr
template <int CH>
__device__ __forceinline__ float exact_logit(const u32x4_t (&xc)[CH], const RouteArgs& a, int e, int lane) {
  const int nch = a.H >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t wc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = lane + 64 * i;
    wc[i] = c < nch ? ld16(a.wr + (size_t)e * a.H + c * 8) : zero;
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < CH; ++i) s = dot8_f64(xc[i], wc[i], s);
  s = wave_sum_f64(s);
  float le = (float)s;
  if (a.bias) le = le + a.bias[e];
  return le;
}

template <int NW>  // waves (tokens) per workgroup
struct SelShared {
  float v[NW][kMaxCand];
  int e[NW][kMaxCand];
  float selv[NW][kMaxK];
  int sele[NW][kMaxK];
  __attribute__((aligned(16))) float key[NW][kMaxE];
};

// One wave selects token t (t < T).  NS: the number of stored split
// partials when it is known at compile time (their loads are then issued
// back to back, unpredicated), or 0 (P.ks).
template <int M, int CH, int NS, int NW>  // M = ceil(E / 64) experts per lane; CH = ceil(H / 512) row chunks per lane
__device__ __forceinline__ void select_token(const SelParams& P, int t, int wave, int lane, SelShared<NW>& sh) {
  float (&s_v)[NW][kMaxCand] = sh.v;
  int (&s_e)[NW][kMaxCand] = sh.e;
  float (&s_selv)[NW][kMaxK] = sh.selv;
  int (&s_sele)[NW][kMaxK] = sh.sele;
  float (&s_key)[NW][kMaxE] = sh.key;
  const RouteArgs& a = P.a;
  const int T = a.T, E = a.E, k = a.k;

  float av[M], bd[M];
  uint32_t key[M];
  // all split partials are loaded before any is added (one round trip)
  constexpr int kS = NS > 0 ? NS : kMaxSplit;
  const int nsp = NS > 0 ? NS : P.ks;
  float pl[M][kS], ps[M][kS];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    const int ec = e < E ? e : E - 1;  // lanes past E read a valid element, never used
#pragma unroll
    for (int ks = 0; ks < kS; ++ks) {
      if (NS > 0) {
        pl[m][ks] = P.part[((size_t)ks * T + t) * E + ec];
        ps[m][ks] = P.pabs[((size_t)ks * T + t) * E + ec];
      } else {
        const bool ok = e < E && ks < nsp;
        pl[m][ks] = ok ? P.part[((size_t)ks * T + t) * E + e] : 0.f;
        ps[m][ks] = ok ? P.pabs[((size_t)ks * T + t) * E + e] : 0.f;
      }
    }
  }
  if (a.live && t >= *a.live) return;  // row past the live count of a graph replay
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    av[m] = -INFINITY;
    bd[m] = 0.f;
    key[m] = 0u;
    if (e < E) {
      float l = 0.f, s = 0.f;
#pragma unroll
      for (int ks = 0; ks < kS; ++ks) {
        if (ks < nsp) {
          l += pl[m][ks];
          s += ps[m][ks];
        }
      }
      const float bv = a.bias ? a.bias[e] : 0.f;
      av[m] = a.bias ? l + bv : l;
      bd[m] = P.gamma * s + 2.5e-7f * (fabsf(l) + fabsf(bv)) + 1e-30f;
      key[m] = okey(av[m] - bd[m]);
    }
  }
  // L = k-th largest lower bound (radix select, most significant bit first)
  uint32_t theta = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t trial = theta | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) cnt += __popcll(__ballot(key[m] >= trial));
    if (cnt >= k) theta = trial;
  }
  const float L = okey_inv(theta);

  bool cand[M];
  int ncand = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    cand[m] = e < E && av[m] + bd[m] >= L;
    const uint64_t mask = __ballot(cand[m]);
    if (cand[m]) {
      const int slot = ncand + __popcll(mask & ((1ull << lane) - 1ull));
      if (slot < kMaxCand) {
        s_v[wave][slot] = av[m];
        s_e[wave][slot] = e;
      }
    }
    ncand += __popcll(mask);
  }
  wave_sync_lds();

  const int nch = a.H >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  if (ncand <= kMaxCand) {
    // candidate i lives in lane i
    const bool mine = lane < ncand;
    float cv = mine ? s_v[wave][lane] : -INFINITY;
    const int ce = mine ? s_e[wave][lane] : INT_MAX;
    float cb = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float bm = __shfl(bd[m], ce & 63);  // bound of expert ce (held by lane ce % 64)
      if (mine && (ce >> 6) == m) cb = bm;
    }
    // Interval of candidate i: [cv - cb, cv + cb] holds its exact logit.  A
    // candidate whose interval meets no other candidate's is ordered against
    // every other one by its approximate value; only candidates whose
    // intervals overlap get the exact value re-formed (typically two).
    // (candidate j's values are read from its lane: uniform j, no LDS round trip)
    const float lo = cv - cb, hi = cv + cb;
    bool need = false;
    for (int j = 0; j < ncand; ++j) {
      const float loj = readlane_f(lo, j), hij = readlane_f(hi, j);
      need |= mine && j != lane && loj <= hi && lo <= hij;
    }
    uint64_t rmask = __ballot(need);
    if (rmask) {
      u32x4_t xc[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = lane + 64 * i;
        xc[i] = c < nch ? ld16(a.x + (size_t)t * a.H + c * 8) : zero;
      }
      constexpr int NB = CH >= 8 ? 2 : (CH >= 4 ? 4 : 8);  // rows per batch (loads in flight: NB * CH)
      while (rmask) {
        int lj[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          lj[b] = rmask ? __builtin_ctzll(rmask) : -1;  // candidate lane
          if (rmask) rmask &= rmask - 1;
        }
        u32x4_t wc[NB][CH];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int ej = lj[b] >= 0 ? __builtin_amdgcn_readlane(ce, lj[b]) : -1;
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            const int c = lane + 64 * i;
            wc[b][i] = (ej >= 0 && c < nch) ? ld16(a.wr + (size_t)ej * a.H + c * 8) : zero;
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (lj[b] >= 0) {
            double sd = 0.0;
#pragma unroll
            for (int i = 0; i < CH; ++i) sd = dot8_f64(xc[i], wc[b][i], sd);
            sd = wave_sum_f64(sd);
            float le = (float)sd;
            if (a.bias) le = le + a.bias[__builtin_amdgcn_readlane(ce, lj[b])];
            if (lane == lj[b]) cv = le;
          }
        }
      }
    }
    // final order over the candidates by (value desc, index asc)
    int rank = 0;
    for (int j = 0; j < ncand; ++j) rank += beats(readlane_f(cv, j), __builtin_amdgcn_readlane(ce, j), cv, ce);
    if (mine && rank < k) {
      s_selv[wave][rank] = cv;
      s_sele[wave][rank] = ce;
    }
    if (a.logits) {
      // approximate for everyone, then the candidates' final values on top
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (lane + 64 * m < E) a.logits[(size_t)t * E + lane + 64 * m] = av[m];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (mine) a.logits[(size_t)t * E + ce] = cv;
    }
  } else {
    // more candidates than lanes (e.g. all-equal logits): exact values for
    // every candidate, rank over all experts
    u32x4_t xc[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = lane + 64 * i;
      xc[i] = c < nch ? ld16(a.x + (size_t)t * a.H + c * 8) : zero;
    }
    float ex[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      ex[m] = -INFINITY;
      uint64_t mask = __ballot(cand[m]);
      while (mask) {
        const int bit = __builtin_ctzll(mask);
        mask &= mask - 1;
        const float le = exact_logit<CH>(xc, a, bit + 64 * m, lane);
        if (lane == bit) ex[m] = le;
      }
      if (lane + 64 * m < E) s_key[wave][lane + 64 * m] = ex[m];
    }
    wave_sync_lds();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = lane + 64 * m;
      if (cand[m]) {
        int rank = 0;
        for (int f = 0; f < E; ++f) rank += beats(s_key[wave][f], f, ex[m], e);
        if (rank < k) {
          s_selv[wave][rank] = ex[m];
          s_sele[wave][rank] = e;
        }
      }
      if (a.logits && e < E) a.logits[(size_t)t * E + e] = cand[m] ? ex[m] : av[m];
    }
  }
  wave_sync_lds();
  // w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0); the sum is a butterfly over
  // lanes 0..k-1 (others add 0), the same on every run
  const float lmax = s_selv[wave][0];
  const float pj = lane < k ? expf(s_selv[wave][lane] - lmax) : 0.f;
  float sum = pj;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (a.softmax_all) {
    // the full softmax: add the experts not chosen, with their MFMA logits
    // (each lane its own experts in order, then a butterfly)
    float rest = 0.f;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int e = lane + 64 * m;
      bool chosen = false;
      for (int j = 0; j < k; ++j) chosen |= s_sele[wave][j] == e;
      if (e < E && !chosen) rest += expf(av[m] - lmax);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rest += __shfl_xor(rest, off);
    sum += rest;
  }
  if (lane < k) {
    a.ids[(size_t)t * k + lane] = s_sele[wave][lane];
    a.wts[(size_t)t * k + lane] = pj / sum;
  }
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Bucketing of at most 64 slots by one wave, after the selection of a small
// batch in the same workgroup: the histogram, exclusive
// scan, work list and stable permutation the bucketing kernel forms (a
// slot's position is its expert's offset plus the number of same-expert
// slots before it, found with eight ballots over the id bits), without a
// launch of its own.
__device__ void bucket_small(const PermuteArgs& pa, int lane, int* s_cnt, int* s_off) {
  const int E = pa.E;
  const int N = pa.live ? min(pa.N, *pa.live * pa.k) : pa.N;
  for (int e = lane; e < kMaxE; e += 64) s_cnt[e] = 0;
  wave_sync_lds();
  const bool v = lane < N;
  int e = v ? pa.ids[lane] : 0;
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  if (v) atomicAdd(&s_cnt[e], 1);
  wave_sync_lds();
  int c[4], tc[4], csum = 0, tsum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = 4 * lane + q;
    c[q] = ee < E ? s_cnt[ee] : 0;
    csum += c[q];
    tc[q] = pa.tile > 0 ? (c[q] + pa.tile - 1) / pa.tile : 0;
    tc[q] = (tc[q] + pa.group - 1) / pa.group * pa.group;
    tsum += tc[q];
  }
  const int cincl = wave_incl_scan(csum, lane);
  int run = cincl - csum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = 4 * lane + q;
    if (ee < E) {
      s_off[ee] = run;
      pa.offsets[ee] = run;
      pa.counts[ee] = c[q];
    }
    run += c[q];
  }
  if (lane == 63) pa.offsets[E] = cincl;
  if (pa.items) {
    const int tincl = wave_incl_scan(tsum, lane);
    int trun = tincl - tsum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = 4 * lane + q;
      for (int i = 0; i < tc[q]; ++i) {
        pa.items[2 * (trun + i)] = ee;
        pa.items[2 * (trun + i) + 1] = i * pa.tile;
      }
      trun += tc[q];
    }
    if (lane == 63) *pa.n_items = tincl;
  }
  wave_sync_lds();
  uint64_t m = __ballot(v);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = v && ((e >> b) & 1);
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  const int rank = __popcll(m & ((1ull << lane) - 1ull));
  if (v) {
    const int p = s_off[e] + rank;
    pa.perm[p] = lane;
    if (pa.pos) pa.pos[lane] = p;
  }
}

// NW waves (tokens) per workgroup.  FUSE: one workgroup holds the whole
// batch (T <= NW, T * k <= 64) and wave 0 buckets its slots once every wave
// has written its token's ids
constexpr int kSelWaves = 4, kFuseMaxT = 8;
template <int M, int CH, int NS, bool FUSE, int NW>
__global__ __launch_bounds__(64 * NW) void route_select(SelParams P) {
  __shared__ SelShared<NW> sh;
  __shared__ int s_cnt[FUSE ? kMaxE : 1], s_off[FUSE ? kMaxE : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * NW + wave;
  if (t < P.a.T) select_token<M, CH, NS, NW>(P, t, wave, lane, sh);
  if constexpr (FUSE) {
    __syncthreads();  // the ids of every token are written (workgroup scope)
    if (wave == 0) bucket_small(P.pa, lane, s_cnt, s_off);
  }
}

template <int M, int NS, bool FUSE, int NW>
void launch_select_ns(const SelParams& P, hipStream_t s) {
  const int ch = (P.a.H + 511) / 512;
  const dim3 grid((P.a.T + NW - 1) / NW), block(64 * NW);
  if (ch <= 1)
    hipLaunchKernelGGL((route_select<M, 1, NS, FUSE, NW>), grid, block, 0, s, P);
  else if (ch <= 2)
    hipLaunchKernelGGL((route_select<M, 2, NS, FUSE, NW>), grid, block, 0, s, P);
  else if (ch <= 4)
    hipLaunchKernelGGL((route_select<M, 4, NS, FUSE, NW>), grid, block, 0, s, P);
  else
    hipLaunchKernelGGL((route_select<M, 8, NS, FUSE, NW>), grid, block, 0, s, P);
}

template <int M, bool FUSE, int NW>
void launch_select_f(const SelParams& P, hipStream_t s) {
  if (P.ks == 1)
    launch_select_ns<M, 1, FUSE, NW>(P, s);
  else if (P.ks == 8)
    launch_select_ns<M, 8, FUSE, NW>(P, s);
  else
    launch_select_ns<M, 0, FUSE, NW>(P, s);
}

// the split counts of H = 2048 (8 stored at decode sizes, 1 at large T) get
// their own kernels; any other count takes the predicated loads
template <int M>
void launch_select(const SelParams& P, bool fuse, hipStream_t s) {
  if (fuse && P.a.T <= kSelWaves)
    launch_select_f<M, true, kSelWaves>(P, s);
  else if (fuse)
    launch_select_f<M, true, kFuseMaxT>(P, s);
  else
    launch_select_f<M, false, kSelWaves>(P, s);
}

}  // namespace

int route_splits(int H) {
  // K splits of the partial-logit pass: a function of H only, so a token's
  // approximate logits (and with them its routing weights) do not depend on
  // the batch it is in.  Slices of >= 256 k, at most 16 splits.
  int ks = 1;
  while (ks * 2 <= 16 && H % (ks * 2 * 256) == 0) ks *= 2;
  return ks;
}

size_t route_scratch_floats(int t_max, int E, int H) { return 2 * (size_t)route_splits(H) * t_max * E; }

// Small T: one workgroup per (16 tokens, K split), so the router weights
// are read by many CUs at once, and every split's partial is stored.  Large
// T: the token tiles alone fill the chip, so a workgroup sums all splits
// itself and stores finished sums (1 or all ks per workgroup: any other
// grouping would add the split sums in another association and change the
// bits).
int route_stored_splits(int T, int H) {
  const int ntt = (T + kTok - 1) / kTok;
  return ntt >= 128 ? 1 : route_splits(H);
}

template <int NT, bool PN>
void launch_partial(const PartParams& pp, dim3 grid, hipStream_t s) {
  const int klen = pp.H / pp.ks;
  if (klen % (32 * 4) == 0)
    hipLaunchKernelGGL((route_partial<NT, 4, PN>), grid, dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL((route_partial<NT, 1, PN>), grid, dim3(256), 0, s, pp);
}

// plain token rows: the LDS-staged form; with the pre-block step: the
// register form, which forms the token operand on the fly
// plain token rows where one workgroup sums all K splits of its tokens
// (large T) and there are at least two expert tiles per wave of four: eight
// waves, half the expert tiles each
template <int NT>
bool partial_eight_waves(const PartParams& pp) { return NT >= 2 && pp.per_wg == pp.ks; }

template <int NT>
void launch_partial(const PartParams& pp, dim3 grid, hipStream_t s) {
  if (pp.res)
    launch_partial<NT, true>(pp, grid, s);
  else if (partial_eight_waves<NT>(pp))
    hipLaunchKernelGGL((route_partial_lds<(NT + 1) / 2, 8>), grid, dim3(512), 0, s, pp);
  else
    hipLaunchKernelGGL((route_partial_lds<NT>), grid, dim3(256), 0, s, pp);
}

// the instantiation launch_partial<NT> picks for pp (the same choice)
template <int NT>
const void* partial_fn(const PartParams& pp) {
  const bool u4 = (pp.H / pp.ks) % (32 * 4) == 0;
  if (pp.res) return u4 ? (const void*)&route_partial<NT, 4, true> : (const void*)&route_partial<NT, 1, true>;
  void (*lds_form)(PartParams) = partial_eight_waves<NT>(pp) ? route_partial_lds<(NT + 1) / 2, 8> : route_partial_lds<NT>;
  return (const void*)lds_form;
}

hipError_t launch_route(const RouteArgs& a, float* scratch, hipStream_t s, const PermuteArgs* fuse, bool* fused,
                        RouteNode* node) {
  const int ks = route_splits(a.H);
  const int ntt = (a.T + kTok - 1) / kTok;
  const int nst = route_stored_splits(a.T, a.H);  // stored partials per token
  const int per_wg = ks / nst;
  PartParams pp{a.x, a.wr, a.T, a.H, a.E, ks, per_wg, scratch, scratch + (size_t)nst * a.T * a.E};
  if (a.pn) {
    pp.res = a.pn->res;
    pp.delta = a.pn->delta;
    pp.gamma = a.pn->gamma;
    pp.eps = a.pn->eps;
    pp.res_out = a.pn->res_out;
    pp.x_out = const_cast<uint16_t*>(a.x);  // the block's x is the pre-block output
  }
  pp.live_rows = a.T;
  pp.live_out = a.live ? const_cast<int32_t*>(a.live) : nullptr;
  const dim3 pgrid(ntt, nst);
  const int n_et = a.E / 16;
  const void* fn;
  bool eight = false;  // the eight-wave form (512 threads)
  if (n_et <= 4) {
    launch_partial<1>(pp, pgrid, s);
    fn = partial_fn<1>(pp);
  } else if (n_et <= 8) {
    launch_partial<2>(pp, pgrid, s);
    fn = partial_fn<2>(pp);
    eight = !pp.res && partial_eight_waves<2>(pp);
  } else if (n_et <= 12) {
    launch_partial<3>(pp, pgrid, s);
    fn = partial_fn<3>(pp);
    eight = !pp.res && partial_eight_waves<3>(pp);
  } else {
    launch_partial<4>(pp, pgrid, s);
    fn = partial_fn<4>(pp);
    eight = !pp.res && partial_eight_waves<4>(pp);
  }
  if (node) {
    static_assert(sizeof(PartParams) <= sizeof(node->args), "router node arguments");
    node->fn = const_cast<void*>(fn);
    node->grid = pgrid;
    node->block = dim3(eight ? 512 : 256);
    std::memcpy(node->args, &pp, sizeof(pp));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // longest fp32 addition chain: 32 inside one MFMA, one per k-step of the
  // slice, the ks split partials, plus slack; doubled.
  const int depth = 32 + (a.H / ks) / 32 + ks + 8;
  SelParams sp{a, pp.part, pp.pabs, nst, (float)(2.0 * depth * 5.9604644775390625e-08), PermuteArgs{}};
  // a batch of at most kFuseMaxT tokens is selected by one workgroup, which
  // then also buckets its slots (one launch fewer)
  const bool fuse_now = fuse && a.T <= kFuseMaxT && a.T * a.k <= 64;
  if (fuse_now) sp.pa = *fuse;
  if (fused) *fused = fuse_now;
  if (a.E <= 64)
    launch_select<1>(sp, fuse_now, s);
  else if (a.E <= 128)
    launch_select<2>(sp, fuse_now, s);
  else
    launch_select<4>(sp, fuse_now, s);
  return hipGetLastError();
}

hipError_t set_route_live(hipGraphExec_t ge, hipGraphNode_t gn, const RouteNode& rn, int live_rows) {
  PartParams pp;
  std::memcpy(&pp, rn.args, sizeof(pp));
  pp.live_rows = live_rows;
  void* args[1] = {&pp};
  hipKernelNodeParams kp{};
  kp.func = rn.fn;
  kp.gridDim = rn.grid;
  kp.blockDim = rn.block;
  kp.sharedMemBytes = 0;
  kp.kernelParams = args;
  kp.extra = nullptr;
  return hipGraphExecKernelNodeSetParams(ge, gn, &kp);
}

}  // namespace moe
