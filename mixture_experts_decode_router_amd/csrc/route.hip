// Router for gfx950: logits -> top-k (ties to the lower expert index) ->
// renormalised softmax weights, one fused kernel per 16-token tile.
//
// The block's router is a linear map to fp32 logits followed by softmax,
// top-k and renormalisation; its pointwise tail is what the compiled walker
// fused (unsloth commit a1bc5cbd page, first paragraph).  The decision (which
// k experts, in which order) is taken on the correctly rounded fp32 logit of
// each expert, so that it is reproducible bit for bit:
//
//   phase 1  bf16 MFMA (fp32 accumulate) gives an approximate logit a[t][e]
//            and, from the same operands with the sign bits cleared,
//            S[t][e] = sum_h |x_h * w_h|.  The fp32 accumulation error of a
//            chain of d additions is at most d * 2^-24 * S, so
//            |a - l| <= beta = gamma * S + (rounding of the fp32 result and
//            of the bias add), gamma covering the longest chain with a
//            factor-2 margin.
//   phase 2  one wave per token.  Let L be the k-th largest lower bound
//            a - beta.  Any expert with a + beta < L is beaten strictly by k
//            others, so the true top-k lies within C = {e : a + beta >= L}
//            (usually k or k+1 experts).  Each candidate's dot product is
//            re-formed in fp64 from the exact bf16 products and rounded to
//            fp32 (plus the fp32 bias); the top-k of C by (value desc,
//            index asc) is the top-k of all experts.
//
// Softmax weights w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), fp32, j in
// selection order (equal to the full softmax renormalised over the top k).
#include <float.h>
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kTok = 16;        // tokens per workgroup (one MFMA column block)
constexpr int kWaves = 8;       // 512 threads: phase-1 work items, then one wave per token
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kPart = 256;      // ks * E <= max(E, 128) partial rows per token in LDS

struct KParams {
  RouteArgs a;
  int ks;         // K splits of phase 1 (items = E/16 * ks)
  float gamma;    // relative error bound of the phase-1 accumulation
};

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

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

template <int CH>  // 16-byte chunks per lane covering one row: ceil(H / 512)
__global__ __launch_bounds__(512) void route_kernel(KParams P) {
  __shared__ float s_l[kPart * kTok];
  __shared__ float s_s[kPart * kTok];
  __shared__ float s_selv[kTok * kMaxK];
  __shared__ int s_sele[kTok * kMaxK];
  const RouteArgs& a = P.a;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kTok;
  const int H = a.H, E = a.E, T = a.T, k = a.k;
  const int n_et = E >> 4;
  const int ks_n = P.ks;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // ---------------- phase 1: approximate logits and |x||w| sums (MFMA)
  for (int item = wave; item < n_et * ks_n; item += kWaves) {
    const int et = item % n_et, ks = item / n_et;
    const int r = lane & 15, g = lane >> 4;
    const int klen = H / ks_n;
    const int kbeg = ks * klen;
    const int trow = t0 + r;
    const bool tv = trow < T;
    const uint16_t* pa = a.wr + (size_t)(et * 16 + r) * H + kbeg + g * 8;
    const uint16_t* pb = a.x + (size_t)(tv ? trow : 0) * H + kbeg + g * 8;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, aab = {0.f, 0.f, 0.f, 0.f};
    const uint32_t absm = 0x7fff7fffu;
    int kk = 0;
    for (; kk + 32 * 16 <= klen; kk += 32 * 16) {
      u32x4_t av[16], bv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        av[u] = ld16(pa + kk + u * 32);
        bv[u] = tv ? ld16(pb + kk + u * 32) : zero;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        acc = mfma16(av[u], bv[u], acc);
        aab = mfma16(av[u] & absm, bv[u] & absm, aab);
      }
    }
    for (; kk < klen; kk += 32) {
      u32x4_t av = ld16(pa + kk);
      u32x4_t bv = tv ? ld16(pb + kk) : zero;
      acc = mfma16(av, bv, acc);
      aab = mfma16(av & absm, bv & absm, aab);
    }
    // lane holds D[4g+q][r]: expert et*16 + 4g + q, token r
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = (ks * kTok + r) * E + et * 16 + 4 * g + q;
      s_l[idx] = acc[q];
      s_s[idx] = aab[q];
    }
  }
  __syncthreads();

  // ---------------- phase 2: one wave per token, kTok / kWaves tokens per wave
  for (int tl = wave; tl < kTok; tl += kWaves) {
  const int t = t0 + tl;
  if (t >= T) break;
  constexpr int M = kMaxE / 64;
  float av[M], bd[M];
  bool valid[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int e = lane + 64 * m;
    valid[m] = e < E;
    av[m] = -INFINITY;
    bd[m] = 0.f;
    if (valid[m]) {
      float l = 0.f, s = 0.f;
      for (int ks = 0; ks < ks_n; ++ks) {
        l += s_l[(ks * kTok + tl) * E + e];
        s += s_s[(ks * kTok + tl) * E + e];
      }
      const float bv = a.bias ? a.bias[e] : 0.f;
      av[m] = a.bias ? l + bv : l;
      bd[m] = P.gamma * s + 2.5e-7f * (fabsf(l) + fabsf(bv)) + 1e-30f;
    }
  }

  // k-th largest lower bound L
  float L = -INFINITY;
  {
    uint32_t removed = 0;
    for (int j = 0; j < k; ++j) {
      float v = -INFINITY;
      int i = INT_MAX;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int e = lane + 64 * m;
        const float lo = av[m] - bd[m];
        if (valid[m] && !((removed >> m) & 1u) && (lo > v || (lo == v && e < i))) {
          v = lo;
          i = e;
        }
      }
      wave_argmax(v, i);
      L = v;
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (i == lane + 64 * m) removed |= 1u << m;
    }
  }

  bool cand[M];
  float ex[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    cand[m] = valid[m] && (av[m] + bd[m] >= L);
    ex[m] = av[m];
  }

  // re-form each candidate's logit in fp64 from the exact products
  const int nch = H >> 3;
  u32x4_t xc[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = lane + 64 * i;
    xc[i] = (c < nch) ? ld16(a.x + (size_t)t * H + c * 8) : zero;
  }
  constexpr int NB = CH >= 8 ? 2 : 32 / CH;  // candidates per batch (row loads in flight per lane: NB * CH)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    uint64_t mask = __ballot(cand[m]);
    while (mask) {
      int eb[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (mask) {
          eb[b] = __builtin_ctzll(mask) + 64 * m;
          mask &= mask - 1;
        } else {
          eb[b] = -1;
        }
      }
      u32x4_t wc[NB][CH];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int c = lane + 64 * i;
          wc[b][i] = (eb[b] >= 0 && c < nch) ? ld16(a.wr + (size_t)eb[b] * H + c * 8) : zero;
        }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < CH; ++i) s = dot8_f64(xc[i], wc[b][i], s);
        s = wave_sum_f64(s);
        if (eb[b] >= 0) {
          float le = (float)s;
          if (a.bias) le = le + a.bias[eb[b]];
          if (lane == (eb[b] & 63)) ex[m] = le;
        }
      }
    }
  }

  // top-k of the candidates by (exact fp32 logit desc, index asc); the
  // choices go through LDS so that lane j can emit choice j
  float* sel_v = s_selv + tl * kMaxK;
  int* sel_e = s_sele + tl * kMaxK;
  {
    uint32_t taken = 0;
    for (int j = 0; j < k; ++j) {
      float v = -INFINITY;
      int i = INT_MAX;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int e = lane + 64 * m;
        if (cand[m] && !((taken >> m) & 1u) && (ex[m] > v || (ex[m] == v && e < i))) {
          v = ex[m];
          i = e;
        }
      }
      wave_argmax(v, i);
      if (lane == 0) {
        sel_v[j] = v;
        sel_e[j] = i;
      }
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (i == lane + 64 * m) taken |= 1u << m;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0); the sum is a butterfly over
  // lanes 0..k-1 (others add 0), the same on every run
  const float pj = lane < k ? expf(sel_v[lane] - sel_v[0]) : 0.f;
  float sum = pj;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    a.ids[(size_t)t * k + lane] = sel_e[lane];
    a.wts[(size_t)t * k + lane] = pj / sum;
  }
  if (a.logits) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (valid[m]) a.logits[(size_t)t * E + lane + 64 * m] = cand[m] ? ex[m] : av[m];
  }
  }  // token loop
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  int ks = 1;
  {
    int lim = (16 * kWaves) / a.E;  // phase-1 items (E/16 * ks) fill the waves
    if (a.H / 256 < lim) lim = a.H / 256;
    while (ks * 2 <= lim) ks *= 2;
    while (ks > 1 && (a.H % ks != 0 || (a.H / ks) % 32 != 0)) ks >>= 1;
  }
  // longest fp32 addition chain: 32 inside one MFMA, one per k-step, the
  // partial sums over the splits, plus slack; doubled for margin.
  const int depth = 32 + (a.H / ks) / 32 + ks + 8;
  KParams P{a, ks, (float)(2.0 * depth * 5.9604644775390625e-08)};
  const dim3 grid((a.T + kTok - 1) / kTok), block(64 * kWaves);
  const int ch = (a.H + 511) / 512;
  if (ch <= 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, block, 0, s, P);
  else if (ch <= 2)
    hipLaunchKernelGGL(route_kernel<2>, grid, block, 0, s, P);
  else if (ch <= 4)
    hipLaunchKernelGGL(route_kernel<4>, grid, block, 0, s, P);
  else
    hipLaunchKernelGGL(route_kernel<8>, grid, block, 0, s, P);
  return hipGetLastError();
}

}  // namespace moe
