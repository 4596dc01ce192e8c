// LoRA down-projections of the grouped expert GEMMs: for every routed row p
// of a work item (expert e, up to 16 of its rows),
//   U[p][j] = sum_k A[e][j][k] * src[row(p)][k],   j < 16 (the adapter rank)
// with src the block input x (row = the token of slot perm[p]) for the
// gate/up adapter, or h (row = p) for the down adapter.  The expert GEMM
// epilogues then add scale * sum_j B[e][n][j] * U[p][j] to their fp32
// accumulators (the rank-16, fp32-adapter LoRA of the unsloth commit
// 4f2bfe7f69 page's workload, injected into the grouped GEMMs).
//
// One workgroup per item (per 16-row sub-tile, or per eight of them, of a
// longer item); K is cut into 64-k blocks, block b going to wave
// b % 16 (at most four per wave).  The 16 x 16 tile U^T = A[e] (16 x K) *
// src^T (K x 16 rows) is one fp32 MFMA accumulation per wave over its blocks
// in order (16x16x4: lane (r, g) feeds A row r and the column of row r, in
// the i-th MFMA of a block k = 8g + i for i < 8 and 32 + 8g + i - 8 after,
// so that the four lanes of a row read each of its two 64-byte halves of the
// block together); the waves' tiles are then added in wave order.  A row's U depends only on its input row and expert, never
// on the batch.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRank = 16;
constexpr int kWaves = 16;
constexpr int kMaxBlocks = 4;  // 64-k blocks per wave (K <= 64 * 4 * 16 = 4096)

// float offset of the v-th group of four A values of a lane in a 64-k block
// (k = 8g + 4v for v < 2, 32 + 8g + 4(v - 2) after; the lane base holds 8g)
__device__ __forceinline__ int a_off(int v) { return v < 2 ? 4 * v : 32 + 4 * (v - 2); }

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// SUBS: 16-row sub-tiles per workgroup (1 at decode sizes; all eight of a
// 128-row item on the MFMA path's work list, so each wave loads its A blocks
// once for 128 rows instead of once per 16).  Per sub-tile the MFMA sequence
// and the wave-order sum are the same, so a row's U does not depend on SUBS.
template <int SUBS>
__global__ __launch_bounds__(64 * kWaves) void lora_a_kernel(LoraAArgs a) {
  __shared__ f32x4_t s_part[kWaves][64];
  const int per = a.subs / SUBS;  // workgroups per work item
  const int item = blockIdx.x / per, sub0 = (blockIdx.x - item * per) * SUBS;
  if (item >= *a.n_items) return;  // uniform over the workgroup
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1] + 16 * sub0;
  const int c = a.counts[e] - m0;
  if (c <= 0) return;  // sub-tiles past the item's rows
  const int nt = min((c + 15) / 16, SUBS);  // sub-tiles holding rows
  const int base = a.offsets[e] + m0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nb = a.K / 64;                  // 64-k blocks
  const int nw = nb < kWaves ? nb : kWaves;  // waves holding at least one
  f32x4_t acc[SUBS];
#pragma unroll
  for (int t = 0; t < SUBS; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (wave < nw) {
    int row[SUBS];  // this lane's source row in each sub-tile (0 past the rows: its products are never stored)
#pragma unroll
    for (int t = 0; t < SUBS; ++t) {
      const int m = 16 * t + r;
      row[t] = (t < nt && m < c) ? (a.by_token ? a.perm[base + m] / a.k : base + m) : 0;
    }
    const float* ar = a.A + ((size_t)e * kRank + r) * a.K + 8 * g;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    if constexpr (SUBS == 1) {
      // all blocks' operands in flight before the first MFMA
      const bool tv = r < c;
      const uint16_t* xr = a.src + (size_t)row[0] * a.K + 8 * g;
      f32x4_t av[kMaxBlocks][4];
      u32x4_t xv[kMaxBlocks][2];
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i) {
        const int b = wave + kWaves * i;
        if (b < nb) {
#pragma unroll
          for (int v = 0; v < 4; ++v) av[i][v] = *reinterpret_cast<const f32x4_t*>(ar + 64 * b + a_off(v));
#pragma unroll
          for (int v = 0; v < 2; ++v) xv[i][v] = tv ? ld16(xr + 64 * b + 32 * v) : zero;
        }
      }
#pragma unroll
      for (int i = 0; i < kMaxBlocks; ++i) {
        if (wave + kWaves * i < nb) {
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const uint32_t w = xv[i][m >> 3][(m & 7) >> 1];
            acc[0] = mfma_f32(av[i][m >> 2][m & 3], (m & 1) ? bf16hi(w) : bf16lo(w), acc[0]);
          }
        }
      }
    } else {
      // per block: its A values once, then every sub-tile's rows
      for (int i = 0; i < kMaxBlocks; ++i) {
        const int b = wave + kWaves * i;
        if (b >= nb) break;
        f32x4_t av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) av[v] = *reinterpret_cast<const f32x4_t*>(ar + 64 * b + a_off(v));
#pragma unroll
        for (int t = 0; t < SUBS; ++t) {
          if (t < nt) {
            const bool tv = 16 * t + r < c;
            const uint16_t* xr = a.src + (size_t)row[t] * a.K + 8 * g + 64 * b;
            const u32x4_t xv[2] = {tv ? ld16(xr) : zero, tv ? ld16(xr + 32) : zero};
#pragma unroll
            for (int m = 0; m < 16; ++m) {
              const uint32_t w = xv[m >> 3][(m & 7) >> 1];
              acc[t] = mfma_f32(av[m >> 2][m & 3], (m & 1) ? bf16hi(w) : bf16lo(w), acc[t]);
            }
          }
        }
      }
    }
  }
  // lane l of each wave holds D[4(l/16) + q][l % 16] = U[row l % 16][j = 4(l/16) + q]
  // of each sub-tile; the waves' tiles are added in wave order
#pragma unroll
  for (int t = 0; t < SUBS; ++t) {
    if (t >= nt) break;  // uniform
    s_part[wave][lane] = acc[t];
    __syncthreads();
    if (tid < 256) {
      const int l = tid & 63, q = tid >> 6;
      const int tok = l & 15, j = 4 * (l >> 4) + q;
      if (16 * t + tok < c) {
        float sum = 0.f;
        for (int w = 0; w < nw; ++w) sum += s_part[w][l][q];
        a.U[(size_t)(base + 16 * t + tok) * kRank + j] = sum;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- backward
// Sixteen adapter rows j times the (up to 16) routed rows of a work item,
// reduced over K in 64-k blocks spread over the waves as in lora_a_kernel:
//   out[tok][j] = sum_k P(j, k) Q(tok, k)
// fetch(r, k0, p, q) gives lane row r's 16 k of both operands (P row j = r
// as the MFMA A operand, Q row tok = r as B): element 4v + i is k = k0 + 16v
// + i, with k0 = 64b + 4g, so that the four lanes of a row read 64
// contiguous bytes of it in each of their four 16-byte loads.  The
// waves' tiles are added in wave order.  Ends with a barrier, so s_part can
// be used again.
template <typename Fetch>
__device__ __forceinline__ void rank16_reduce(int nb, int M, float* out, f32x4_t (&s_part)[kWaves][64],
                                              Fetch fetch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nw = nb < kWaves ? nb : kWaves;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (wave < nw) {
#pragma unroll
    for (int i = 0; i < kMaxBlocks; ++i) {
      const int b = wave + kWaves * i;
      if (b < nb) {
        float p[16], q[16];
        fetch(r, 64 * b + 4 * g, p, q);
#pragma unroll
        for (int m = 0; m < 16; ++m) acc = mfma_f32(p[m], q[m], acc);
      }
    }
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (tid < 256) {
    const int l = tid & 63, qq = tid >> 6;
    const int tok = l & 15, j = 4 * (l >> 4) + qq;
    if (tok < M) {
      float sum = 0.f;
      for (int w = 0; w < nw; ++w) sum += s_part[w][l][qq];
      out[(size_t)tok * kRank + j] = sum;
    }
  }
  __syncthreads();
}

// Per routed row p of a work item (expert e):
//   z[p][j] = sum_n B[e][n][j] v[p][n]    (v: DOWN w_p d_out[t_p], n < H;
//                                          GATE_UP (d_g, d_u)[p], n < 2I)
// and for DOWN also the fp32 adapter input of the down projection,
//   U_d[p][j] = sum_i A_d[e][j][i] h[p][i],  h = silu(g) u in fp32 from the
// g, u the training forward kept (the forward's U_d, formed from the bf16 h,
// is overwritten), so the adapter gradients carry no bf16 rounding of h.
__global__ __launch_bounds__(64 * kWaves) void lora_bt_kernel(BwdArgs a, int mode) {
  __shared__ f32x4_t s_part[kWaves][64];
  // one workgroup per 16-row sub-tile of a work item (row_tiles per item)
  const int item = blockIdx.x / a.row_tiles, sub = blockIdx.x - item * a.row_tiles;
  if (item >= *a.n_items) return;  // uniform over the workgroup
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1] + 16 * sub;
  const int c = a.counts[e] - m0;
  if (c <= 0) return;  // a sub-tile past the item's rows
  const int M = c < 16 ? c : 16, base = a.offsets[e] + m0;
  const bool down = mode == 0;
  const int H = a.H, I = a.I;
  const int Nn = down ? H : 2 * I;
  const float* B = (down ? a.lb_down : a.lb_gate_up) + (size_t)e * Nn * kRank;
  float* Z = (down ? a.z_down : a.z_gate_up) + (size_t)base * kRank;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  rank16_reduce(Nn / 64, M, Z, s_part, [&](int r, int k0, float (&p)[16], float (&q)[16]) {
    const bool tv = r < M;
    const float* vrow;
    float vs = 1.f;
    if (down) {
      const int slot = tv ? a.perm[base + r] : 0;
      vrow = a.d_out + (size_t)(slot / a.k) * H;
      vs = tv ? a.wts[slot] : 0.f;
    } else {
      vrow = a.gu + (size_t)(tv ? base + r : 0) * 2 * I;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4_t vv = tv ? *reinterpret_cast<const f32x4_t*>(vrow + k0 + 16 * v) : zero;
#pragma unroll
      for (int i = 0; i < 4; ++i) q[4 * v + i] = vs * vv[i];
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) p[m] = B[(size_t)(k0 + 16 * (m >> 2) + (m & 3)) * kRank + r];
  });
  if (!down) return;
  const float* A = a.la_down + (size_t)e * kRank * I;
  float* Ud = a.u_down + (size_t)base * kRank;
  rank16_reduce(I / 64, M, Ud, s_part, [&](int r, int k0, float (&p)[16], float (&q)[16]) {
    const bool tv = r < M;
    const float* gp = a.gu + (size_t)(tv ? base + r : 0) * 2 * I + k0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4_t gv = tv ? *reinterpret_cast<const f32x4_t*>(gp + 16 * v) : zero;
      const f32x4_t uv = tv ? *reinterpret_cast<const f32x4_t*>(gp + I + 16 * v) : zero;
      const f32x4_t av = *reinterpret_cast<const f32x4_t*>(A + (size_t)r * I + k0 + 16 * v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[4 * v + i] = silu(gv[i]) * uv[i];
        p[4 * v + i] = av[i];
      }
    }
  });
}

// Adapter gradients of every expert, summed over its routed rows in a fixed
// order (no atomics; zero for an expert no row reached), times the scale.
//   part 0 (down; before the down transposed GEMV turns g, u into d_g, d_u):
//     d_b_down[e][c][j] = s sum_p (w_p d_out[t_p][c]) U_d[p][j]
//     d_a_down[e][j][i] = s sum_p z_d[p][j] h[p][i],  h = silu(g) u (fp32)
//   part 1 (gate/up; after it):
//     d_b_gate_up[e][n][j] = s sum_p (d_g, d_u)[p][n] U_gu[p][j]
//     d_a_gate_up[e][j][h] = s sum_p z_gu[p][j] x[t_p][h]
// Each is a column c of the streamed operand (d_y, h, (d_g, d_u) or x) times
// the row's rank-16 vector (U or z).  A 256-thread workgroup covers 256 / G
// columns of one expert's B or A gradient with G row groups (G = GROUPS):
// thread (group q, column c) sums rows q, q + G, ... of the expert's sorted
// rows (its 16 sums, row by row in ascending order),
// the routed rows' vectors (and tokens, weights) staged in LDS kGradRows
// rows at a time, each thread's column loads issued 8 rows at a time; then
// the groups' partial sums are added in group order through LDS.  With 8
// groups (prefill sizes) a heavily routed expert's rows are walked by 8
// threads per column; at decode sizes (a few rows per expert) one group and
// 256 columns per workgroup keep the launch small.  Either way the result
// is the same on every run.  B-gradient rows are 16 contiguous floats;
// A-gradient rows are written column-coalesced.
constexpr int kGradRows = 128;

template <int GROUPS>
__global__ __launch_bounds__(256) void lora_grad_kernel(BwdArgs a, int part) {
  constexpr int kCols = 256 / GROUPS;       // columns per workgroup
  constexpr int kPer = kGradRows / GROUPS;  // rows per thread per staged chunk
  __shared__ f32x4_t s_vec[kGradRows][4];
  __shared__ int s_tok[kGradRows];
  __shared__ float s_w[kGradRows];
  __shared__ float s_red[GROUPS][GROUPS > 1 ? kCols : 1][kRank + 1];  // +1: no bank conflicts on the column reads
  const int H = a.H, I = a.I;
  const int nB = part == 0 ? H : 2 * I;  // columns (rows of the [n][16] array) of the B gradient
  const int nA = part == 0 ? I : H;      // columns of the [16][n] A gradient
  const int wgB = (nB + kCols - 1) / kCols;
  const int e = blockIdx.y;
  const bool isB = (int)blockIdx.x < wgB;
  const int grp = threadIdx.x / kCols, cl = threadIdx.x % kCols;
  const int col = (isB ? blockIdx.x : blockIdx.x - wgB) * kCols + cl;
  const bool cv = col < (isB ? nB : nA);
  const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
  const float* vec = part == 0 ? (isB ? a.u_down : a.z_down) : (isB ? a.u_gate_up : a.z_gate_up);
  float acc[kRank];
#pragma unroll
  for (int j = 0; j < kRank; ++j) acc[j] = 0.f;
  for (int c0 = p0; c0 < p1; c0 += kGradRows) {
    const int nr = p1 - c0 < kGradRows ? p1 - c0 : kGradRows;
    __syncthreads();  // the previous chunk's LDS reads are done
    for (int i = threadIdx.x; i < 4 * nr; i += 256) {
      const int r = i >> 2, qq = i & 3;
      s_vec[r][qq] = *reinterpret_cast<const f32x4_t*>(vec + (size_t)(c0 + r) * kRank + 4 * qq);
    }
    if (threadIdx.x < nr) {
      const int slot = a.perm[c0 + threadIdx.x];
      s_tok[threadIdx.x] = slot / a.k;
      s_w[threadIdx.x] = a.wts[slot];
    }
    __syncthreads();
    // this thread's rows grp, grp + GROUPS, ... of the chunk, 8 at a time
    for (int u0 = 0; u0 < kPer; u0 += 8) {
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = grp + GROUPS * (u0 + u);
        float v = 0.f;
        if (cv && r < nr) {
          const size_t p = (size_t)(c0 + r);
          if (part == 0) {
            if (isB) {
              v = s_w[r] * a.d_out[(size_t)s_tok[r] * H + col];
            } else {
              const float* gp = a.gu + p * 2 * I + col;
              v = silu(gp[0]) * gp[I];
            }
          } else {
            v = isB ? a.gu[p * 2 * I + col] : __uint_as_float((uint32_t)a.x[(size_t)s_tok[r] * H + col] << 16);
          }
        }
        sv[u] = v;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = grp + GROUPS * (u0 + u);
        if (r < nr) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const f32x4_t z = s_vec[r][qq];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[4 * qq + i] = fmaf(sv[u], z[i], acc[4 * qq + i]);
          }
        }
      }
    }
  }
  const float sc = a.lora_scale;
  if constexpr (GROUPS == 1) {
    if (!cv) return;
    if (isB) {
      float* o = (part == 0 ? a.g_b_down : a.g_b_gate_up) + ((size_t)e * nB + col) * kRank;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        *reinterpret_cast<f32x4_t*>(o + 4 * qq) =
            f32x4_t{sc * acc[4 * qq], sc * acc[4 * qq + 1], sc * acc[4 * qq + 2], sc * acc[4 * qq + 3]};
    } else {
      float* o = (part == 0 ? a.g_a_down : a.g_a_gate_up) + (size_t)e * kRank * nA + col;
#pragma unroll
      for (int j = 0; j < kRank; ++j) o[(size_t)j * nA] = sc * acc[j];
    }
  } else {
    // the groups' partial sums, added in group order: thread (q, c)
    // finishes rank values 2q, 2q + 1 of column c
    static_assert(GROUPS == 1 || kRank == 2 * GROUPS, "two rank values per thread in the final sum");
#pragma unroll
    for (int j = 0; j < kRank; ++j) s_red[grp][cl][j] = acc[j];
    __syncthreads();
    if (!cv) return;
    float fin[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < GROUPS; ++q) sum += s_red[q][cl][2 * grp + t];
      fin[t] = sc * sum;
    }
    if (isB) {
      float* o = (part == 0 ? a.g_b_down : a.g_b_gate_up) + ((size_t)e * nB + col) * kRank + 2 * grp;
      o[0] = fin[0];
      o[1] = fin[1];
    } else {
      float* o = (part == 0 ? a.g_a_down : a.g_a_gate_up) + (size_t)e * kRank * nA + col;
      o[(size_t)(2 * grp) * nA] = fin[0];
      o[(size_t)(2 * grp + 1) * nA] = fin[1];
    }
  }
}

// The same adapter gradients at prefill sizes, in two passes that spread a
// heavily routed expert over many workgroups.  Pass 1: one workgroup per
// (work item, 256 columns of the B or the A gradient); wave w takes 64 of
// the columns and accumulates, over the item's rows four at a time, the
// 16 x 16 tiles D_t[i][j] = sum_p data[p][c0 + 4i + t] vec[p][j] (t < 4) with
// fp32 MFMA 16x16x4 (lane (r, g) feeds row p = 4s + g: columns c0 + 4r .. +3
// as the A operand of the four tiles, vec[p][r] as the B operand), and stores
// the item's partial gradient.  Pass 2 adds each expert's item partials in
// item order, times the scale.  data / vec as in lora_grad_kernel.
// Partial layout per item: the B part [nB][16], then the A part [16][nA]
// (the gradients' own layouts, so pass 2 reads and writes contiguously).
constexpr int kItemCols = 256;
constexpr int kItemBatch = 8;  // row steps (4 rows each) whose loads are in flight together

template <int PART>
__global__ __launch_bounds__(256) void lora_grad_item_kernel(BwdArgs a) {
  __shared__ int s_tok[kMfmaTile];
  __shared__ float s_w[kMfmaTile];
  const int item = blockIdx.x;
  if (item >= *a.n_items) return;  // uniform over the workgroup
  const int e = a.items[2 * item], m0 = a.items[2 * item + 1];
  const int cnt = a.counts[e] - m0;
  const int rows = 16 * a.row_tiles;
  const int M = cnt < rows ? cnt : rows;
  if (M <= 0) return;  // an item past the expert's rows (pass 2 skips it)
  const int base = a.offsets[e] + m0;
  const int H = a.H, I = a.I, k = a.k;
  const int nB = PART == 0 ? H : 2 * I, nA = PART == 0 ? I : H;
  const int gB = (nB + kItemCols - 1) / kItemCols;
  const bool isB = (int)blockIdx.y < gB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if ((PART == 0 && isB) || (PART == 1 && !isB)) {
    // the rows' tokens (and routing weights): token-indexed operands
    for (int i = tid; i < M; i += 256) {
      const int slot = a.perm[base + i];
      s_tok[i] = slot / k;
      s_w[i] = a.wts[slot];
    }
    __syncthreads();
  }
  const int n = isB ? nB : nA;
  const int c0 = (isB ? (int)blockIdx.y : (int)blockIdx.y - gB) * kItemCols + 64 * wave;
  if (c0 >= n) return;  // no barrier follows
  const int r = lane & 15, g = lane >> 4;
  const int c = c0 + 4 * r;  // this lane's four columns
  const float* vec = PART == 0 ? (isB ? a.u_down : a.z_down) : (isB ? a.u_gate_up : a.z_gate_up);
  const int nsteps = (M + 3) / 4;
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsteps; s0 += kItemBatch) {
    f32x4_t dv[kItemBatch];
    float vv[kItemBatch];
#pragma unroll
    for (int u = 0; u < kItemBatch; ++u) {
      const int lr = 4 * (s0 + u) + g;  // the lane's row of this step (item-local)
      const bool ok = lr < M;
      const size_t p = (size_t)base + (ok ? lr : 0);
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
      if (ok) {
        if (PART == 0 && isB) {
          const f32x4_t o = *reinterpret_cast<const f32x4_t*>(a.d_out + (size_t)s_tok[lr] * H + c);
          const float w = s_w[lr];
          d = f32x4_t{w * o[0], w * o[1], w * o[2], w * o[3]};
        } else if (PART == 0) {
          const f32x4_t gg = *reinterpret_cast<const f32x4_t*>(a.gu + p * 2 * I + c);
          const f32x4_t uu = *reinterpret_cast<const f32x4_t*>(a.gu + p * 2 * I + I + c);
          d = f32x4_t{silu(gg[0]) * uu[0], silu(gg[1]) * uu[1], silu(gg[2]) * uu[2], silu(gg[3]) * uu[3]};
        } else if (isB) {
          d = *reinterpret_cast<const f32x4_t*>(a.gu + p * 2 * I + c);
        } else {
          const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(a.x + (size_t)s_tok[lr] * H + c);
          d = f32x4_t{bf16lo(xv[0]), bf16hi(xv[0]), bf16lo(xv[1]), bf16hi(xv[1])};
        }
      }
      dv[u] = d;
      vv[u] = ok ? vec[p * kRank + r] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kItemBatch; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma_f32(dv[u][t], vv[u], acc[t]);
  }
  // lane (r, g) holds D_t[4g + q][r]: column c0 + 16g + 4q + t, rank index r
  float* P = a.lora_part + (size_t)item * (nB + nA) * kRank;
  if (isB) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) P[(size_t)(c0 + 16 * g + 4 * q + t) * kRank + r] = acc[t][q];
  } else {
    float* PA = P + (size_t)nB * kRank + (size_t)r * nA + c0 + 16 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4_t*>(PA + 4 * q) = f32x4_t{acc[0][q], acc[1][q], acc[2][q], acc[3][q]};
  }
}

// Pass 2: workgroup (chunk of 1024 floats, expert e) adds the partials of
// e's items in item order (items of one expert are consecutive in the work
// list; items past the expert's rows hold nothing and are skipped); zero
// for an expert no row reached.
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(BwdArgs a, int part) {
  const int e = blockIdx.y;
  const int H = a.H, I = a.I;
  const int nB = part == 0 ? H : 2 * I, nA = part == 0 ? I : H;
  const int nitems = *a.n_items;
  // e's items: [i0, i1) = (items of experts < e, items of experts <= e)
  int i0 = 0, i1 = 0;
  for (int c0 = 0; c0 < nitems; c0 += 256) {
    const int i = c0 + (int)threadIdx.x;
    const int ei = i < nitems ? a.items[2 * i] : INT_MAX;
    i0 += __syncthreads_count(ei < e);
    i1 += __syncthreads_count(ei <= e);
  }
  const int per = (nB + nA) * kRank;  // floats per item
  const int v = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (v >= per) return;
  const int cnt = a.counts[e];
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  for (int i = i0; i < i1; i += 4) {  // four items' loads in flight, added in item order
    f32x4_t pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = i + u < i1 && a.items[2 * (i + u) + 1] < cnt;
      pv[u] = ok ? *reinterpret_cast<const f32x4_t*>(a.lora_part + (size_t)(i + u) * per + v) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s += pv[u];
  }
  const float sc = a.lora_scale;
  const f32x4_t o = {sc * s[0], sc * s[1], sc * s[2], sc * s[3]};
  if (v < nB * kRank)
    *reinterpret_cast<f32x4_t*>((part == 0 ? a.g_b_down : a.g_b_gate_up) + (size_t)e * nB * kRank + v) = o;
  else
    *reinterpret_cast<f32x4_t*>((part == 0 ? a.g_a_down : a.g_a_gate_up) + (size_t)e * kRank * nA + v - nB * kRank) =
        o;
}

}  // namespace

hipError_t launch_lora_bt(const BwdArgs& a, bool down, hipStream_t s) {
  const int Nn = down ? a.H : 2 * a.I;
  if (Nn % 64 || Nn > 64 * kMaxBlocks * kWaves || a.I % 64 || a.I > 64 * kMaxBlocks * kWaves)
    return hipErrorInvalidValue;
  if (a.row_tiles < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_bt_kernel, dim3(a.max_items * a.row_tiles), dim3(64 * kWaves), 0, s, a, down ? 0 : 1);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const BwdArgs& a, bool down, hipStream_t s) {
  const int nB = down ? a.H : 2 * a.I, nA = down ? a.I : a.H;
  // prefill sizes with room for every item's partial: per-item MFMA pass,
  // then the ordered sum over each expert's items
  if (a.lora_part && (long)a.T * a.k >= 32L * a.E && nB % 64 == 0 && nA % 64 == 0 &&
      16 * a.row_tiles <= kMfmaTile && (size_t)a.max_items * (nB + nA) * kRank <= a.lora_part_floats) {
    const int groups = (nB + kItemCols - 1) / kItemCols + (nA + kItemCols - 1) / kItemCols;
    if (down)
      hipLaunchKernelGGL(lora_grad_item_kernel<0>, dim3(a.max_items, groups), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(lora_grad_item_kernel<1>, dim3(a.max_items, groups), dim3(256), 0, s, a);
    const int per4 = (nB + nA) * kRank / 4;
    hipLaunchKernelGGL(lora_grad_reduce_kernel, dim3((per4 + 255) / 256, a.E), dim3(256), 0, s, a, down ? 0 : 1);
  } else if ((long)a.T * a.k >= 32L * a.E) {  // prefill sizes (on average >= 32 routed rows per expert): 8 row groups
    constexpr int cols = 256 / 8;
    hipLaunchKernelGGL(lora_grad_kernel<8>, dim3((nB + cols - 1) / cols + (nA + cols - 1) / cols, a.E), dim3(256), 0,
                       s, a, down ? 0 : 1);
  } else {
    hipLaunchKernelGGL(lora_grad_kernel<1>, dim3((nB + 255) / 256 + (nA + 255) / 256, a.E), dim3(256), 0, s, a,
                       down ? 0 : 1);
  }
  return hipGetLastError();
}

hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s) {
  if (a.K % 64 || a.K > 64 * kMaxBlocks * kWaves) return hipErrorInvalidValue;
  if (a.subs < 1) return hipErrorInvalidValue;
  if (a.subs % 8 == 0)  // the MFMA path's 128-row items: one workgroup per 8 sub-tiles
    hipLaunchKernelGGL(lora_a_kernel<8>, dim3(a.max_items * (a.subs / 8)), dim3(64 * kWaves), 0, s, a);
  else
    hipLaunchKernelGGL(lora_a_kernel<1>, dim3(a.max_items * a.subs), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
