// Capture-safe bucketing of token-expert slots by expert, one workgroup:
// histogram (the scatter_add form of the per-expert count), exclusive scan
// (the cumsum), stable counting-sort permutation (the argsort), and the
// expert work list for the grouped GEMMs -- all on the device, so nothing in
// the step reads a size back to the host (the failure that broke graph
// capture on the unsloth commit 80aaf1121b page, last paragraph).
//
// Stability: slots are taken in chunks of 1024 in ascending order.  Inside a
// chunk, a slot's position is the expert's running cursor, plus the number of
// same-expert slots in lower waves of the chunk, plus its rank among
// same-expert lanes of its own wave (found with eight ballots over the bits of
// the expert id).  So slots of one expert keep ascending order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 256;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// slots to bucket: all N, or the first live * k of a graph replay whose
// bucket is larger than its live row count
__device__ __forceinline__ int live_slots(const PermuteArgs& a) {
  return a.live ? min(a.N, *a.live * a.k) : a.N;
}

// inclusive scan of one int per lane across the wave
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteArgs a) {
  __shared__ int s_hist[kMaxE];
  __shared__ int s_cursor[kMaxE];
  __shared__ int s_wcnt[kWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = live_slots(a), E = a.E;

  for (int e = tid; e < kMaxE; e += kThreads) s_hist[e] = 0;
  for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();

  // histogram with LDS integer atomics (order-independent result)
  for (int s = tid; s < N; s += kThreads) atomicAdd(&s_hist[clamp_expert(a.ids[s], E)], 1);
  __syncthreads();

  // exclusive scan of counts (and of work-list tiles) by wave 0; lane owns experts 4*lane..4*lane+3
  if (wave == 0) {
    int c[4], tsum = 0, csum = 0, tc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      c[q] = e < E ? s_hist[e] : 0;
      csum += c[q];
      tc[q] = a.tile > 0 ? (c[q] + a.tile - 1) / a.tile : 0;
      tc[q] = (tc[q] + a.group - 1) / a.group * a.group;
      tsum += tc[q];
    }
    const int cincl = wave_incl_scan(csum, lane);
    int run = cincl - csum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      if (e < E) {
        s_cursor[e] = run;
        a.offsets[e] = run;
        a.counts[e] = c[q];
      }
      run += c[q];
    }
    if (lane == 63) a.offsets[E] = cincl;
    if (a.items) {
      const int tincl = wave_incl_scan(tsum, lane);
      int trun = tincl - tsum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * lane + q;
        for (int i = 0; i < tc[q]; ++i) {
          a.items[2 * (trun + i)] = e;
          a.items[2 * (trun + i) + 1] = i * a.tile;
        }
        trun += tc[q];
      }
      if (lane == 63) *a.n_items = tincl;
    }
  }
  __syncthreads();

  // stable scatter, chunk by chunk; the next chunk's ids are prefetched
  int e_next = tid < N ? clamp_expert(a.ids[tid], E) : 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int base = 0; base < N; base += kThreads) {
    const int s = base + tid;
    const bool v = s < N;
    const int e = e_next;
    const int sn = s + kThreads;
    e_next = sn < N ? clamp_expert(a.ids[sn], E) : 0;

    uint64_t m = __ballot(v);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = v && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    if (v && rank == 0) s_wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (v) {
      int p = s_cursor[e] + rank;
      for (int w2 = 0; w2 < wave; ++w2) p += s_wcnt[w2][e];
      a.perm[p] = s;
      if (a.pos) a.pos[s] = p;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kThreads) {
      int add = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) {
        add += s_wcnt[w2][e2];
        s_wcnt[w2][e2] = 0;
      }
      s_cursor[e2] += add;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------
// Large N: the same three steps spread over workgroups.  Slots are cut into
// chunks of kChunk; (1) each chunk's expert histogram, (2) every chunk's
// workgroup loads all chunk histograms, forms the expert offsets (exclusive
// scan of the totals) and its own starting cursor per expert (offset + slots
// of that expert in earlier chunks), and scatters its slots in ascending
// order exactly as the single-workgroup kernel does; chunk 0 also writes
// counts, offsets and the work list.
constexpr int kChunk = 2048;
constexpr int kChunkThreads = 1024;
constexpr int kMaxChunks = 65536 / kChunk;  // T*k <= 65536

__global__ __launch_bounds__(kChunkThreads) void permute_chunk_hist(PermuteArgs a) {
  __shared__ int s_h[kMaxE];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  for (int e = tid; e < kMaxE; e += kChunkThreads) s_h[e] = 0;
  __syncthreads();
  const int s0 = c * kChunk, s1 = min(live_slots(a), s0 + kChunk);
  for (int s = s0 + tid; s < s1; s += kChunkThreads) atomicAdd(&s_h[clamp_expert(a.ids[s], a.E)], 1);
  __syncthreads();
  for (int e = tid; e < a.E; e += kChunkThreads) a.chunk_base[(size_t)c * a.E + e] = s_h[e];
}

__global__ __launch_bounds__(kChunkThreads) void permute_chunk_scatter(PermuteArgs a) {
  constexpr int kW = kChunkThreads / 64;
  __shared__ int s_ch[kMaxChunks * kMaxE];  // all chunk histograms
  __shared__ int s_tot[kMaxE];
  __shared__ int s_cursor[kMaxE];
  __shared__ int s_wcnt[kW][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const int c = blockIdx.x;
  const int nchunk = (a.N + kChunk - 1) / kChunk;
  for (int i = tid; i < nchunk * E; i += kChunkThreads) s_ch[i] = a.chunk_base[i];
  for (int e = tid; e < kMaxE; e += kChunkThreads)
    for (int w = 0; w < kW; ++w) s_wcnt[w][e] = 0;
  __syncthreads();
  // per expert: total count and slots in chunks before this one
  for (int e = tid; e < E; e += kChunkThreads) {
    int tot = 0, before = 0;
    for (int cc = 0; cc < nchunk; ++cc) {
      const int v = s_ch[cc * E + e];
      before += cc < c ? v : 0;
      tot += v;
    }
    s_tot[e] = tot;
    s_cursor[e] = before;
  }
  __syncthreads();
  // exclusive scan of the totals (wave 0, 4 experts per lane) -> offsets
  if (wave == 0) {
    int cnt[4], tc[4], csum = 0, tsum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      cnt[q] = e < E ? s_tot[e] : 0;
      csum += cnt[q];
      tc[q] = a.tile > 0 ? (cnt[q] + a.tile - 1) / a.tile : 0;
      tc[q] = (tc[q] + a.group - 1) / a.group * a.group;
      tsum += tc[q];
    }
    const int cincl = wave_incl_scan(csum, lane);
    int run = cincl - csum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      if (e < E) {
        s_cursor[e] += run;
        if (c == 0) {
          a.offsets[e] = run;
          a.counts[e] = cnt[q];
        }
      }
      run += cnt[q];
    }
    if (c == 0) {
      if (lane == 63) a.offsets[E] = cincl;
      if (a.items) {
        const int tincl = wave_incl_scan(tsum, lane);
        int trun = tincl - tsum;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * lane + q;
          for (int i = 0; i < tc[q]; ++i) {
            a.items[2 * (trun + i)] = e;
            a.items[2 * (trun + i) + 1] = i * a.tile;
          }
          trun += tc[q];
        }
        if (lane == 63) *a.n_items = tincl;
      }
    }
  }
  __syncthreads();
  const int s0 = c * kChunk, s1 = min(live_slots(a), s0 + kChunk);
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int base = s0; base < s1; base += kChunkThreads) {
    const int s = base + tid;
    const bool v = s < s1;
    const int e = v ? clamp_expert(a.ids[s], E) : 0;
    uint64_t m = __ballot(v);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = v && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    if (v && rank == 0) s_wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (v) {
      int p = s_cursor[e] + rank;
      for (int w2 = 0; w2 < wave; ++w2) p += s_wcnt[w2][e];
      a.perm[p] = s;
      if (a.pos) a.pos[s] = p;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kChunkThreads) {
      int add = 0;
      for (int w2 = 0; w2 < kW; ++w2) {
        add += s_wcnt[w2][e2];
        s_wcnt[w2][e2] = 0;
      }
      s_cursor[e2] += add;
    }
    __syncthreads();
  }
}

}  // namespace

size_t permute_scratch_ints(int n_max, int E) { return (size_t)((n_max + kChunk - 1) / kChunk) * E; }

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.N <= 2 * kChunk || a.chunk_base == nullptr) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const int nchunk = (a.N + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(permute_chunk_hist, dim3(nchunk), dim3(kChunkThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_chunk_scatter, dim3(nchunk), dim3(kChunkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
