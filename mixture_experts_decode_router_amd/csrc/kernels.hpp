// Host-side launchers of the gfx950 MoE kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Decode/prefill token-tile height of the skinny expert kernels: one MFMA
// column block of 16 tokens.
constexpr int kSkinnyTile = 16;
// Token-tile height of the LDS-tiled MFMA expert kernels (large groups).
#ifndef MOE_MFMA_TILE
#define MOE_MFMA_TILE 128
#endif
constexpr int kMfmaTile = MOE_MFMA_TILE;

// Pre-block step fused into the router pass: x = bf16(r / sqrt(mean(r^2) +
// eps) * gamma) with r = bf16(res + delta), written to RouteArgs::x.
struct PrenormArgs {
  const uint16_t* res;    // bf16 [T][H]
  const uint16_t* delta;  // bf16 [T][H] or null
  const uint16_t* gamma;  // bf16 [H]
  float eps;
  uint16_t* res_out;      // bf16 [T][H] or null
};

struct RouteArgs {
  const uint16_t* x;      // bf16 [T][H] (with pn: written by the router pass, then read)
  const uint16_t* wr;     // bf16 [E][H]
  const float* bias;      // [E] or null
  int T, H, E, k;
  int32_t* ids;           // [T][k]
  float* wts;             // [T][k]
  float* logits;          // [T][E] or null
  const int32_t* live;    // device row count T_live <= T (graph replays: the router's first kernel writes
                          // T there, or the count a replay set), or null: rows >= T_live get no output
  bool softmax_all;       // weights = full softmax over E at the chosen (else renormalised over the k)
  const PrenormArgs* pn;  // host struct: fuse the pre-block step, or null
};
struct PermuteArgs;
// The router's first kernel as launched: enough to re-issue its arguments
// with another live row count into a captured graph (the kernel's first
// workgroup writes that count to RouteArgs::live for the rest of the step).
struct RouteNode {
  void* fn;
  dim3 grid, block;
  alignas(16) unsigned char args[192];
};
// scratch: route_scratch_floats(t_max, E, H) floats of device memory.
// fuse: the bucketing to run as well when the batch is small enough for the
// select workgroup to do it (*fused says whether it did), or null.
// With a.live set, the first kernel stores a.T there (graph captures).
// node: receives the first kernel's launch, or null.
hipError_t launch_route(const RouteArgs& a, float* scratch, hipStream_t s, const PermuteArgs* fuse = nullptr,
                        bool* fused = nullptr, RouteNode* node = nullptr);
// sets the live row count of a captured router node (see RouteNode)
hipError_t set_route_live(hipGraphExec_t ge, hipGraphNode_t gn, const RouteNode& rn, int live_rows);
size_t route_scratch_floats(int t_max, int E, int H);
// number of K-split partial logits stored per token at batch size T (the
// scratch holds them [nst][T][E] from its start: the router's approximate
// logits, bias not added, are their sum in split order)
int route_stored_splits(int T, int H);

struct PermuteArgs {
  const int32_t* ids;     // [N]
  int N, E;
  int tile;               // token-tile height for the work list (0: no list)
  int group;              // pad each expert's tile count to a multiple of this (>= 1)
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* perm;          // [N]
  int32_t* pos;           // [N] or null
  int32_t* items;         // [max_items][2] = (expert, first row in its group) or null
  int32_t* n_items;       // [1] or null
  int32_t* chunk_base;    // permute_scratch_ints(N, E) ints, or null (single workgroup)
  const int32_t* live;    // device row count, or null: only the first min(N, live * k) slots are bucketed
  int k;                  // slots per row (with live)
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
size_t permute_scratch_ints(int n_max, int E);

// Largest slot count (T * k) of the direct form of the 16-row expert kernels.
constexpr int kDirectMaxN = 1024;

struct ExpertArgs {
  // routing (device)
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const int32_t* n_items;
  int max_items;          // grid bound on the work list
  int H, I, E, k;
  // activations
  const uint16_t* x;      // bf16 [T][H]
  uint16_t* h;            // bf16 [N][I]  (sorted-slot order)
  float* y;               // fp32 [N][H]  (flat-slot order)
  // weights
  const uint16_t* w_gate_up;  // bf16 [E][2I][H]
  const uint16_t* w_down;     // bf16 [E][H][I]
  const uint8_t* q_gate_up;   // [E][2I][H/2]
  const float* s_gate_up;     // [E][2I][H/64]
  const uint8_t* q_down;      // [E][H][I/2]
  const float* s_down;        // [E][H][I/64]
  const float* codebook;      // [16]
  // LoRA (skinny kernels): acc[n][p] += lora_scale * sum_j B[e][n][j] * U[p][j]
  bool lora;
  float lora_scale;
  const float* lb_gate_up;    // fp32 [E][2I][16]
  const float* lb_down;       // fp32 [E][H][16]
  const float* u_gate_up;     // fp32 [N][16], sorted-slot order
  const float* u_down;        // fp32 [N][16], sorted-slot order
  float* gu;                  // or null; else the bf16 gate/up kernels also keep g and u here:
                              // fp32 [N][2I] (g, then u), sorted-slot order
  // direct form of the 16-row bf16 kernels (ids set; no LoRA, gu null): no
  // work list, each wave finds its expert's slots among the first
  // min(N, *live * k) routed ids (N <= kDirectMaxN), and the gate/up kernel
  // records the bucketing in r_* (counts [E], offsets [E+1], perm [N], pos
  // [N] or null) as the bucketing kernel would, work list aside
  const int32_t* ids;         // [N] or null (work-list form)
  int N;
  const int32_t* live;        // device row count, or null
  int32_t* r_counts;
  int32_t* r_offsets;
  int32_t* r_perm;
  int32_t* r_pos;
};

// U[p][:] = A[e] src-row(p) for every row of the skinny work list (rank 16)
struct LoraAArgs {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const int32_t* n_items;
  int max_items, k, K;
  int subs;               // 16-row sub-tiles per work item (1, or kMfmaTile / 16 on the MFMA path's work list)
  const uint16_t* src;    // x [T][K] (by_token) or h [N][K] (sorted-slot order)
  bool by_token;
  const float* A;         // fp32 [E][16][K]
  float* U;               // fp32 [N][16]
};
hipError_t launch_lora_a(const LoraAArgs& a, hipStream_t s);
// tiled: weights in the fragment-tiled layout written by launch_pack
hipError_t launch_gate_up(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s);
hipError_t launch_down(const ExpertArgs& a, bool nf4, bool tiled, hipStream_t s);

// Backward of the block (frozen tiled bf16 weights, the forward's routing
// and per-slot y; skinny work list)
struct BwdArgs {
  int T, H, I, E, k, max_items;
  const int32_t* ids;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const int32_t* n_items;
  const float* wts;           // [T][k]
  const float* y;             // forward y [N][H], flat-slot order
  const float* d_out;         // [T][H]
  float* d_x;                 // [T][H]
  float* d_w;                 // [T][k] or null
  const uint16_t* w_router;   // bf16 [E][H]
  const uint16_t* w_gate_up;  // tiled bf16
  const uint16_t* w_down;     // tiled bf16
  // tiled 4-bit weights (nf4 true): codes, fp32 absmax per 64, fp32 codebook [16]
  bool nf4;
  const uint8_t* q_gate_up;
  const float* s_gate_up;
  const uint8_t* q_down;
  const float* s_down;
  const float* codebook;
  float* gu;                  // [N][2I]: g, u kept by the forward, then d_g, d_u
  uint16_t* gub;              // [N][2I]: d_g, d_u rounded to bf16 by the tiled down pass (its gate/up pass's
                              // A operand); the tiled bf16 backward needs it
  float* d_xs;                // [N][H], flat-slot order (may reuse y's memory)
  int row_tiles;              // 16-row tiles per work item: 1 (16-row GEMVs), or kMfmaTile / 16 after an
                              // MFMA forward (the tiled transposed GEMMs; bf16 weights)
  // LoRA (lora true): the adapters, the forward's U = A x / A h, the backward's
  // z = B^T v, and the adapter gradients (same shapes as the adapters)
  bool lora;
  float lora_scale;
  const uint16_t* x;          // bf16 [T][H] (the forward's input; LoRA or wgrad)
  const uint16_t* h;          // bf16 [N][I] sorted-slot order (the forward's h)
  const float* la_gate_up;    // [E][16][H]
  const float* lb_gate_up;    // [E][2I][16]
  const float* la_down;       // [E][16][I]
  const float* lb_down;       // [E][H][16]
  const float* u_gate_up;     // [N][16]
  float* u_down;              // [N][16] (the backward rewrites it from the fp32 h)
  float* z_gate_up;           // [N][16]
  float* z_down;              // [N][16]
  float* g_a_gate_up;
  float* g_b_gate_up;
  float* g_a_down;
  float* g_b_down;
  float* lora_part;           // prefill adapter gradients: per-item partial sums (may reuse y's memory), or null
  size_t lora_part_floats;    // its capacity
  // top-k weights without renormalisation (unrenorm true): the router's
  // stored split partial logits [r_nst][T][E] and bias (or null), for the
  // softmax over all E experts
  bool unrenorm;
  const float* r_part;
  int r_nst;
  const float* r_bias;
  // expert-weight gradients (wgrad true): fp32, the weights' row-major shapes
  bool wgrad;
  const float* hf;            // fp32 h [N][I] (sorted-slot order) formed by launch_h, or null
  float* g_w_gate_up;         // [E][2I][H]
  float* g_w_down;            // [E][H][I]
};
hipError_t launch_bwd_weights(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_t(const BwdArgs& a, bool down, hipStream_t s);
hipError_t launch_bwd_combine(const BwdArgs& a, hipStream_t s);
// expert-weight gradients: down ones before bwd_t(down), gate/up ones after it
hipError_t launch_wgrad(const BwdArgs& a, bool down, hipStream_t s);
// h = silu(g) u in fp32 for every routed row, into hf (fp32 [T*k][I])
hipError_t launch_h(const BwdArgs& a, float* hf, hipStream_t s);
// LoRA backward: z = B^T v per routed row (down: v = w d_out, and U_d = A_d h
// from the fp32 g, u; gate/up: v = (d_g, d_u))
hipError_t launch_lora_bt(const BwdArgs& a, bool down, hipStream_t s);
// LoRA adapter gradients: down ones before bwd_t(down), gate/up ones after it
hipError_t launch_lora_grad(const BwdArgs& a, bool down, hipStream_t s);

// LDS-tiled MFMA grouped GEMMs (bf16 weights in the tiled layout only);
// the work list must use kMfmaTile.  With a.lora the epilogues add the
// adapters' B U terms exactly as the 16-row kernels do.
hipError_t launch_gate_up_mfma(const ExpertArgs& a, hipStream_t s);
hipError_t launch_down_mfma(const ExpertArgs& a, hipStream_t s);
// the same work list and outputs for tiled 4-bit weights (adapters allowed,
// kept pre-activations allowed)
hipError_t launch_gate_up_mfma_nf4(const ExpertArgs& a, hipStream_t s);
hipError_t launch_down_mfma_nf4(const ExpertArgs& a, hipStream_t s);

struct PackArgs {
  bool nf4;
  int E, H, I;
  const void* src_gate_up;  // bf16 [E][2I][H] or codes [E][2I][H/2]
  const void* src_down;     // bf16 [E][H][I]  or codes [E][H][I/2]
  const float* src_s_gate_up;
  const float* src_s_down;
  void* dst_gate_up;
  void* dst_down;
  float* dst_s_gate_up;
  float* dst_s_down;
};
hipError_t launch_pack(const PackArgs& a, hipStream_t s);

struct CombineArgs {
  const float* y;         // [T*k][H]
  const float* wts;       // [T][k]
  void* out;              // [T][H], fp32 or bf16
  int T, H, k;
  const int32_t* live;    // device row count, or null: rows >= live are not written
  bool out_bf16;          // round the fp32 sums to bf16 (nearest even)
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);


// measurement probes (probe.hip): sink holds n_wg * 4 words (read) or
// n_wg * 256 floats (mfma)
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int n_wg, hipStream_t s);
hipError_t launch_probe_mfma(float* sink, int n_wg, int iters, int shape, hipStream_t s);
hipError_t launch_probe_gather(const void* src, uint32_t row_bytes, uint32_t seg_log, uint32_t tiles, int iters,
                               int order, uint32_t* sink, int n_wg, hipStream_t s);

}  // namespace moe
