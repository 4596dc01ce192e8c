/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse-MoE block library.
 *
 * The block is the Qwen3-MoE sparse feed-forward layer as run on the
 * grouped_mm path described on the unsloth commit 80aaf1121b page
 * (Qwen3-MoE decode CUDA-graph capture), third paragraph: router ->
 * per-expert token counts -> cumulative offsets -> argsort permutation ->
 * one grouped GEMM over all active experts -> per-token weighted add.  The
 * router turns fp32 logits into the top-k experts (ties go to the lower
 * expert index) and renormalises their softmax weights; each expert is a
 * SwiGLU MLP; the result is a plain tensor (unsloth commit 4f2bfe7f69 page,
 * second paragraph).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers unless marked "host".  Tensors are
 *     dense, row-major, and 16-byte aligned.  bf16 data is passed as void*.
 *   - The caller owns every buffer.  Entry points never allocate device
 *     memory, never synchronise the stream and never copy to the host
 *     (except moe_read_counts, which says so).  Work is enqueued on `stream`
 *     (NULL = the default stream) in call order.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-MOE_OK status means nothing was launched.  moe_last_error() gives
 *     a message for the calling thread's last failure.  A fault on the GPU
 *     surfaces at the caller's next synchronising HIP call.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     on every run, eager or graph-replayed (no floating-point atomics).
 *   - Supported shapes: hidden and inter multiples of 128 in [128, 4096];
 *     n_experts a multiple of 16 in [16, 256]; 1 <= top_k <= min(n_experts,
 *     16); 1 <= t_max and t_max * top_k <= 65536.  Other shapes return
 *     MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,       /* null/misaligned pointer, T out of range, bad bucket list */
  MOE_ERR_UNSUPPORTED = 2,       /* shape or format outside the built kernels */
  MOE_ERR_WORKSPACE = 3,         /* workspace smaller than moe_workspace_size() */
  MOE_ERR_NOT_CAPTURABLE = 4,    /* graph capture refused; stream left uncaptured, run eagerly */
  MOE_ERR_CAPTURE_VIOLATION = 5, /* a synchronising call was made on a capturing stream */
  MOE_ERR_HIP = 6                /* a HIP runtime call failed (message in moe_last_error) */
} moe_status;

typedef enum {
  MOE_W_BF16 = 0,           /* bf16 expert weights, row-major */
  MOE_W_NF4_B64 = 1,        /* 4-bit codes + one fp32 absmax per 64 consecutive weights, row-major */
  MOE_W_BF16_TILED = 2,     /* MOE_W_BF16 in the tiled layout written by moe_pack_weights */
  MOE_W_NF4_B64_TILED = 3   /* MOE_W_NF4_B64 in the tiled layout written by moe_pack_weights */
} moe_wformat;

typedef enum {
  MOE_OUT_F32 = 0,   /* out fp32 [T][H] */
  MOE_OUT_BF16 = 1   /* out bf16 [T][H]: the fp32 result rounded to nearest even */
} moe_outdtype;

typedef enum {
  MOE_TOPK_RENORM = 0,  /* w_j = softmax over the k chosen logits (= full softmax renormalised) */
  MOE_TOPK_SOFTMAX = 1  /* w_j = softmax over all E logits, taken at the k chosen (sum < 1) */
} moe_topk_weights;

/* Shape of one MoE layer.  t_max bounds T for every call made with this
 * config and sizes the workspace.  Zero-initialised trailing fields give the
 * defaults (fp32 output, renormalised top-k weights). */
typedef struct {
  int32_t hidden;       /* H: model width */
  int32_t inter;        /* I: expert intermediate width */
  int32_t n_experts;    /* E */
  int32_t top_k;        /* k */
  int32_t t_max;        /* largest token count T passed with this config */
  int32_t wfmt;         /* moe_wformat */
  int32_t out_dtype;    /* moe_outdtype */
  int32_t topk_weights; /* moe_topk_weights */
  int32_t train;        /* 1: moe_forward also keeps the gate/up pre-activations for moe_backward */
} moe_config;

/* Layer weights (device, read-only).  Expert tensors are stacked on E.
 *   w_router   bf16 [E][H]
 *   router_bias fp32 [E] or NULL: added to the fp32 router logits before
 *              selection and softmax.
 * MOE_W_BF16:
 *   w_gate_up  bf16 [E][2I][H]   rows [0,I) = gate, rows [I,2I) = up
 *   w_down     bf16 [E][H][I]
 * MOE_W_NF4_B64 (weight = codebook[code] * absmax, 64 weights per absmax
 * along the last axis; element 2i in the low nibble of byte i):
 *   q_gate_up  uint8 [E][2I][H/2]    s_gate_up fp32 [E][2I][H/64]
 *   q_down     uint8 [E][H][I/2]     s_down    fp32 [E][H][I/64]
 *   codebook   fp32 [16], finite normal values (or zero) of magnitude <= 1.
 *              The kernels take each entry as two bf16 parts, hi = the
 *              nearest bf16 and lo = the bf16 nearest to (entry - hi), which
 *              carry it to within 2^-18 of its magnitude; an entry that is
 *              a bf16 value enters exactly.  The absmax scales are applied
 *              to fp32 partial sums over each 64-block.
 * The _TILED formats hold the same values in the layout moe_pack_weights
 * writes (same buffer sizes).  Unused fields may be NULL.
 *   lora       host pointer to rank-16 adapters on every expert (see
 *              moe_lora), read during the call (or the capture), or NULL. */

/* Low-rank adapters on the expert GEMMs (the rank-16 LoRA with fp32
 * adapters of the unsloth commit 4f2bfe7f69 page's workload), fused into the
 * decode expert kernels: every expert's stacked gate/up matrix acts as
 * W_gu + scale * B_gu A_gu and its down matrix as W_d + scale * B_d A_d:
 *   [gate; up] = W_gu x + scale * B_gu (A_gu x)   (before SiLU * up)
 *   y          = W_d h  + scale * B_d (A_d h)      (h: the bf16 h the down GEMM reads)
 * A x is formed in fp32 per routed row (fixed order, batch-independent),
 * the B products in fp32 in the GEMM epilogues: the 16-row decode kernels
 * and the MFMA prefill kernels (T * top_k >= 32 * n_experts, tiled bf16 or
 * 4-bit weights) add them with the same arithmetic, so a row's result does
 * not depend on the batch.  Device arrays, fp32, 16-byte aligned:
 *   a_gate_up [E][r][H]   b_gate_up [E][2I][r] (gate rows, then up rows)
 *   a_down    [E][r][I]   b_down    [E][H][r] */
typedef struct {
  const float* a_gate_up;
  const float* b_gate_up;
  const float* a_down;
  const float* b_down;
  float scale;    /* alpha / r, finite */
  int32_t rank;   /* r; 16 is supported */
} moe_lora;

typedef struct {
  const void* w_router;
  const float* router_bias;
  const void* w_gate_up;
  const void* w_down;
  const uint8_t* q_gate_up;
  const float* s_gate_up;
  const uint8_t* q_down;
  const float* s_down;
  const float* codebook;
  const moe_lora* lora;
} moe_weights;

/* Routing arrays inside a forward workspace (device pointers), valid after a
 * moe_forward or a graph replay has completed on the stream. */
typedef struct {
  int32_t* topk_ids;   /* [T][k] */
  float* topk_w;       /* [T][k] */
  int32_t* counts;     /* [E] */
  int32_t* offsets;    /* [E+1] */
  int32_t* perm;       /* [T*k] */
  int32_t* pos;        /* [T*k] */
} moe_views;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int32_t status);

/* Message describing the calling thread's most recent non-OK status. */
const char* moe_last_error(void);

/* MOE_OK if the config is within the supported shapes. */
moe_status moe_config_check(const moe_config* cfg);

/* Bytes of workspace moe_forward / moe_graph_capture need for cfg (sized
 * for cfg->t_max); 0 if cfg is invalid. */
size_t moe_workspace_size(const moe_config* cfg);

/* Router: fp32 logits l[t][e] = sum_h x[t][h]*w_router[e][h] (+ bias[e]),
 * the top-k experts per token (largest logit first, equal logits -> lower
 * expert index) and their softmax weights: renormalised over the chosen,
 * w_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) (MOE_TOPK_RENORM), or the
 * full softmax over all E experts at the chosen ones (MOE_TOPK_SOFTMAX; the
 * experts not chosen enter the sum with their bounded MFMA logits).
 * The k chosen experts and their order are those of the correctly rounded
 * fp32 logits: an MFMA pass gives each logit with a proven error bound, and
 * whenever the bound leaves the set or the order open, the candidates' dot
 * products are re-formed in fp64 and rounded.  The weights use the logits
 * the decision was taken on (exact, or within the bound when no
 * re-formation was needed).
 *   x         bf16 [T][H]
 *   topk_ids  int32 [T][k]   (out)
 *   topk_w    fp32  [T][k]   (out)
 *   logits    fp32  [T][E]   (out, nullable): the values described above,
 *             within the error bound of the exact fp32 logits.
 *   workspace >= moe_workspace_size(cfg) bytes (partial-logit scratch).
 * Defined by the router step of the grouped_mm path (unsloth commit
 * 80aaf1121b page, third paragraph; router fusion on the unsloth commit
 * a1bc5cbd page, first paragraph). */
moe_status moe_route(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T,
                     int32_t* topk_ids, float* topk_w, float* logits, void* workspace,
                     size_t ws_bytes, hipStream_t stream);

/* Bucketing of the T*k token-expert slots s = t*k + j by expert, with no
 * host synchronisation (the capture-safe replacement for bincount described
 * on the unsloth commit 80aaf1121b page, last paragraph):
 *   counts[e]   = number of slots routed to e                  int32 [E]
 *   offsets     = exclusive scan of counts, offsets[E] = T*k   int32 [E+1]
 *   perm[p]     = slot placed at position p, slots grouped by expert in
 *                 ascending expert order, ascending s inside a group
 *                 (a stable argsort of the flat ids)           int32 [T*k]
 *   pos[s]      = p with perm[p] = s (nullable)                int32 [T*k]
 *   workspace >= moe_workspace_size(cfg) bytes (chunk histograms at large T*k).
 * topk_ids values must lie in [0, E); an out-of-range id is clamped into
 * that range (the call stays memory-safe, its results are then unspecified). */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t T,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                       void* workspace, size_t ws_bytes, hipStream_t stream);

/* Whole block: route -> permute -> grouped gate/up with SiLU*up ->
 * grouped down -> per-token weighted combine (the router, bincount, cumsum,
 * argsort, grouped_mm and index_add_ steps of the grouped_mm MoE path on the
 * unsloth commit 80aaf1121b page, third paragraph; the result a plain tensor
 * as on the unsloth commit 4f2bfe7f69 page, second paragraph).
 *   x     bf16 [T][H]
 *   out   [T][H], fp32 or bf16 (cfg->out_dtype): out[t] = sum_{j ascending}
 *         topk_w[t][j] * y[t][j], formed in fp32 (bf16: then rounded to nearest even)
 *   workspace  >= moe_workspace_size(cfg) bytes, 256-byte aligned; its
 *              contents need no initialisation and are overwritten.
 * Calls sharing one workspace must be ordered on one stream. */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T,
                       void* out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument.  The workspace is a static device array inside the
 * library, 16 MiB on each GPU the library runs on, held until the process
 * ends; its address is looked up once per device on the first call there.
 * Same results as moe_forward(cfg, w, x, T, out, <workspace>, ...).  A
 * config whose moe_workspace_size() exceeds 16 MiB (the Qwen3-30B-A3B layer
 * in bf16 fits up to t_max = 192) -> MOE_ERR_WORKSPACE.  Every call on one GPU
 * shares that array and leaves its last contents there (nothing in it needs
 * to start at any value): calls that may overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller; calls on one stream
 * are ordered by the stream.  The routing arrays of the last call are not
 * exposed (moe_workspace_views needs a caller-owned workspace). */
moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T,
                               void* out, hipStream_t stream);

/* moe_forward that also records `events[0..5]` (host array of hipEvent_t
 * created by the caller) on `stream` before route, permute, gate/up, down,
 * combine and after combine, for per-stage timing.  Same results. */
moe_status moe_forward_timed(const moe_config* cfg, const moe_weights* w, const void* x,
                             int32_t T, void* out, void* workspace, size_t ws_bytes,
                             hipStream_t stream, hipEvent_t* events /* host, 6 */);

/* The pre-block step fused into the block's router pass (the layernorm +
 * residual + router fusion of the unsloth commit a1bc5cbd page, first
 * paragraph), per row t:
 *   r = bf16(residual + delta)                        (rounded once, nearest even)
 *   x = bf16(r / sqrt(mean_h(r^2) + eps) * gamma)     (formed in fp32, rounded once)
 * x is the block's input.  Every workgroup of the router pass that covers a
 * row forms the row's mean square in one fixed order, so x is the same
 * whatever the batch; an element of x may differ by one bf16 step from the
 * correctly rounded value only where that value lies within fp32 rounding
 * of a midpoint between two bf16 numbers. */
typedef struct {
  const void* residual;  /* bf16 [T][H]: the residual stream */
  const void* delta;     /* bf16 [T][H]: added to it first (the sublayer output), or NULL (r = residual) */
  const void* gamma;     /* bf16 [H]: the RMSNorm weight */
  float eps;             /* RMSNorm epsilon, finite and > 0 */
  void* residual_out;    /* bf16 [T][H]: r, or NULL */
  void* x_out;           /* bf16 [T][H]: x, which the rest of the block reads */
} moe_prenorm;

/* moe_forward with the pre-block step: x is formed from pn (see
 * moe_prenorm), written to pn->x_out (and r to pn->residual_out), then the
 * block runs on it; out, the routing arrays in the workspace and x_out are
 * bit-identical to moe_prenorm's x followed by moe_forward(x).  All pointers
 * 16-byte aligned; x_out and residual_out must not overlap residual, delta,
 * gamma or each other (the router pass reads whole rows in every workgroup
 * while others write) -> MOE_ERR_INVALID_ARG. */
moe_status moe_forward_prenorm(const moe_config* cfg, const moe_weights* w, const moe_prenorm* pn,
                               int32_t T, void* out, void* workspace, size_t ws_bytes,
                               hipStream_t stream);

/* Backward of the block for frozen weights: given dL/dout, the gradients
 * with respect to the block input x and to the routing weights, for the
 * routing the forward took (the top-k choice is piecewise constant in x):
 *   d_topk_w[t][j] = <d_out[t], y[t][j]>
 *   d_l[t][j]      = w_j (d_topk_w[t][j] - sum_i w_i d_topk_w[t][i])
 *   d_x[t]         = sum_j d_l[t][j] w_router[id_j]
 *                  + sum_j (W_gate^T d_g + W_up^T d_u) of slot t*k+j,
 *     d_h = W_down^T (w_j d_out[t]), d_g = d_h * u * silu'(g), d_u = d_h * silu(g),
 *     g, u the slot's gate/up pre-activations, which the forward kept.
 * Must follow moe_forward(cfg, w, x, T, ...) with cfg->train = 1 on the same
 * `workspace` and stream with no other use of the workspace in between: it
 * reads that call's routing arrays, per-slot y and pre-activations (and
 * overwrites y and the pre-activations).  Supported: tiled weights
 * (MOE_W_BF16_TILED, or MOE_W_NF4_B64_TILED as below), any T (where the
 * forward ran the MFMA prefill kernels, bf16 or 4-bit, the backward's
 * transposed products run as tiled GEMMs over the same 128-row work items);
 * else
 * MOE_ERR_UNSUPPORTED (cfg->train = 0 too).
 * With top-k weights without renormalisation (MOE_TOPK_SOFTMAX) the logit gradient
 * reaches every expert, d_l[e] = [e chosen] w_e d_topk_w_e - p_e sum_j w_j
 * d_topk_w_j with p the softmax over all E (from the router's approximate
 * logits, within ~1e-6 of the fp32 ones), and d_x's router share runs over
 * all E rows of w_router.  Sums run in a fixed order, no float atomics, so the result is
 * the same on every run.
 * With LoRA adapters (w->lora, the same ones the forward used) the chain
 * rule runs through W + scale * B A, and the adapters' gradients, summed
 * over every routed (token, expert) pair, are written to d_lora:
 *   d_B_d  = scale * sum d_y (A_d h)^T,       d_A_d  = scale * sum (B_d^T d_y) h^T
 *   d_B_gu = scale * sum [d_g; d_u] (A_gu x)^T,  d_A_gu = scale * sum (B_gu^T [d_g; d_u]) x^T
 * (d_y = w_j d_out[t]; h = silu(g) * u in fp32 from the kept g, u, which
 * also replaces the forward's A_d h rows in the workspace); an expert no
 * row reached gets zeros.  Needs 2 * I <= 4096.
 * With d_weights, also the gradients of the expert weights themselves,
 * summed over the routed pairs (the same expression with or without
 * adapters, since W + scale * B A has derivative 1 in W):
 *   d_W_gate_up[e] = sum [d_g; d_u] x^T,   d_W_down[e] = sum d_y h^T
 * (h = silu(g) * u in fp32 as above), zeros for an expert no row reached.
 * Bf16 weights only: with a 4-bit base (frozen) d_weights must be NULL, else
 * MOE_ERR_UNSUPPORTED.  With tiled 4-bit weights the transposed products run
 * over the codes, W[m][n] = codebook[code] * absmax[m][n / 64].
 *   d_out     fp32 [T][H]
 *   d_x       fp32 [T][H] (written)
 *   d_topk_w  fp32 [T][k] (written), or NULL
 *   d_lora    host pointer to the gradient arrays (device, written, shapes of
 *             moe_lora's arrays), non-NULL exactly when w->lora is
 *   d_weights host pointer to the expert-weight gradient arrays (device,
 *             written, 16-byte aligned), or NULL */
typedef struct {
  float* d_a_gate_up;  /* [E][r][H] */
  float* d_b_gate_up;  /* [E][2I][r] */
  float* d_a_down;     /* [E][r][I] */
  float* d_b_down;     /* [E][H][r] */
} moe_lora_grads;

typedef struct {
  float* d_w_gate_up;  /* [E][2I][H] fp32, row-major (gate rows, then up rows) */
  float* d_w_down;     /* [E][H][I] fp32, row-major */
} moe_weight_grads;

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T,
                        const float* d_out, float* d_x, float* d_topk_w, const moe_lora_grads* d_lora,
                        const moe_weight_grads* d_weights, void* workspace, size_t ws_bytes,
                        hipStream_t stream);

/* One-time conversion of row-major expert weights (cfg->wfmt = MOE_W_BF16 or
 * MOE_W_NF4_B64) into the tiled layout of MOE_W_BF16_TILED /
 * MOE_W_NF4_B64_TILED, in which every 16-row MFMA fragment of a k-step is
 * one contiguous kilobyte in the order the 64 lanes of a wave load it.  Per
 * expert, for a matrix of R rows x K columns (gate/up: R = 2I, K = H; down:
 * R = H, K = I), with rt < R/16, r < 16, g < 4:
 *   bf16    16-byte chunk (rt*K/32 + ks)*64 + 16g + r
 *             = W[16rt + r][32ks + 8g .. 32ks + 8g + 7]
 *   codes   16-byte chunk (rt*K/128 + kb)*64 + 16g + r; its 4-byte word st
 *             (st < 4) = codes of row 16rt + r for k in [128kb + 32st + 8g,
 *             128kb + 32st + 8g + 8)
 *   scales  float (rt*K/128 + kb)*32 + 2r + h = absmax of row 16rt + r,
 *             64-block 2kb + h
 * Writes dst's expert tensors (w_gate_up, w_down; or q_gate_up, s_gate_up,
 * q_down, s_down), caller-allocated with the source sizes and not
 * overlapping the source; other fields of dst are not touched.  Stream
 * ordered, no host synchronisation. */
moe_status moe_pack_weights(const moe_config* cfg, const moe_weights* src, const moe_weights* dst,
                            hipStream_t stream);

/* Device pointers of the routing arrays inside `workspace` (pure host
 * arithmetic; nothing is read from the device). */
moe_status moe_workspace_views(const moe_config* cfg, void* workspace, size_t ws_bytes,
                               moe_views* views /* host out */);

/* Copies counts[E] from a forward workspace to host memory and synchronises
 * the stream.  Refused with MOE_ERR_CAPTURE_VIOLATION on a capturing stream. */
moe_status moe_read_counts(const moe_config* cfg, const void* workspace, size_t ws_bytes,
                           int32_t* host_counts /* host, E */, hipStream_t stream);

/* Measurement aids (not part of the block): the achievable rates its
 * kernels are held to, timed by the caller around the call.
 * moe_probe_read streams `bytes` (a multiple of 16) from `src` once with the
 * load form the decode expert GEMMs stream weights with (16-byte
 * non-temporal loads, each wave instruction one contiguous KiB, each wave
 * walking its own contiguous range) and writes one XOR of the words each
 * wave read to `sink` (uint32 [n_wg * 4]), so no load can be dropped; n_wg
 * workgroups of 256 threads.
 * moe_probe_mfma runs n_wg workgroups of 4 waves, each wave issuing `iters`
 * rounds of independent bf16 MFMAs on register operands (shape 0: eight
 * 16x16x32, 131072 flops per round; shape 1: four 32x32x16, 131072 flops
 * per round), no memory traffic but `sink` (fp32 [n_wg * 256], the sums of
 * the accumulators).
 * moe_probe_gather copies 16-row x 64-byte tiles of `src` (rows of
 * `row_bytes`, a power of two >= 64; bytes / row_bytes a power of two >= 16,
 * bytes <= 2^31) global -> LDS with the LDS-DMA copy the prefill expert
 * GEMMs fetch gathered token rows with: each of the n_wg * 4 waves copies
 * `iters` tiles, tiles w, w + 4 n_wg, ... modulo the tile count, 8 per batch,
 * with the lanes one row each (order 0: lane l row l % 16, 16-byte chunk
 * l / 16) or four per 64-byte row segment (order 1: row l / 4, chunk l % 4),
 * and writes the XOR of the words each wave copied to `sink` (uint32
 * [n_wg * 4]); with iters * 4 n_wg equal to the tile count every word is
 * copied once.  Bad arguments -> MOE_ERR_INVALID_ARG. */
moe_status moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg, hipStream_t stream);
moe_status moe_probe_mfma(float* sink, int32_t n_wg, int32_t iters, int32_t shape, hipStream_t stream);
moe_status moe_probe_gather(const void* src, size_t bytes, int32_t row_bytes, int32_t order, int32_t iters,
                            uint32_t* sink, int32_t n_wg, hipStream_t stream);

/* Per-batch-size hipGraphs of moe_forward (the bucketed decode-step capture
 * of the unsloth commit 80aaf1121b page, second paragraph): one graph per
 * bucket size, all reading `x_static` (bf16 [t_max][H]) and writing
 * `out_static` ([t_max][H] in cfg->out_dtype) through one shared workspace.  Those
 * buffers and the weights must outlive the graph; their addresses are baked
 * in.  `buckets` (host) must be strictly ascending within [1, t_max].
 * `stream` must be a created stream (not NULL) that is not capturing.  On
 * any capture failure everything made so far is released, the stream is
 * left uncaptured and MOE_ERR_NOT_CAPTURABLE is returned, so the caller can
 * run moe_forward eagerly instead. */
typedef struct moe_graph moe_graph;
moe_status moe_graph_capture(const moe_config* cfg, const moe_weights* w, const int32_t* buckets,
                             int32_t n_buckets, const void* x_static, void* out_static,
                             void* workspace, size_t ws_bytes, hipStream_t stream,
                             moe_graph** graph /* host out */);

/* moe_graph_capture of moe_forward_prenorm: the graphs read the buffers of
 * `pn_static` ([t_max][H] each; gamma [H]) and write its x_out, residual_out
 * and `out_static`; replay as above (rows [T, bucket) of x_out and
 * residual_out are left untouched too). */
moe_status moe_graph_capture_prenorm(const moe_config* cfg, const moe_weights* w, const int32_t* buckets,
                                     int32_t n_buckets, const moe_prenorm* pn_static, void* out_static,
                                     void* workspace, size_t ws_bytes, hipStream_t stream,
                                     moe_graph** graph /* host out */);

/* Launches the graph of the smallest bucket >= T on `stream` (the replay of
 * the bucket captured for a batch size, with the batch's rows copied into
 * the static input first and the output rows read back from the static
 * output, on the unsloth commit 80aaf1121b page, second paragraph).  The
 * graph's first node, the router's first kernel, also writes the live row
 * count T into the workspace, and the later kernels read it there: rows
 * [T, bucket) of x_static are routed to no expert and counted nowhere
 * (counts sum to T*k), and rows [T, bucket) of out_static are left
 * untouched; rows < T are bit-identical to moe_forward of those T rows.
 * When T differs from the previous replay of the same graph, that node's
 * argument is updated on the host first (no extra launch).  So whatever was written to the workspace between replays
 * (eager calls, other graphs on it, any fill) does not change a replay's
 * result.  A graph must be replayed from one thread at a time.
 * T larger than the largest bucket -> MOE_ERR_INVALID_ARG. */
moe_status moe_graph_replay(moe_graph* graph, int32_t T, hipStream_t stream);

/* Bucket size moe_graph_replay(graph, T) would use, or -1. */
int32_t moe_graph_bucket_for(const moe_graph* graph, int32_t T);

/* Releases the graphs (NULL is a no-op).  Do not replay afterwards. */
void moe_graph_destroy(moe_graph* graph);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
