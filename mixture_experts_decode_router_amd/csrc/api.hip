// Host implementation of the C ABI in include/moe.h: argument validation,
// workspace carve-up, stream-ordered launches and per-bucket hipGraphs.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "moe.h"

// Device scratch of moe_forward_noalloc: one array per GPU, in the code
// object, so the call needs no allocation.  Host code uses only the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in there), fetched on the first call on each device.
constexpr size_t kNoAllocScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t ids, wts, counts, offsets, perm, pos, items, n_items, live, route, chunks, h, y, u_gu, u_d, gu, gub, z_gu,
      z_d, total;
  int max_items;
};

// bound on the work-list length: sum over experts of ceil(c_e / tile)
// rounded up to a multiple of group
int max_items_for(int N, int E, int tile = moe::kSkinnyTile, int group = 1) {
  return std::min(E, N) * group + (N + tile - 1) / tile;
}

Layout layout(const moe_config& c) {
  Layout L{};
  const size_t N = (size_t)c.t_max * c.top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  L.max_items = std::max(max_items_for((int)N, c.n_experts),
                         max_items_for((int)N, c.n_experts, moe::kMfmaTile));
  L.ids = take(N * 4);
  L.wts = take(N * 4);
  L.counts = take((size_t)c.n_experts * 4);
  L.offsets = take((size_t)(c.n_experts + 1) * 4);
  L.perm = take(N * 4);
  L.pos = take(N * 4);
  L.items = take((size_t)L.max_items * 8);
  L.n_items = take(4);
  L.live = take(4);
  L.route = take(moe::route_scratch_floats(c.t_max, c.n_experts, c.hidden) * 4);
  L.chunks = take(moe::permute_scratch_ints((int)N, c.n_experts) * 4);
  L.h = take(N * c.inter * 2);
  L.y = take(N * c.hidden * 4);
  L.u_gu = take(N * 16 * 4);  // LoRA: A_gu x per routed row
  L.u_d = take(N * 16 * 4);   // LoRA: A_d h per routed row
  L.gu = take(c.train ? N * 2 * c.inter * 4 : 0);  // training forward: gate/up pre-activations
  L.gub = take(c.train ? N * 2 * c.inter * 2 : 0);  // backward: d_g, d_u in bf16 (tiled bf16 weights)
  L.z_gu = take(c.train ? N * 16 * 4 : 0);         // LoRA backward: B_gu^T [d_g; d_u] per routed row
  L.z_d = take(c.train ? N * 16 * 4 : 0);          // LoRA backward: B_d^T d_y per routed row
  L.total = off;
  return L;
}

moe_status check_cfg(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  char buf[256];
  if (c->hidden < 128 || c->hidden > 4096 || c->hidden % 128 ||
      c->inter < 128 || c->inter > 4096 || c->inter % 128 ||
      c->n_experts < 16 || c->n_experts > 256 || c->n_experts % 16 || c->top_k < 1 ||
      c->top_k > 16 || c->top_k > c->n_experts || c->wfmt < MOE_W_BF16 || c->wfmt > MOE_W_NF4_B64_TILED) {
    snprintf(buf, sizeof buf, "unsupported shape: hidden=%d inter=%d n_experts=%d top_k=%d wfmt=%d",
             c->hidden, c->inter, c->n_experts, c->top_k, c->wfmt);
    return fail(MOE_ERR_UNSUPPORTED, buf);
  }
  if (c->t_max < 1 || (long long)c->t_max * c->top_k > 65536) {
    snprintf(buf, sizeof buf, "t_max=%d out of range (need 1 <= t_max and t_max*top_k <= 65536)", c->t_max);
    return fail(MOE_ERR_UNSUPPORTED, buf);
  }
  if ((c->out_dtype != MOE_OUT_F32 && c->out_dtype != MOE_OUT_BF16) ||
      (c->topk_weights != MOE_TOPK_RENORM && c->topk_weights != MOE_TOPK_SOFTMAX) || (c->train != 0 && c->train != 1)) {
    snprintf(buf, sizeof buf, "unsupported out_dtype=%d, topk_weights=%d or train=%d", c->out_dtype, c->topk_weights,
             c->train);
    return fail(MOE_ERR_UNSUPPORTED, buf);
  }
  return MOE_OK;
}

moe_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, align)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned");
  return MOE_OK;
}

#define MOE_TRY(x)                   \
  do {                               \
    moe_status _s = (x);             \
    if (_s != MOE_OK) return _s;     \
  } while (0)

bool is_nf4(const moe_config& c) { return c.wfmt == MOE_W_NF4_B64 || c.wfmt == MOE_W_NF4_B64_TILED; }

bool is_tiled(const moe_config& c) { return c.wfmt == MOE_W_BF16_TILED || c.wfmt == MOE_W_NF4_B64_TILED; }
// Large groups (on average >= 32 rows per expert) go to the LDS-tiled MFMA
// kernels (tiled weights, bf16 or 4-bit, with or without LoRA adapters, in
// inference and in training, whose backward then runs over the same 128-row
// work items); they give the same per-row bits as the 16-row kernels.
bool mfma_path_for(const moe_config& c, int T) {
  return is_tiled(c) && (long)T * c.top_k >= 32L * c.n_experts;
}

moe_status check_weights(const moe_config& c, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_TRY(check_ptr(w->w_router, "w_router"));
  if (w->router_bias && !aligned(w->router_bias, 4))
    return fail(MOE_ERR_INVALID_ARG, "router_bias is not 4-byte aligned");
  if (!is_nf4(c)) {
    MOE_TRY(check_ptr(w->w_gate_up, "w_gate_up"));
    MOE_TRY(check_ptr(w->w_down, "w_down"));
  } else {
    MOE_TRY(check_ptr(w->q_gate_up, "q_gate_up"));
    MOE_TRY(check_ptr(w->s_gate_up, "s_gate_up"));
    MOE_TRY(check_ptr(w->q_down, "q_down"));
    MOE_TRY(check_ptr(w->s_down, "s_down"));
    MOE_TRY(check_ptr(w->codebook, "codebook"));
  }
  if (w->lora) {
    const moe_lora& l = *w->lora;
    if (l.rank != 16) return fail(MOE_ERR_UNSUPPORTED, "LoRA rank " + std::to_string(l.rank) + " (16 is supported)");
    MOE_TRY(check_ptr(l.a_gate_up, "lora a_gate_up"));
    MOE_TRY(check_ptr(l.b_gate_up, "lora b_gate_up"));
    MOE_TRY(check_ptr(l.a_down, "lora a_down"));
    MOE_TRY(check_ptr(l.b_down, "lora b_down"));
    if (!std::isfinite(l.scale)) return fail(MOE_ERR_INVALID_ARG, "LoRA scale is not finite");
  }
  return MOE_OK;
}

moe_status check_T(const moe_config& c, int32_t T) {
  if (T < 1 || T > c.t_max) {
    char buf[128];
    snprintf(buf, sizeof buf, "T=%d outside [1, t_max=%d]", T, c.t_max);
    return fail(MOE_ERR_INVALID_ARG, buf);
  }
  return MOE_OK;
}

moe_status check_ws(const moe_config& c, const void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const size_t need = layout(c).total;
  if (ws_bytes < need) {
    char buf[128];
    snprintf(buf, sizeof buf, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    return fail(MOE_ERR_WORKSPACE, buf);
  }
  return MOE_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Enqueues the whole block; arguments already validated.
// live: device row count for graph replays of a larger bucket (rows >= *live
// are routed nowhere and not written), or null for an eager call of T rows.
// pn: fuse the pre-block step into the router pass; x is then its output.
// rnode: receives the router's first kernel launch (graph captures), or null.
moe_status enqueue_forward(const moe_config& c, const moe_weights& w, const void* x, int32_t T, void* out,
                           void* ws, hipStream_t s, hipEvent_t* ev, const int32_t* live = nullptr,
                           const moe::PrenormArgs* pn = nullptr, moe::RouteNode* rnode = nullptr) {
  const Layout L = layout(c);
  const int N = T * c.top_k;
  hipError_t e;
  auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], s) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "hipEventRecord");

  moe::RouteArgs ra{};
  ra.x = static_cast<const uint16_t*>(x);
  ra.wr = static_cast<const uint16_t*>(w.w_router);
  ra.bias = w.router_bias;
  ra.T = T;
  ra.H = c.hidden;
  ra.E = c.n_experts;
  ra.k = c.top_k;
  ra.ids = at<int32_t>(ws, L.ids);
  ra.wts = at<float>(ws, L.wts);
  ra.logits = nullptr;
  ra.live = live;
  ra.softmax_all = c.topk_weights == MOE_TOPK_SOFTMAX;
  ra.pn = pn;

  // both paths give bit-identical per-row results
  const bool mfma_path = mfma_path_for(c, T);
  const int tile = mfma_path ? moe::kMfmaTile : moe::kSkinnyTile;
  moe::PermuteArgs pa{};
  pa.ids = ra.ids;
  pa.N = N;
  pa.E = c.n_experts;
  pa.tile = tile;
  pa.group = 1;
  pa.counts = at<int32_t>(ws, L.counts);
  pa.offsets = at<int32_t>(ws, L.offsets);
  pa.perm = at<int32_t>(ws, L.perm);
  pa.pos = at<int32_t>(ws, L.pos);
  pa.items = at<int32_t>(ws, L.items);
  pa.n_items = at<int32_t>(ws, L.n_items);
  pa.chunk_base = at<int32_t>(ws, L.chunks);
  pa.live = live;
  pa.k = c.top_k;
  // most experts hold rows: the 16-row kernels find their slots themselves
  // (no bucketing launch); else a small batch is bucketed by the router's
  // select workgroup, a larger one by the bucketing kernel
  const bool direct = !mfma_path && !is_nf4(c) && !w.lora && !c.train && N >= 2 * c.n_experts &&
                      N <= moe::kDirectMaxN;
  bool fused = false;
  if ((e = moe::launch_route(ra, at<float>(ws, L.route), s, direct ? nullptr : &pa, &fused, rnode)) != hipSuccess)
    return hip_fail(e, "route launch");
  if ((e = mark(1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (!direct && !fused && (e = moe::launch_permute(pa, s)) != hipSuccess) return hip_fail(e, "permute launch");
  if ((e = mark(2)) != hipSuccess) return hip_fail(e, "hipEventRecord");

  moe::ExpertArgs ea{};
  ea.counts = pa.counts;
  ea.offsets = pa.offsets;
  ea.perm = pa.perm;
  ea.items = pa.items;
  ea.n_items = pa.n_items;
  ea.max_items = max_items_for(N, c.n_experts, tile, pa.group);
  ea.H = c.hidden;
  ea.I = c.inter;
  ea.E = c.n_experts;
  ea.k = c.top_k;
  ea.x = ra.x;
  ea.h = at<uint16_t>(ws, L.h);
  ea.gu = c.train ? at<float>(ws, L.gu) : nullptr;
  ea.y = at<float>(ws, L.y);
  ea.w_gate_up = static_cast<const uint16_t*>(w.w_gate_up);
  ea.w_down = static_cast<const uint16_t*>(w.w_down);
  ea.q_gate_up = w.q_gate_up;
  ea.s_gate_up = w.s_gate_up;
  ea.q_down = w.q_down;
  ea.s_down = w.s_down;
  ea.codebook = w.codebook;
  if (direct) {
    ea.ids = ra.ids;
    ea.N = N;
    ea.live = live;
    ea.r_counts = pa.counts;
    ea.r_offsets = pa.offsets;
    ea.r_perm = pa.perm;
    ea.r_pos = pa.pos;
  }
  const bool nf4 = is_nf4(c), tiled = is_tiled(c);
  moe::LoraAArgs la{};
  if (w.lora) {  // adapter terms in the expert kernels' epilogues, at every size
    ea.lora = true;
    ea.lora_scale = w.lora->scale;
    ea.lb_gate_up = w.lora->b_gate_up;
    ea.lb_down = w.lora->b_down;
    ea.u_gate_up = at<float>(ws, L.u_gu);
    ea.u_down = at<float>(ws, L.u_d);
    la.counts = pa.counts;
    la.offsets = pa.offsets;
    la.perm = pa.perm;
    la.items = pa.items;
    la.n_items = pa.n_items;
    la.max_items = ea.max_items;
    la.subs = tile / moe::kSkinnyTile;
    la.k = c.top_k;
    la.K = c.hidden;
    la.src = ea.x;
    la.by_token = true;
    la.A = w.lora->a_gate_up;
    la.U = at<float>(ws, L.u_gu);
    if ((e = moe::launch_lora_a(la, s)) != hipSuccess) return hip_fail(e, "LoRA A launch");
  }
  e = mfma_path ? (nf4 ? moe::launch_gate_up_mfma_nf4(ea, s) : moe::launch_gate_up_mfma(ea, s))
                : moe::launch_gate_up(ea, nf4, tiled, s);
  if (e != hipSuccess) return hip_fail(e, "gate/up launch");
  if ((e = mark(3)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (w.lora) {
    la.K = c.inter;
    la.src = ea.h;
    la.by_token = false;
    la.A = w.lora->a_down;
    la.U = at<float>(ws, L.u_d);
    if ((e = moe::launch_lora_a(la, s)) != hipSuccess) return hip_fail(e, "LoRA A launch");
  }
  e = mfma_path ? (nf4 ? moe::launch_down_mfma_nf4(ea, s) : moe::launch_down_mfma(ea, s))
                : moe::launch_down(ea, nf4, tiled, s);
  if (e != hipSuccess) return hip_fail(e, "down launch");
  if ((e = mark(4)) != hipSuccess) return hip_fail(e, "hipEventRecord");

  moe::CombineArgs ca{};
  ca.y = ea.y;
  ca.wts = ra.wts;
  ca.out = out;
  ca.T = T;
  ca.H = c.hidden;
  ca.k = c.top_k;
  ca.live = live;
  ca.out_bf16 = c.out_dtype == MOE_OUT_BF16;
  if ((e = moe::launch_combine(ca, s)) != hipSuccess) return hip_fail(e, "combine launch");
  if ((e = mark(5)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return MOE_OK;
}

moe_status check_forward_args(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T,
                              const void* out, const void* ws, size_t ws_bytes) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_weights(*cfg, w));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(out, "out"));
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  return MOE_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

// pn for rows [0, rows): pointers, eps, and no output overlapping an input
moe_status check_prenorm(const moe_config& c, const moe_prenorm* pn, int32_t rows, moe::PrenormArgs* out) {
  if (!pn) return fail(MOE_ERR_INVALID_ARG, "prenorm is NULL");
  MOE_TRY(check_ptr(pn->residual, "residual"));
  MOE_TRY(check_ptr(pn->gamma, "gamma"));
  MOE_TRY(check_ptr(pn->x_out, "x_out"));
  if (pn->delta) MOE_TRY(check_ptr(pn->delta, "delta"));
  if (pn->residual_out) MOE_TRY(check_ptr(pn->residual_out, "residual_out"));
  if (!(std::isfinite(pn->eps) && pn->eps > 0.f)) return fail(MOE_ERR_INVALID_ARG, "eps must be finite and > 0");
  const size_t nb = (size_t)rows * c.hidden * 2, gb = (size_t)c.hidden * 2;
  const void* ins[3] = {pn->residual, pn->delta, pn->gamma};
  const size_t in_b[3] = {nb, nb, gb};
  const void* outs[2] = {pn->x_out, pn->residual_out};
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[o], nb, ins[i], in_b[i]))
        return fail(MOE_ERR_INVALID_ARG, "x_out / residual_out must not overlap residual, delta or gamma");
  if (overlaps(pn->x_out, nb, pn->residual_out, nb))
    return fail(MOE_ERR_INVALID_ARG, "x_out and residual_out overlap");
  out->res = static_cast<const uint16_t*>(pn->residual);
  out->delta = static_cast<const uint16_t*>(pn->delta);
  out->gamma = static_cast<const uint16_t*>(pn->gamma);
  out->eps = pn->eps;
  out->res_out = static_cast<uint16_t*>(pn->residual_out);
  return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

struct moe_graph {
  moe_config cfg;
  std::vector<int32_t> buckets;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
  // each graph's first node (the router's first kernel) also writes the live
  // row count the later kernels read; its argument is the row count of that
  // graph's last replay
  std::vector<hipGraphNode_t> live_nodes;
  std::vector<moe::RouteNode> live_launch;
  std::vector<int32_t> live_vals;
  int32_t* live = nullptr;  // device row count read by the captured kernels (in the workspace)
};

static void graph_release(moe_graph* g) {
  for (auto ge : g->execs)
    if (ge) (void)hipGraphExecDestroy(ge);
  for (auto gr : g->graphs)
    if (gr) (void)hipGraphDestroy(gr);
  delete g;
}

extern "C" {

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_NOT_CAPTURABLE: return "MOE_ERR_NOT_CAPTURABLE";
    case MOE_ERR_CAPTURE_VIOLATION: return "MOE_ERR_CAPTURE_VIOLATION";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_config_check(const moe_config* cfg) { return check_cfg(cfg); }

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  return layout(*cfg).total;
}

moe_status moe_route(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, int32_t* topk_ids,
                     float* topk_w, float* logits, void* workspace, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_TRY(check_ptr(w->w_router, "w_router"));
  if (w->router_bias && !aligned(w->router_bias, 4))
    return fail(MOE_ERR_INVALID_ARG, "router_bias is not 4-byte aligned");
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(topk_ids, "topk_ids", 4));
  MOE_TRY(check_ptr(topk_w, "topk_w", 4));
  if (logits && !aligned(logits, 4)) return fail(MOE_ERR_INVALID_ARG, "logits is not 4-byte aligned");
  MOE_TRY(check_ws(*cfg, workspace, ws_bytes));
  moe::RouteArgs ra{};
  ra.x = static_cast<const uint16_t*>(x);
  ra.wr = static_cast<const uint16_t*>(w->w_router);
  ra.bias = w->router_bias;
  ra.T = T;
  ra.H = cfg->hidden;
  ra.E = cfg->n_experts;
  ra.k = cfg->top_k;
  ra.ids = topk_ids;
  ra.wts = topk_w;
  ra.softmax_all = cfg->topk_weights == MOE_TOPK_SOFTMAX;
  ra.logits = logits;
  const hipError_t e = moe::launch_route(ra, at<float>(workspace, layout(*cfg).route), stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "route launch");
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t T, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* pos, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_ptr(topk_ids, "topk_ids", 4));
  MOE_TRY(check_ptr(counts, "counts", 4));
  MOE_TRY(check_ptr(offsets, "offsets", 4));
  MOE_TRY(check_ptr(perm, "perm", 4));
  if (pos && !aligned(pos, 4)) return fail(MOE_ERR_INVALID_ARG, "pos is not 4-byte aligned");
  MOE_TRY(check_ws(*cfg, workspace, ws_bytes));
  moe::PermuteArgs pa{};
  pa.ids = topk_ids;
  pa.N = T * cfg->top_k;
  pa.E = cfg->n_experts;
  pa.tile = 0;
  pa.group = 1;
  pa.counts = counts;
  pa.offsets = offsets;
  pa.perm = perm;
  pa.pos = pos;
  pa.items = nullptr;
  pa.n_items = nullptr;
  pa.chunk_base = at<int32_t>(workspace, layout(*cfg).chunks);
  const hipError_t e = moe::launch_permute(pa, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "permute launch");
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, void* out,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_forward_args(cfg, w, x, T, out, workspace, ws_bytes));
  return enqueue_forward(*cfg, *w, x, T, out, workspace, stream, nullptr);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, void* out,
                               hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const size_t need = layout(*cfg).total;
  if (need > kNoAllocScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "config needs " + std::to_string(need) + " bytes of workspace; the static scratch "
                                   "holds " + std::to_string(kNoAllocScratchBytes) + " (use moe_forward with a workspace)");
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  MOE_TRY(check_forward_args(cfg, w, x, T, out, ws, need));
  return enqueue_forward(*cfg, *w, x, T, out, ws, stream, nullptr);
}

moe_status moe_forward_prenorm(const moe_config* cfg, const moe_weights* w, const moe_prenorm* pn, int32_t T,
                               void* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!pn) return fail(MOE_ERR_INVALID_ARG, "prenorm is NULL");
  MOE_TRY(check_forward_args(cfg, w, pn->x_out, T, out, workspace, ws_bytes));
  moe::PrenormArgs pa{};
  MOE_TRY(check_prenorm(*cfg, pn, T, &pa));
  return enqueue_forward(*cfg, *w, pn->x_out, T, out, workspace, stream, nullptr, nullptr, &pa);
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, const float* d_out,
                        float* d_x, float* d_topk_w, const moe_lora_grads* d_lora, const moe_weight_grads* d_weights,
                        void* workspace, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_forward_args(cfg, w, x, T, d_x, workspace, ws_bytes));
  const moe_config& c = *cfg;
  if (c.train != 1 || (c.wfmt != MOE_W_BF16_TILED && c.wfmt != MOE_W_NF4_B64_TILED))
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward supports train=1 configs with tiled bf16 or 4-bit weights");
  if (d_weights && c.wfmt != MOE_W_BF16_TILED)
    return fail(MOE_ERR_UNSUPPORTED, "expert-weight gradients need bf16 weights (a 4-bit base is frozen)");
  MOE_TRY(check_ptr(d_out, "d_out"));
  if (d_topk_w && !aligned(d_topk_w, 4)) return fail(MOE_ERR_INVALID_ARG, "d_topk_w is not 4-byte aligned");
  if (!w->lora != !d_lora)
    return fail(MOE_ERR_INVALID_ARG, w->lora ? "adapters given but d_lora is NULL" : "d_lora given without adapters");
  if (w->lora) {
    if (2 * c.inter > 4096) return fail(MOE_ERR_UNSUPPORTED, "the LoRA backward needs 2*inter <= 4096");
    MOE_TRY(check_ptr(d_lora->d_a_gate_up, "d_a_gate_up"));
    MOE_TRY(check_ptr(d_lora->d_b_gate_up, "d_b_gate_up"));
    MOE_TRY(check_ptr(d_lora->d_a_down, "d_a_down"));
    MOE_TRY(check_ptr(d_lora->d_b_down, "d_b_down"));
  }
  if (d_weights) {
    MOE_TRY(check_ptr(d_weights->d_w_gate_up, "d_w_gate_up"));
    MOE_TRY(check_ptr(d_weights->d_w_down, "d_w_down"));
  }
  const Layout L = layout(c);
  const int N = T * c.top_k;
  moe::BwdArgs b{};
  b.T = T;
  b.H = c.hidden;
  b.I = c.inter;
  b.E = c.n_experts;
  b.k = c.top_k;
  b.max_items = max_items_for(N, c.n_experts, moe::kSkinnyTile, 1);
  b.ids = at<int32_t>(workspace, L.ids);
  b.counts = at<int32_t>(workspace, L.counts);
  b.offsets = at<int32_t>(workspace, L.offsets);
  b.perm = at<int32_t>(workspace, L.perm);
  b.items = at<int32_t>(workspace, L.items);
  b.n_items = at<int32_t>(workspace, L.n_items);
  b.wts = at<float>(workspace, L.wts);
  b.y = at<float>(workspace, L.y);
  b.d_out = d_out;
  b.d_x = d_x;
  b.d_w = d_topk_w;
  b.w_router = static_cast<const uint16_t*>(w->w_router);
  b.w_gate_up = static_cast<const uint16_t*>(w->w_gate_up);
  b.w_down = static_cast<const uint16_t*>(w->w_down);
  if (is_nf4(c)) {
    b.nf4 = true;
    b.q_gate_up = w->q_gate_up;
    b.s_gate_up = w->s_gate_up;
    b.q_down = w->q_down;
    b.s_down = w->s_down;
    b.codebook = w->codebook;
  }
  b.gu = at<float>(workspace, L.gu);
  b.gub = at<uint16_t>(workspace, L.gub);
  b.d_xs = at<float>(workspace, L.y);  // y is read first, then its memory holds the per-slot d_x
  b.x = static_cast<const uint16_t*>(x);
  if (c.topk_weights == MOE_TOPK_SOFTMAX) {
    b.unrenorm = true;
    b.r_part = at<float>(workspace, L.route);
    b.r_nst = moe::route_stored_splits(T, c.hidden);
    b.r_bias = w->router_bias;
  }
  if (d_weights) {
    b.wgrad = true;
    b.g_w_gate_up = d_weights->d_w_gate_up;
    b.g_w_down = d_weights->d_w_down;
  }
  if (w->lora) {
    const moe_lora& l = *w->lora;
    b.lora = true;
    b.lora_scale = l.scale;
    b.h = at<uint16_t>(workspace, L.h);
    b.la_gate_up = l.a_gate_up;
    b.lb_gate_up = l.b_gate_up;
    b.la_down = l.a_down;
    b.lb_down = l.b_down;
    b.u_gate_up = at<float>(workspace, L.u_gu);
    b.u_down = at<float>(workspace, L.u_d);
    b.z_gate_up = at<float>(workspace, L.z_gu);
    b.z_down = at<float>(workspace, L.z_d);
    b.g_a_gate_up = d_lora->d_a_gate_up;
    b.g_b_gate_up = d_lora->d_b_gate_up;
    b.g_a_down = d_lora->d_a_down;
    b.g_b_down = d_lora->d_b_down;
    // y's memory is free while the adapter gradients are formed (read by the
    // routing-weight gradients before, rewritten by the gate/up pass after)
    b.lora_part = at<float>(workspace, L.y);
    b.lora_part_floats = (size_t)c.t_max * c.top_k * c.hidden;
  }
  hipError_t e;
  // the transposed products run over the forward's work list: 16-row items
  // (the 16-row GEMVs) or, after the MFMA forward, 128-row items (the tiled
  // transposed GEMMs); the adapter kernels take 16-row sub-tiles of either
  b.row_tiles = mfma_path_for(c, T) ? moe::kMfmaTile / moe::kSkinnyTile : 1;
  b.max_items = max_items_for(N, c.n_experts, moe::kSkinnyTile * b.row_tiles, 1);
  // the down-adapter and down-weight gradients read g, u, so they come
  // before the down pass turns those into d_g, d_u; the gate/up ones after it
  if ((e = moe::launch_bwd_weights(b, stream)) != hipSuccess) return hip_fail(e, "backward weights launch");
  if (b.lora) {
    if ((e = moe::launch_lora_bt(b, true, stream)) != hipSuccess) return hip_fail(e, "LoRA down B^T launch");
    if ((e = moe::launch_lora_grad(b, true, stream)) != hipSuccess) return hip_fail(e, "LoRA down gradient launch");
  }
  if (b.wgrad && c.inter <= c.hidden) {
    // y has been read: its memory holds the fp32 h of every routed row until
    // the gate/up pass writes the per-slot d_x there
    float* hf = at<float>(workspace, L.y);
    if ((e = moe::launch_h(b, hf, stream)) != hipSuccess) return hip_fail(e, "h launch");
    b.hf = hf;
  }
  if (b.wgrad && (e = moe::launch_wgrad(b, true, stream)) != hipSuccess)
    return hip_fail(e, "down weight gradient launch");
  b.hf = nullptr;
  if ((e = moe::launch_bwd_t(b, true, stream)) != hipSuccess) return hip_fail(e, "backward down launch");
  if (b.lora) {
    if ((e = moe::launch_lora_bt(b, false, stream)) != hipSuccess) return hip_fail(e, "LoRA gate/up B^T launch");
    if ((e = moe::launch_lora_grad(b, false, stream)) != hipSuccess)
      return hip_fail(e, "LoRA gate/up gradient launch");
  }
  if (b.wgrad && (e = moe::launch_wgrad(b, false, stream)) != hipSuccess)
    return hip_fail(e, "gate/up weight gradient launch");
  if ((e = moe::launch_bwd_t(b, false, stream)) != hipSuccess) return hip_fail(e, "backward gate/up launch");
  if ((e = moe::launch_bwd_combine(b, stream)) != hipSuccess) return hip_fail(e, "backward combine launch");
  return MOE_OK;
}

moe_status moe_forward_timed(const moe_config* cfg, const moe_weights* w, const void* x, int32_t T, void* out,
                             void* workspace, size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  MOE_TRY(check_forward_args(cfg, w, x, T, out, workspace, ws_bytes));
  if (!events) return fail(MOE_ERR_INVALID_ARG, "events is NULL");
  for (int i = 0; i < 6; ++i)
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[i] is NULL");
  return enqueue_forward(*cfg, *w, x, T, out, workspace, stream, events);
}

moe_status moe_pack_weights(const moe_config* cfg, const moe_weights* src, const moe_weights* dst,
                            hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->wfmt != MOE_W_BF16 && cfg->wfmt != MOE_W_NF4_B64)
    return fail(MOE_ERR_INVALID_ARG, "moe_pack_weights converts from a row-major format (MOE_W_BF16 or MOE_W_NF4_B64)");
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  moe::PackArgs pa{};
  pa.nf4 = is_nf4(*cfg);
  pa.E = cfg->n_experts;
  pa.H = cfg->hidden;
  pa.I = cfg->inter;
  if (!pa.nf4) {
    MOE_TRY(check_ptr(src->w_gate_up, "src w_gate_up"));
    MOE_TRY(check_ptr(src->w_down, "src w_down"));
    MOE_TRY(check_ptr(dst->w_gate_up, "dst w_gate_up"));
    MOE_TRY(check_ptr(dst->w_down, "dst w_down"));
    if (src->w_gate_up == dst->w_gate_up || src->w_down == dst->w_down)
      return fail(MOE_ERR_INVALID_ARG, "packing cannot be done in place");
    pa.src_gate_up = src->w_gate_up;
    pa.src_down = src->w_down;
    pa.dst_gate_up = const_cast<void*>(dst->w_gate_up);
    pa.dst_down = const_cast<void*>(dst->w_down);
  } else {
    MOE_TRY(check_ptr(src->q_gate_up, "src q_gate_up"));
    MOE_TRY(check_ptr(src->s_gate_up, "src s_gate_up"));
    MOE_TRY(check_ptr(src->q_down, "src q_down"));
    MOE_TRY(check_ptr(src->s_down, "src s_down"));
    MOE_TRY(check_ptr(dst->q_gate_up, "dst q_gate_up"));
    MOE_TRY(check_ptr(dst->s_gate_up, "dst s_gate_up"));
    MOE_TRY(check_ptr(dst->q_down, "dst q_down"));
    MOE_TRY(check_ptr(dst->s_down, "dst s_down"));
    if (src->q_gate_up == dst->q_gate_up || src->q_down == dst->q_down || src->s_gate_up == dst->s_gate_up ||
        src->s_down == dst->s_down)
      return fail(MOE_ERR_INVALID_ARG, "packing cannot be done in place");
    pa.src_gate_up = src->q_gate_up;
    pa.src_down = src->q_down;
    pa.src_s_gate_up = src->s_gate_up;
    pa.src_s_down = src->s_down;
    pa.dst_gate_up = const_cast<uint8_t*>(dst->q_gate_up);
    pa.dst_down = const_cast<uint8_t*>(dst->q_down);
    pa.dst_s_gate_up = const_cast<float*>(dst->s_gate_up);
    pa.dst_s_down = const_cast<float*>(dst->s_down);
  }
  const hipError_t e = moe::launch_pack(pa, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "pack launch");
}

moe_status moe_workspace_views(const moe_config* cfg, void* workspace, size_t ws_bytes, moe_views* v) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_ws(*cfg, workspace, ws_bytes));
  if (!v) return fail(MOE_ERR_INVALID_ARG, "views is NULL");
  const Layout L = layout(*cfg);
  v->topk_ids = at<int32_t>(workspace, L.ids);
  v->topk_w = at<float>(workspace, L.wts);
  v->counts = at<int32_t>(workspace, L.counts);
  v->offsets = at<int32_t>(workspace, L.offsets);
  v->perm = at<int32_t>(workspace, L.perm);
  v->pos = at<int32_t>(workspace, L.pos);
  return MOE_OK;
}

moe_status moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg, hipStream_t stream) {
  MOE_TRY(check_ptr(src, "src"));
  MOE_TRY(check_ptr(sink, "sink", 4));
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (n_wg < 1 || n_wg > 65536) return fail(MOE_ERR_INVALID_ARG, "n_wg must lie in [1, 65536]");
  const hipError_t e = moe::launch_probe_read(src, bytes, sink, n_wg, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "probe launch");
}

moe_status moe_probe_mfma(float* sink, int32_t n_wg, int32_t iters, int32_t shape, hipStream_t stream) {
  MOE_TRY(check_ptr(sink, "sink", 4));
  if (n_wg < 1 || n_wg > 65536) return fail(MOE_ERR_INVALID_ARG, "n_wg must lie in [1, 65536]");
  if (iters < 1) return fail(MOE_ERR_INVALID_ARG, "iters must be >= 1");
  if (shape != 0 && shape != 1) return fail(MOE_ERR_INVALID_ARG, "shape must be 0 (16x16x32) or 1 (32x32x16)");
  const hipError_t e = moe::launch_probe_mfma(sink, n_wg, iters, shape, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "probe launch");
}

moe_status moe_probe_gather(const void* src, size_t bytes, int32_t row_bytes, int32_t order, int32_t iters,
                            uint32_t* sink, int32_t n_wg, hipStream_t stream) {
  MOE_TRY(check_ptr(src, "src"));
  MOE_TRY(check_ptr(sink, "sink", 4));
  auto pow2 = [](size_t v) { return v != 0 && (v & (v - 1)) == 0; };
  if (row_bytes < 64 || !pow2((size_t)row_bytes))
    return fail(MOE_ERR_INVALID_ARG, "row_bytes must be a power of two >= 64");
  if (bytes % (size_t)row_bytes || !pow2(bytes / (size_t)row_bytes) || bytes / (size_t)row_bytes < 16 ||
      bytes > ((size_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "bytes / row_bytes must be a power of two >= 16, bytes <= 2^31");
  if (order != 0 && order != 1) return fail(MOE_ERR_INVALID_ARG, "order must be 0 (row per lane) or 1 (row-major)");
  if (iters < 1 || iters > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "iters must lie in [1, 2^20]");
  if (n_wg < 1 || n_wg > 65536) return fail(MOE_ERR_INVALID_ARG, "n_wg must lie in [1, 65536]");
  uint32_t seg_log = 0;
  while ((64u << seg_log) < (uint32_t)row_bytes) ++seg_log;
  const uint32_t tiles = (uint32_t)(bytes / (size_t)row_bytes / 16) << seg_log;
  const hipError_t e = moe::launch_probe_gather(src, (uint32_t)row_bytes, seg_log, tiles, iters, order, sink, n_wg, stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "probe launch");
}

moe_status moe_read_counts(const moe_config* cfg, const void* workspace, size_t ws_bytes, int32_t* host_counts,
                           hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_ws(*cfg, workspace, ws_bytes));
  if (!host_counts) return fail(MOE_ERR_INVALID_ARG, "host_counts is NULL");
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (st != hipStreamCaptureStatusNone)
    return fail(MOE_ERR_CAPTURE_VIOLATION, "moe_read_counts synchronises and cannot run on a capturing stream");
  const Layout L = layout(*cfg);
  e = hipMemcpyAsync(host_counts, static_cast<const char*>(workspace) + L.counts, (size_t)cfg->n_experts * 4,
                     hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipStreamSynchronize(stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "hipStreamSynchronize");
}

}  // extern "C"

static moe_status capture_impl(const moe_config* cfg, const moe_weights* w, const int32_t* buckets,
                               int32_t n_buckets, const void* x_static, const moe_prenorm* pn,
                               void* out_static, void* workspace, size_t ws_bytes, hipStream_t stream,
                               moe_graph** graph) {
  if (!graph) return fail(MOE_ERR_INVALID_ARG, "graph out-pointer is NULL");
  *graph = nullptr;
  MOE_TRY(check_forward_args(cfg, w, x_static, 1, out_static, workspace, ws_bytes));
  if (!buckets || n_buckets < 1) return fail(MOE_ERR_INVALID_ARG, "empty bucket list");
  for (int i = 0; i < n_buckets; ++i) {
    if (buckets[i] < 1 || buckets[i] > cfg->t_max || (i && buckets[i] <= buckets[i - 1]))
      return fail(MOE_ERR_INVALID_ARG, "buckets must be strictly ascending within [1, t_max]");
  }
  moe::PrenormArgs pa{};
  if (pn) MOE_TRY(check_prenorm(*cfg, pn, buckets[n_buckets - 1], &pa));
  if (!stream) return fail(MOE_ERR_NOT_CAPTURABLE, "capture needs a created stream, not the NULL stream");
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (st != hipStreamCaptureStatusNone) return fail(MOE_ERR_NOT_CAPTURABLE, "stream is already capturing");

  moe_graph* g = new moe_graph();
  g->cfg = *cfg;
  g->live = at<int32_t>(workspace, layout(*cfg).live);
  for (int i = 0; i < n_buckets; ++i) {
    const int32_t b = buckets[i];
    e = hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      graph_release(g);
      return fail(MOE_ERR_NOT_CAPTURABLE, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
    }
    // the router's first kernel writes the live row count (the bucket size
    // until a replay with fewer rows sets the node's argument)
    moe::RouteNode rn{};
    const moe_status rs = enqueue_forward(*cfg, *w, x_static, b, out_static, workspace, stream, nullptr,
                                          g->live, pn ? &pa : nullptr, &rn);
    const std::string launch_msg = rs == MOE_OK ? std::string() : g_last_error;
    hipGraph_t gr = nullptr;
    e = hipStreamEndCapture(stream, &gr);
    if (rs != MOE_OK || e != hipSuccess || !gr) {
      if (gr) (void)hipGraphDestroy(gr);
      graph_release(g);
      return fail(MOE_ERR_NOT_CAPTURABLE,
                  "capture of bucket " + std::to_string(b) + " failed: " +
                      (rs != MOE_OK ? launch_msg : std::string(hipGetErrorString(e))));
    }
    // the router node: the graph's only root (capture on one stream makes a
    // chain)
    size_t nroot = 0;
    hipGraphNode_t root = nullptr;
    hipGraphNodeType rtype = hipGraphNodeTypeEmpty;
    e = hipGraphGetRootNodes(gr, nullptr, &nroot);
    if (e == hipSuccess && nroot == 1) e = hipGraphGetRootNodes(gr, &root, &nroot);
    if (e == hipSuccess && root) e = hipGraphNodeGetType(root, &rtype);
    if (e != hipSuccess || nroot != 1 || !root || rtype != hipGraphNodeTypeKernel) {
      (void)hipGraphDestroy(gr);
      graph_release(g);
      return fail(MOE_ERR_NOT_CAPTURABLE, "captured graph does not start with the router kernel");
    }
    hipGraphExec_t ge = nullptr;
    e = hipGraphInstantiate(&ge, gr, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      (void)hipGraphDestroy(gr);
      graph_release(g);
      return fail(MOE_ERR_NOT_CAPTURABLE, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    }
    g->buckets.push_back(b);
    g->graphs.push_back(gr);
    g->execs.push_back(ge);
    g->live_nodes.push_back(root);
    g->live_launch.push_back(rn);
    g->live_vals.push_back(b);
  }
  *graph = g;
  return MOE_OK;
}

extern "C" {

moe_status moe_graph_capture(const moe_config* cfg, const moe_weights* w, const int32_t* buckets, int32_t n_buckets,
                             const void* x_static, void* out_static, void* workspace, size_t ws_bytes,
                             hipStream_t stream, moe_graph** graph) {
  return capture_impl(cfg, w, buckets, n_buckets, x_static, nullptr, out_static, workspace, ws_bytes, stream,
                      graph);
}

moe_status moe_graph_capture_prenorm(const moe_config* cfg, const moe_weights* w, const int32_t* buckets,
                                     int32_t n_buckets, const moe_prenorm* pn_static, void* out_static,
                                     void* workspace, size_t ws_bytes, hipStream_t stream, moe_graph** graph) {
  if (graph) *graph = nullptr;
  if (!pn_static) return fail(MOE_ERR_INVALID_ARG, "prenorm is NULL");
  return capture_impl(cfg, w, buckets, n_buckets, pn_static->x_out, pn_static, out_static, workspace, ws_bytes,
                      stream, graph);
}

int32_t moe_graph_bucket_for(const moe_graph* g, int32_t T) {
  if (!g || T < 1) return -1;
  for (int32_t b : g->buckets)
    if (b >= T) return b;
  return -1;
}

moe_status moe_graph_replay(moe_graph* g, int32_t T, hipStream_t stream) {
  if (!g) return fail(MOE_ERR_INVALID_ARG, "graph is NULL");
  for (size_t i = 0; i < g->buckets.size(); ++i) {
    if (g->buckets[i] >= T && T >= 1) {
      // the captured kernels read the live row count the graph's first node
      // writes; its argument changes only when T does
      if (T != g->live_vals[i]) {
        const hipError_t e = moe::set_route_live(g->execs[i], g->live_nodes[i], g->live_launch[i], T);
        if (e != hipSuccess) return hip_fail(e, "hipGraphExecKernelNodeSetParams");
        g->live_vals[i] = T;
      }
      const hipError_t e = hipGraphLaunch(g->execs[i], stream);
      return e == hipSuccess ? MOE_OK : hip_fail(e, "hipGraphLaunch");
    }
  }
  return fail(MOE_ERR_INVALID_ARG, "T=" + std::to_string(T) + " exceeds the largest captured bucket");
}

void moe_graph_destroy(moe_graph* g) {
  if (g) graph_release(g);
}

}  // extern "C"
