"""Plain, slow fp64 CPU oracle of the sparse-MoE block forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The HIP library never
links, calls or falls back to it, and it shares no code with the HIP path.

What it computes (Qwen3-MoE sparse block, decode or prefill, one layer):

  1. router logits   l[t,e] = sum_h X[t,h] * Wr[e,h], rounded to fp32, then
                     plus an optional fp32 per-expert bias (added in fp32).
                     The workload fixes "softmax over fp32 logits"; the fp32
                     value is the correctly rounded fp32 of the dot product of
                     the bf16 operands (their products are exact).
  2. top-k           the k experts with the largest fp32 logit; equal logits
                     go to the lower expert index; ids stored best first.
  3. weights         softmax over all E logits (fp64), then renormalised over
                     the k chosen: w_j = p[id_j] / sum_j' p[id_j'] (or, in
                     the variant without renormalisation, w_j = p[id_j]).
  4. bucketing       per-expert counts (histogram), exclusive-scan offsets
                     (E+1 entries), and the stable permutation of the flat
                     token-expert slots s = t*k + j grouped by expert: the
                     bincount/scatter_add + cumsum + argsort steps of the
                     grouped_mm MoE path [unsloth commit 80aaf1121b page
                     (Qwen3-MoE decode CUDA-graph capture), third and last
                     paragraphs].
  5. experts         SwiGLU MLP per chosen expert: g = Wg x, u = Wu x,
                     h = silu(g) * u with silu(z) = z / (1 + exp(-z)),
                     y = Wd h  (the grouped GEMMs of the same path).
  0. (optional)      the pre-block step: r = bf16(residual + delta),
                     x = bf16(r / sqrt(mean(r^2) + eps) * gamma), the
                     block's input [a1bc5cbd page, first paragraph].
                     (optional LoRA: each of the two stacked matrices W gets
                     + scale * B (A input), fp32 adapters, rank 16 on the
                     4f2bfe7f69 page.)
  (backward)        for fixed routing, the chain rule back to x and to the
                     routing weights (backward_per_token).
  6. combine         out[t] = sum_j w[t,j] * y[t,j], j ascending (the
                     index_add_ step of the same path), returned as a plain
                     tensor [unsloth commit 4f2bfe7f69 page (first MoE decode
                     bench), second paragraph].

4-bit expert weights: W[n, k] = fp32(codebook[code] * absmax[n, k // 64]) with
codes packed two per byte (even element in the low nibble).

Everything is numpy fp64 (bf16 and fp32 inputs convert exactly).  The
per-token loop `forward_per_token` is the definition; `forward_batched` is the
same arithmetic grouped by expert (one matmul per expert) for large T, and is
checked against the per-token loop by the tests.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

NF4_BLOCK = 64


# --------------------------------------------------------------------------
# storage formats -> fp64
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit pattern, one rounding to nearest, ties to even
    (zeros and finite values in the bf16 normal range).  Not via fp32: that
    would round twice."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    u = v.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint64)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    # bf16 keeps 7 of the 52 fraction bits: drop 45, round to nearest even
    keep = mag >> np.uint64(45)
    rest = mag & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rest > half) | ((rest == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    keep = keep + up.astype(np.uint64)
    # rebias the exponent from 1023 to 127 (bits above the 7 fraction bits)
    exp = (keep >> np.uint64(7)).astype(np.int64) - 1023 + 127
    frac = (keep & np.uint64(0x7F)).astype(np.int64)
    zero = mag == np.uint64(0)
    assert np.all(zero | ((exp > 0) & (exp < 255))), "value outside the bf16 normal range"
    bits = (sign.astype(np.int64) << 15) | np.where(zero, 0, (exp << 7) | frac)
    return bits.astype(np.uint16)


def nf4_unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> codes uint8 [..., K]; element 2i is the low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & np.uint8(0x0F)
    hi = packed >> np.uint8(4)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def nf4_dequant(packed: np.ndarray, absmax: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """4-bit blockwise weights -> fp32 values W = fp32(codebook[code] * absmax),
    one absmax per 64 consecutive weights along the last axis."""
    codes = nf4_unpack(packed)
    cb = np.asarray(codebook, dtype=np.float32)
    vals = cb[codes]                                             # fp32
    sc = np.repeat(np.asarray(absmax, dtype=np.float32), NF4_BLOCK, axis=-1)
    return (vals * sc).astype(np.float32)                        # fp32 product


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------
def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray,
                  bias: Optional[np.ndarray] = None, exact: bool = False) -> np.ndarray:
    """fp32 router logits [T][E].

    The dot product of bf16 operands is formed in fp64 (numpy matmul; with
    exact=True each entry is math.fsum over the exact products, the correctly
    rounded fp64 sum) and then rounded to fp32.  The bias, if any, is added in
    fp32 arithmetic.
    """
    x = bf16_bits_to_f64(x_bits)
    wr = bf16_bits_to_f64(wr_bits)
    if exact:
        T, E = x.shape[0], wr.shape[0]
        l64 = np.empty((T, E), dtype=np.float64)
        for t in range(T):
            for e in range(E):
                l64[t, e] = math.fsum((x[t] * wr[e]).tolist())
    else:
        l64 = x @ wr.T
    l32 = l64.astype(np.float32)
    if bias is not None:
        l32 = (l32 + np.asarray(bias, dtype=np.float32)).astype(np.float32)
    return l32


def topk_lowest_index(logits32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, best first; equal logits are
    ordered by ascending expert index.  int32 [T][k]."""
    logits32 = np.asarray(logits32)
    T, E = logits32.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    # lexsort: last key is primary -> sort by (-logit, index)
    order = np.lexsort((idx, -logits32.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def softmax_weights(logits32: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all E logits (fp64, max-subtracted) taken at the chosen
    ids, not renormalised: w_j = p[id_j], so sum_j w_j <= 1.  fp64 [T][k]."""
    l = np.asarray(logits32, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    p = p / p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), axis=1)


def renormalised_weights(logits32: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all E logits, then renormalised over the chosen k:
    w_j = p[id_j] / sum_j' p[id_j'].  fp64 [T][k]."""
    sel = softmax_weights(logits32, ids)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x_bits, wr_bits, k: int, bias=None, exact: bool = False, renorm: bool = True):
    """(ids int32 [T][k], weights fp64 [T][k], logits fp32 [T][E]).

    renorm=False keeps the full-softmax probabilities of the chosen experts
    (the router variant without top-k renormalisation)."""
    l32 = router_logits(x_bits, wr_bits, bias, exact=exact)
    ids = topk_lowest_index(l32, k)
    w = renormalised_weights(l32, ids) if renorm else softmax_weights(l32, ids)
    return ids, w, l32


# --------------------------------------------------------------------------
# pre-block step: residual add, RMSNorm (the layernorm + residual + router
# fusion of the a1bc5cbd page, first paragraph)
# --------------------------------------------------------------------------
def residual_rmsnorm(residual_bits, delta_bits, gamma_bits, eps):
    """r = bf16(residual + delta) (the exact sum rounded once to nearest
    even; delta None: r = residual); x = r / sqrt(mean_h(r^2) + eps) * gamma
    in fp64.  Returns (r bits uint16 [T][H], x fp64 [T][H]); the block's
    input is x rounded once to bf16."""
    r = bf16_bits_to_f64(residual_bits)
    if delta_bits is not None:
        r = r + bf16_bits_to_f64(delta_bits)   # exact: two bf16 values
    r_bits = f64_to_bf16_rne(r)
    r = bf16_bits_to_f64(r_bits)
    ms = np.mean(r * r, axis=1, keepdims=True)
    x = r / np.sqrt(ms + float(eps)) * bf16_bits_to_f64(gamma_bits)[None, :]
    return r_bits, x


# --------------------------------------------------------------------------
# bucketing: histogram, exclusive scan, stable permutation
# --------------------------------------------------------------------------
def histogram(ids_flat: np.ndarray, E: int) -> np.ndarray:
    counts = np.zeros(E, dtype=np.int64)
    for e in np.asarray(ids_flat).tolist():
        counts[e] += 1
    return counts.astype(np.int32)


def exclusive_scan(counts: np.ndarray) -> np.ndarray:
    """offsets[0] = 0, offsets[e+1] = offsets[e] + counts[e]  (E+1 entries)."""
    out = np.zeros(len(counts) + 1, dtype=np.int64)
    run = 0
    for e, c in enumerate(np.asarray(counts).tolist()):
        out[e] = run
        run += c
    out[len(counts)] = run
    return out.astype(np.int32)


def stable_permute(ids_flat: np.ndarray, offsets: np.ndarray):
    """Counting sort of flat slots by expert, keeping slot order inside each
    expert.  perm[p] = slot s placed at position p; pos[s] = p (inverse)."""
    ids_flat = np.asarray(ids_flat).tolist()
    cursor = np.asarray(offsets[:-1], dtype=np.int64).copy()
    n = len(ids_flat)
    perm = np.empty(n, dtype=np.int32)
    pos = np.empty(n, dtype=np.int32)
    for s, e in enumerate(ids_flat):
        p = int(cursor[e])
        cursor[e] += 1
        perm[p] = s
        pos[s] = p
    return perm, pos


def permute(ids: np.ndarray, E: int):
    """(counts [E], offsets [E+1], perm [T*k], pos [T*k]) from ids [T][k]."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = histogram(flat, E)
    offsets = exclusive_scan(counts)
    perm, pos = stable_permute(flat, offsets)
    return counts, offsets, perm, pos


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


class ExpertWeights:
    """fp64 views of the expert weights, converted per expert on first use."""

    def __init__(self, inp):
        self.inp = inp
        self.I = inp.I
        self._cache = {}
        self._pending = {}

    def get(self, e: int):
        if e not in self._cache:
            if self.inp.wfmt not in ("bf16", "nf4"):
                raise ValueError(self.inp.wfmt)
            self._convert(e)
            self._cache[e] = self._pending.pop(e)
        return self._cache[e]

    def preload(self, experts):
        """Convert several experts at once on a thread pool (numpy casts drop
        the GIL); the values are the same as converting one by one."""
        todo = [int(e) for e in experts if int(e) not in self._cache]
        n = min(len(todo), max(1, len(os.sched_getaffinity(0))))
        if n <= 1:
            for e in todo:
                self.get(e)
            return
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(self._convert, todo))
        # dict writes happen here, on one thread
        for e, val in self._pending.items():
            self._cache[e] = val
        self._pending.clear()

    def _convert(self, e: int):
        inp = self.inp
        if inp.wfmt == "bf16":
            gu = bf16_bits_to_f64(inp.w_gate_up[e])
            wd = bf16_bits_to_f64(inp.w_down[e])
        else:
            gu = nf4_dequant(inp.q_gate_up[e], inp.s_gate_up[e], inp.codebook).astype(np.float64)
            wd = nf4_dequant(inp.q_down[e], inp.s_down[e], inp.codebook).astype(np.float64)
        self._pending[e] = (gu[: self.I], gu[self.I:], wd)


class LoRA:
    """Low-rank adapters on every expert's stacked gate/up and down matrices
    (the rank-16 LoRA of the 4f2bfe7f69 page's workload, fp32 adapters):
    W_gu <- W_gu + scale * B_gu A_gu and W_d <- W_d + scale * B_d A_d, applied
    as x W^T + scale * (x A^T) B^T.  Arrays (fp32, exact in fp64):
    a_gate_up [E][r][H], b_gate_up [E][2I][r] (gate rows, then up rows),
    a_down [E][r][I], b_down [E][H][r]."""

    def __init__(self, a_gate_up, b_gate_up, a_down, b_down, scale):
        self.a_gate_up, self.b_gate_up = a_gate_up, b_gate_up
        self.a_down, self.b_down = a_down, b_down
        self.scale = float(scale)

    def get(self, e: int, I: int):
        f = lambda a: np.asarray(a[e], dtype=np.float64)  # noqa: E731
        bgu = f(self.b_gate_up)
        return f(self.a_gate_up), bgu[:I], bgu[I:], f(self.a_down), f(self.b_down)


def expert_mlp(x64: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, lora=None) -> np.ndarray:
    """SwiGLU expert on one token (vector) or a batch (rows): y = Wd (silu(Wg x) * Wu x).
    lora = (A_gu, B_g, B_u, A_d, B_d, scale): each projection gets
    + scale * B (A input) before the nonlinearity / output."""
    g = x64 @ wg.T
    u = x64 @ wu.T
    if lora is not None:
        a_gu, b_g, b_u, a_d, b_d, s = lora
        z = x64 @ a_gu.T
        g = g + s * (z @ b_g.T)
        u = u + s * (z @ b_u.T)
    h = silu(g) * u
    y = h @ wd.T
    if lora is not None:
        y = y + s * ((h @ a_d.T) @ b_d.T)
    return y


def _lora_of(lora, e, I):
    return None if lora is None else (*lora.get(e, I), lora.scale)


# --------------------------------------------------------------------------
# full block
# --------------------------------------------------------------------------
def forward_per_token(inp, weights: Optional[ExpertWeights] = None, exact_router: bool = False,
                      routing=None, renorm: bool = True, lora: Optional[LoRA] = None):
    """The definition: loop over tokens, then over the k chosen experts.

    Returns (out fp64 [T][H], routing dict)."""
    if routing is None:
        ids, w, l32 = route(inp.x, inp.w_router, inp.k, inp.bias, exact=exact_router, renorm=renorm)
    else:
        ids, w, l32 = routing["ids"], routing["w"], routing["logits"]
    W = weights or ExpertWeights(inp)
    x64 = bf16_bits_to_f64(inp.x)
    out = np.zeros((inp.T, inp.H), dtype=np.float64)
    for t in range(inp.T):
        acc = np.zeros(inp.H, dtype=np.float64)
        for j in range(inp.k):
            e = int(ids[t, j])
            wg, wu, wd = W.get(e)
            acc = acc + w[t, j] * expert_mlp(x64[t], wg, wu, wd, _lora_of(lora, e, inp.I))
        out[t] = acc
    return out, dict(ids=ids, w=w, logits=l32)


def forward_batched(inp, weights: Optional[ExpertWeights] = None, routing=None, renorm: bool = True,
                    lora: Optional[LoRA] = None):
    """Same arithmetic grouped by expert: for each expert, one matmul over the
    tokens routed to it, then the per-token weighted sum in ascending j.

    Returns (out fp64 [T][H], routing dict incl. counts/offsets/perm/pos)."""
    if routing is None:
        ids, w, l32 = route(inp.x, inp.w_router, inp.k, inp.bias, renorm=renorm)
    else:
        ids, w, l32 = routing["ids"], routing["w"], routing["logits"]
    counts, offsets, perm, pos = permute(ids, inp.E)
    W = weights or ExpertWeights(inp)
    W.preload(np.nonzero(counts)[0])
    x64 = bf16_bits_to_f64(inp.x)
    T, k = ids.shape
    y_slot = np.zeros((T * k, inp.H), dtype=np.float64)
    for e in range(inp.E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        slots = perm[a:b].astype(np.int64)
        wg, wu, wd = W.get(e)
        y_slot[slots] = expert_mlp(x64[slots // k], wg, wu, wd, _lora_of(lora, e, inp.I))
    out = np.zeros((T, inp.H), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y_slot[np.arange(T) * k + j]
    return out, dict(ids=ids, w=w, logits=l32, counts=counts, offsets=offsets, perm=perm, pos=pos)


# --------------------------------------------------------------------------
# backward of the block (frozen weights): gradients of a loss L with respect
# to the input x and to the routing weights, given dL/dout
# --------------------------------------------------------------------------
def silu_grad(z):
    """d silu / dz = s(z) (1 + z (1 - s(z))), s the logistic function."""
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def backward_per_token(inp, d_out, weights: Optional[ExpertWeights] = None, routing=None,
                       lora: Optional["LoRA"] = None, weight_grads: bool = False, wgrad_experts=None,
                       renorm: bool = True):
    """The chain rule through the block, token by token, for fixed routing
    (the top-k choice is piecewise constant in x):
      d_w[t,j] = <d_out[t], y[t,j]>
      d_l[t,j] = w_j (d_w_j - sum_i w_i d_w_i)   (softmax over the k chosen logits)
      d_y      = w[t,j] d_out[t];  d_h = d_y Wd;  d_g = d_h u silu'(g);  d_u = d_h silu(g)
      d_x[t]   = sum_j (d_g Wg + d_u Wu) + sum_j d_l[t,j] Wr[id_j]
    With LoRA adapters (W -> W + s B A on the stacked gate/up and the down
    matrix), the same chain rule through W + s B A, plus the adapter
    gradients summed over every routed (token, expert) pair:
      d_B_d += s d_y (A_d h)^T,   d_A_d += s (B_d^T d_y) h^T
      d_B_gu += s [d_g; d_u] (A_gu x)^T,   d_A_gu += s (B_gu^T [d_g; d_u]) x^T
    renorm=False (the full softmax taken at the chosen experts, not
    renormalised): w_j = p[id_j] with p the softmax over all E logits, so
      d_l[t,e] = [e chosen] w_e d_w_e - p_e sum_j w_j d_w_j   for every e,
    and the router share of d_x runs over all E experts (d_logits [T][E]).
    With weight_grads, the gradients of the expert weights themselves (the
    same for W alone or W + s B A, whose derivative in W is the identity):
      d_W_gu[e] += [d_g; d_u] x^T,   d_W_d[e] += d_y h^T
    Returns dict(d_x fp64 [T][H], d_w fp64 [T][k], d_logits fp64 [T][k],
    routing, with lora: d_a_gate_up, d_b_gate_up, d_a_down, d_b_down, with
    weight_grads: d_w_gate_up [E][2I][H], d_w_down [E][H][I]; with
    wgrad_experts, a list of experts, only those experts' slices, as dicts
    expert -> array, so that large shapes can be checked expert by expert)."""
    if routing is None:
        ids, w, l32 = route(inp.x, inp.w_router, inp.k, inp.bias, renorm=renorm)
        routing = dict(ids=ids, w=w, logits=l32)
    ids, w = routing["ids"], routing["w"]
    W = weights or ExpertWeights(inp)
    x64 = bf16_bits_to_f64(inp.x)
    wr = bf16_bits_to_f64(inp.w_router)
    d_out = np.asarray(d_out, dtype=np.float64)
    T, k = ids.shape
    d_x = np.zeros((T, inp.H))
    d_w = np.zeros((T, k))
    grads = None
    if lora is not None:
        grads = {n: np.zeros(np.shape(getattr(lora, n)), dtype=np.float64)
                 for n in ("a_gate_up", "b_gate_up", "a_down", "b_down")}
    wgrads = None
    if weight_grads:
        if wgrad_experts is None:
            wgrads = {"w_gate_up": np.zeros((inp.E, 2 * inp.I, inp.H)), "w_down": np.zeros((inp.E, inp.H, inp.I))}
        else:
            wgrads = {"w_gate_up": {int(e): np.zeros((2 * inp.I, inp.H)) for e in wgrad_experts},
                      "w_down": {int(e): np.zeros((inp.H, inp.I)) for e in wgrad_experts}}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            wg, wu, wd = W.get(e)
            if lora is not None:
                a_gu, b_g, b_u, a_d, b_d = lora.get(e, inp.I)
                s = lora.scale
                wg = wg + s * (b_g @ a_gu)
                wu = wu + s * (b_u @ a_gu)
                wd = wd + s * (b_d @ a_d)
            g = wg @ x64[t]
            u = wu @ x64[t]
            h = silu(g) * u
            y = wd @ h
            d_w[t, j] = d_out[t] @ y
            d_y = w[t, j] * d_out[t]
            d_h = d_y @ wd
            d_g = d_h * u * silu_grad(g)
            d_u = d_h * silu(g)
            d_x[t] += d_g @ wg + d_u @ wu
            if wgrads is not None and (wgrad_experts is None or e in wgrads["w_down"]):
                wgrads["w_gate_up"][e][:inp.I] += np.outer(d_g, x64[t])
                wgrads["w_gate_up"][e][inp.I:] += np.outer(d_u, x64[t])
                wgrads["w_down"][e] += np.outer(d_y, h)
            if lora is not None:
                d_gu = np.concatenate([d_g, d_u])
                b_gu = np.concatenate([b_g, b_u])
                grads["b_down"][e] += s * np.outer(d_y, a_d @ h)
                grads["a_down"][e] += s * np.outer(b_d.T @ d_y, h)
                grads["b_gate_up"][e] += s * np.outer(d_gu, a_gu @ x64[t])
                grads["a_gate_up"][e] += s * np.outer(b_gu.T @ d_gu, x64[t])
    if renorm:
        d_l = w * (d_w - np.sum(w * d_w, axis=1, keepdims=True))
        for t in range(T):
            for j in range(k):
                d_x[t] += d_l[t, j] * wr[int(ids[t, j])]
    else:
        l = np.asarray(routing["logits"], dtype=np.float64)
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        d_l = -p * np.sum(w * d_w, axis=1, keepdims=True)
        for t in range(T):
            for j in range(k):
                d_l[t, int(ids[t, j])] += w[t, j] * d_w[t, j]
        d_x += d_l @ wr
    out = dict(d_x=d_x, d_w=d_w, d_logits=d_l, routing=routing)
    if grads is not None:
        out.update({"d_" + n: v for n, v in grads.items()})
    if wgrads is not None:
        out.update({"d_" + n: v for n, v in wgrads.items()})
    return out


def rms(a: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a)))
