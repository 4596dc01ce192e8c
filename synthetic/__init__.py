"""Seeded synthetic inputs for the sparse-MoE block (Qwen3-30B-A3B layer shape).

This module only *makes inputs*: it draws random numbers, rounds them to the
storage formats the block consumes (bf16 bit patterns, packed 4-bit codes with
fp32 block scales), and returns them.  It holds none of the block's arithmetic
(no router, no top-k, no expert MLP, no dequantisation): both the fp64 CPU
oracle and the HIP path read these arrays and compute on their own.

Workloads (the Qwen3-30B-A3B MoE layer is H=2048, E=128, k=8, I=768; the pages
it stands in for decode Qwen3-30B-A3B at batch sizes 8-64 and use 4-bit and
bf16 weights; their model weights, prompts and dataset are not available, so
everything here is synthetic):

  tiny   T=8,    H=256,  E=16,  k=2, I=128, bf16 weights
  q8     T=8,    Qwen layer, bf16
  q64    T=64,   Qwen layer, bf16 (plus a batch sweep T in 1..64)
  q48q   T=48,   Qwen layer, 4-bit blockwise weights (64 per fp32 absmax)
  q4096  T=4096, Qwen layer, bf16, router bias -1.1*ln(e+1) (Zipf-like skew)

Value distributions: weights ~ N(0, 0.02) sampled in fp32, activations
~ N(0, 1) (unit-RMS tokens, as after an RMSNorm), both rounded to bf16 with
round-to-nearest-even.  The bf16 Qwen-shaped layer (router + experts) is drawn
once from seed 2002 and shared by q8, q64, the sweep and q4096; each workload
draws its own activations (seed 1000 + workload number, sweep sub-seed T).
"""
from __future__ import annotations

import os
import statistics
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

QWEN = dict(H=2048, E=128, k=8, I=768)
SWEEP_T = (1, 2, 4, 8, 16, 32, 48, 64)
NF4_BLOCK = 64

_LAYER_SEED = 2002
_LAYER_SEED_TINY = 2001
_LAYER_SEED_Q4 = 2004
_X_SEED = {"tiny": 1001, "q8": 1002, "q64": 1003, "q48q": 1004, "q4096": 1005}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs here are finite normal samples, so no NaN handling is needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
        flat_out[s:s + step] = r.astype(np.uint16)
    return out


def nf4_codebook() -> np.ndarray:
    """16-entry normal-quantile codebook in [-1, 1] (the NormalFloat idea).

    Eight positive levels are N(0,1) quantiles at evenly spaced probabilities
    from 1/2 (excluded) up to delta = 1 - 1/32, scaled so the largest is +1;
    seven negative levels are built the same way and scaled so the smallest is
    -1; plus an exact zero.  Returned ascending as fp32 (each level the
    nearest fp32 value of its quantile), so code 7 is 0.0.
    """
    nd = statistics.NormalDist()
    delta = 1.0 - 1.0 / 32.0
    pos = [nd.inv_cdf(p) for p in np.linspace(0.5, delta, 9)[1:]]
    neg = [nd.inv_cdf(p) for p in np.linspace(0.5, delta, 8)[1:]]
    pos = np.asarray(pos) / max(pos)
    neg = -np.asarray(neg) / max(neg)
    cb = np.sort(np.concatenate([neg, [0.0], pos])).astype(np.float32)
    return cb


def quantize_nf4(w: np.ndarray, codebook: np.ndarray):
    """Blockwise 4-bit quantiser used only to *make* 4-bit inputs.

    w: fp32 [..., K] with K % 64 == 0.  Each run of 64 consecutive weights along
    the last axis gets absmax = max|w| (fp32); each weight gets the code of the
    codebook entry nearest to w/absmax (ties -> lower code); an all-zero block
    gets the 0.0 code.  Codes are packed two per byte: element 2i in the low
    nibble, element 2i+1 in the high nibble.

    Returns (packed uint8 [..., K/2], absmax fp32 [..., K/64]).
    """
    w = np.asarray(w, dtype=np.float32)
    K = w.shape[-1]
    assert K % NF4_BLOCK == 0
    lead = w.shape[:-1]
    blocks = w.reshape(-1, NF4_BLOCK)
    absmax = np.abs(blocks).max(axis=1).astype(np.float32)
    safe = np.where(absmax > 0, absmax, np.float32(1.0))
    r = blocks / safe[:, None]
    mids = ((codebook[1:] + codebook[:-1]) * np.float32(0.5)).astype(np.float32)
    # searchsorted(side='left') puts a value equal to a midpoint on the lower code
    codes = np.searchsorted(mids, r, side="left").astype(np.uint8)
    zero_code = int(np.argmin(np.abs(codebook)))
    codes[absmax == 0, :] = zero_code
    codes = codes.reshape(*lead, K)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, absmax.reshape(*lead, K // NF4_BLOCK)


@dataclass
class MoEInputs:
    """One workload: shapes plus host arrays in the block's storage formats.

    x          uint16 [T][H]        bf16 bits, activations
    w_router   uint16 [E][H]        bf16 bits
    bias       float32 [E] or None  added to the fp32 router logits
    w_gate_up  uint16 [E][2I][H]    bf16 bits; rows [0,I) gate, [I,2I) up
    w_down     uint16 [E][H][I]     bf16 bits
    4-bit variant (wfmt == "nf4"):
    q_gate_up  uint8 [E][2I][H/2],  s_gate_up float32 [E][2I][H/64]
    q_down     uint8 [E][H][I/2],   s_down    float32 [E][H][I/64]
    codebook   float32 [16]
    """
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    wfmt: str
    x: np.ndarray
    w_router: np.ndarray
    bias: Optional[np.ndarray] = None
    w_gate_up: Optional[np.ndarray] = None
    w_down: Optional[np.ndarray] = None
    q_gate_up: Optional[np.ndarray] = None
    s_gate_up: Optional[np.ndarray] = None
    q_down: Optional[np.ndarray] = None
    s_down: Optional[np.ndarray] = None
    codebook: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    def with_x(self, x: np.ndarray, name: Optional[str] = None) -> "MoEInputs":
        d = dict(self.__dict__)
        d["x"] = x
        d["T"] = int(x.shape[0])
        d["name"] = name or self.name
        d["meta"] = dict(self.meta)
        return MoEInputs(**d)


def _pool_map(fn, items):
    """Run fn over items on a thread pool (numpy's generators and casts drop the
    GIL on large arrays).  Results do not depend on the thread count: every
    chunk has its own seed."""
    items = list(items)
    n = min(len(items), max(1, len(os.sched_getaffinity(0))))
    if n <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=n) as ex:
        return list(ex.map(fn, items))


def _child_rng(seed: int, tensor: int, part: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, part])))


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def _per_expert_bf16(seed: int, tensor: int, shape, std: float) -> np.ndarray:
    """[E, ...] tensor whose expert slice e is drawn from child seed (seed, tensor, e)."""
    out = np.empty(shape, dtype=np.uint16)

    def fill(e):
        out[e] = _normal_bf16(_child_rng(seed, tensor, e), shape[1:], std)

    _pool_map(fill, range(shape[0]))
    return out


def _per_expert_nf4(seed: int, tensor: int, shape, std: float, cb: np.ndarray):
    E, N, K = shape
    q = np.empty((E, N, K // 2), dtype=np.uint8)
    s = np.empty((E, N, K // NF4_BLOCK), dtype=np.float32)

    def fill(e):
        w = _child_rng(seed, tensor, e).standard_normal((N, K), dtype=np.float32) * np.float32(std)
        q[e], s[e] = quantize_nf4(w, cb)

    _pool_map(fill, range(E))
    return q, s


_LAYER_CACHE: dict = {}


def layer_bf16(H: int, E: int, I: int, seed: int):
    """Router + expert weights of one bf16 layer: (w_router, w_gate_up, w_down).
    Tensor ids in the child seeds: 0 router, 1 gate/up, 2 down."""
    key = ("bf16", H, E, I, seed)
    if key not in _LAYER_CACHE:
        wr = _normal_bf16(_child_rng(seed, 0, 0), (E, H), 0.02)
        wgu = _per_expert_bf16(seed, 1, (E, 2 * I, H), 0.02)
        wd = _per_expert_bf16(seed, 2, (E, H, I), 0.02)
        _LAYER_CACHE[key] = (wr, wgu, wd)
    return _LAYER_CACHE[key]


def layer_nf4(H: int, E: int, I: int, seed: int):
    """Router (bf16) + 4-bit expert weights of one layer (same child-seed scheme)."""
    key = ("nf4", H, E, I, seed)
    if key not in _LAYER_CACHE:
        cb = nf4_codebook()
        wr = _normal_bf16(_child_rng(seed, 0, 0), (E, H), 0.02)
        qgu, sgu = _per_expert_nf4(seed, 1, (E, 2 * I, H), 0.02, cb)
        qd, sd = _per_expert_nf4(seed, 2, (E, H, I), 0.02, cb)
        _LAYER_CACHE[key] = (wr, qgu, sgu, qd, sd, cb)
    return _LAYER_CACHE[key]


def activations(T: int, H: int, seed) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal_bf16(rng, (T, H), 1.0)


def skew_bias(E: int) -> np.ndarray:
    """Per-expert router bias -1.1*ln(rank+1) with rank = expert index."""
    return (-1.1 * np.log(np.arange(E, dtype=np.float64) + 1.0)).astype(np.float32)


def make(name: str, T: Optional[int] = None) -> MoEInputs:
    """Build a named workload.  `T` overrides the token count (same weights;
    activations are re-drawn from the workload seed with sub-seed T)."""
    if name == "tiny":
        H, E, k, I = 256, 16, 2, 128
        Tn = 8 if T is None else T
        wr, wgu, wd = layer_bf16(H, E, I, _LAYER_SEED_TINY)
        xseed = _X_SEED[name] if T is None else [_X_SEED[name], T]
        return MoEInputs(name, Tn, H, E, k, I, "bf16", activations(Tn, H, xseed), wr,
                         None, wgu, wd)
    H, E, k, I = QWEN["H"], QWEN["E"], QWEN["k"], QWEN["I"]
    default_T = {"q8": 8, "q64": 64, "q48q": 48, "q4096": 4096}[name]
    Tn = default_T if T is None else T
    xseed = _X_SEED[name] if T is None else [_X_SEED[name], T]
    x = activations(Tn, H, xseed)
    if name == "q48q":
        wr, qgu, sgu, qd, sd, cb = layer_nf4(H, E, I, _LAYER_SEED_Q4)
        return MoEInputs(name, Tn, H, E, k, I, "nf4", x, wr, None,
                         q_gate_up=qgu, s_gate_up=sgu, q_down=qd, s_down=sd, codebook=cb)
    wr, wgu, wd = layer_bf16(H, E, I, _LAYER_SEED)
    bias = skew_bias(E) if name == "q4096" else None
    return MoEInputs(name, Tn, H, E, k, I, "bf16", x, wr, bias, wgu, wd)


def router_inputs(name: str, T: Optional[int] = None):
    """(x, w_router, bias, k) of a named workload without drawing its expert
    weights: the same arrays make(name, T) returns for these fields."""
    if name == "tiny":
        H, E, k = 256, 16, 2
        seed = _LAYER_SEED_TINY
        Tn = 8 if T is None else T
    else:
        H, E, k = QWEN["H"], QWEN["E"], QWEN["k"]
        seed = _LAYER_SEED_Q4 if name == "q48q" else _LAYER_SEED
        Tn = {"q8": 8, "q64": 64, "q48q": 48, "q4096": 4096}[name] if T is None else T
    xseed = _X_SEED[name] if T is None else [_X_SEED[name], T]
    wr = _normal_bf16(_child_rng(seed, 0, 0), (E, H), 0.02)
    bias = skew_bias(E) if name == "q4096" else None
    return activations(Tn, H, xseed), wr, bias, k


# pre-block inputs of the fused residual + RMSNorm + router step
PRENORM_EPS = 1e-6     # Qwen3's RMSNorm epsilon
_PRENORM_SEED = 3001


def prenorm_inputs(T: int, H: int, seed=None) -> dict:
    """Residual stream (std 2), the sublayer output added to it (std 1) and
    the norm's per-channel weight (mean 1, std 0.25), all bf16, plus eps.
    Independent streams per part: (seed, 0) residual, (seed, 1) delta,
    (seed, 2) gamma."""
    seed = _PRENORM_SEED if seed is None else seed
    res = _normal_bf16(np.random.Generator(np.random.PCG64([seed, 0])), (T, H), 2.0)
    delta = _normal_bf16(np.random.Generator(np.random.PCG64([seed, 1])), (T, H), 1.0)
    g = np.random.Generator(np.random.PCG64([seed, 2])).standard_normal(H, dtype=np.float32)
    gamma = f32_to_bf16_bits(np.float32(1.0) + np.float32(0.25) * g)
    return dict(residual=res, delta=delta, gamma=gamma, eps=np.float32(PRENORM_EPS))


LORA_RANK = 16
_LORA_SEED = 4001


def lora_adapters(E: int, H: int, I: int, rank: int = LORA_RANK, seed=None, alpha: float = 32.0) -> dict:
    """fp32 adapters ~ N(0, 0.02) for every expert's stacked gate/up (A [E][r][H],
    B [E][2I][r]) and down (A [E][r][I], B [E][H][r]), scale alpha / r.
    Streams (seed, 0..3) in that order."""
    seed = _LORA_SEED if seed is None else seed
    g = lambda part, shape: (np.random.Generator(np.random.PCG64([seed, part]))  # noqa: E731
                             .standard_normal(shape, dtype=np.float32) * np.float32(0.02))
    return dict(a_gate_up=g(0, (E, rank, H)), b_gate_up=g(1, (E, 2 * I, rank)),
                a_down=g(2, (E, rank, I)), b_down=g(3, (E, H, rank)), scale=np.float32(alpha / rank))


def random_codebook(seed: int) -> np.ndarray:
    """16 ascending fp32 values: -1, 14 uniform draws in (-1, 1), +1.  Unlike
    the normal-quantile table it has no structure (no exact zero, entries
    with all 24 significant bits)."""
    rng = np.random.Generator(np.random.PCG64([seed, 77]))
    mid = np.sort(rng.uniform(-1.0, 1.0, 14)).astype(np.float32)
    return np.concatenate([[np.float32(-1.0)], mid, [np.float32(1.0)]]).astype(np.float32)


def make_small(T: int, H: int, E: int, k: int, I: int, seed: int, wfmt: str = "bf16",
               bias: bool = False, x_std: float = 1.0, w_std: float = 0.02,
               codebook: Optional[np.ndarray] = None) -> MoEInputs:
    """Arbitrary small shape for edge-case tests (own seed, one draw order:
    router, gate/up, down, activations).  codebook: the 4-bit table (default
    the normal-quantile one)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    wr = _normal_bf16(rng, (E, H), w_std)
    if wfmt == "bf16":
        wgu = _normal_bf16(rng, (E, 2 * I, H), w_std)
        wd = _normal_bf16(rng, (E, H, I), w_std)
        extra = dict(w_gate_up=wgu, w_down=wd)
    else:
        cb = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=np.float32)
        qgu, sgu = quantize_nf4(rng.standard_normal((E, 2 * I, H), dtype=np.float32) * np.float32(w_std), cb)
        qd, sd = quantize_nf4(rng.standard_normal((E, H, I), dtype=np.float32) * np.float32(w_std), cb)
        extra = dict(q_gate_up=qgu, s_gate_up=sgu, q_down=qd, s_down=sd, codebook=cb)
    x = _normal_bf16(rng, (T, H), x_std)
    b = skew_bias(E) if bias else None
    return MoEInputs(f"small_T{T}_H{H}_E{E}_k{k}_I{I}_{wfmt}", T, H, E, k, I, wfmt, x, wr, b, **extra)
