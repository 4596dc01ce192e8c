"""Shared helpers of the GPU parity tests: workloads, device layers and oracle
results, each built once per test session."""
import functools
import sys

import numpy as np

import oracle as O
import synthetic as S

# tolerance on max|out - oracle| relative to rms(oracle out)
TOL_BF16 = 2e-2
TOL_NF4 = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def workload(name, T=None):
    return S.make(name, T=T)


@functools.lru_cache(maxsize=None)
def layer(name, t_max, tiled=True):
    """Device layer for a named workload (weights are shared between q8,
    q64 and q4096, but the q4096 layer carries the router bias).  tiled:
    expert weights packed into the fragment-tiled layout (else row-major)."""
    from mixture_experts_decode_router_amd.layer import MoELayer
    say(f"[gpu] uploading layer {name} t_max={t_max} tiled={tiled}")
    return MoELayer(workload(name), t_max=t_max, tiled=tiled)


@functools.lru_cache(maxsize=None)
def oracle_weights(name):
    return O.ExpertWeights(workload(name))


@functools.lru_cache(maxsize=None)
def oracle_forward(name, T=None):
    inp = workload(name, T)
    base = "q64" if name in ("q8", "q64", "q4096") else name
    W = oracle_weights(base)
    say(f"[gpu] oracle {name} T={inp.T}")
    return O.forward_batched(inp, W)


def rel_err(out_gpu, out_ref):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    return float(np.abs(out_gpu - out_ref).max() / O.rms(out_ref))


def topk_gap_audit(logits32, k):
    """Smallest gap between adjacent sorted logits among the top k+1 of any
    token (how close the routing decision came to a tie)."""
    s = -np.sort(-logits32.astype(np.float64), axis=1)[:, : k + 1]
    return float(np.diff(-s, axis=1).min()) if s.shape[1] > 1 else float("inf")
