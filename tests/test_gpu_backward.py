"""Backward of the block (frozen weights, the forward's routing) against the
fp64 oracle's chain rule: input and routing-weight gradients within the bf16
tolerance; the same bits on every run and whatever the batch; the
unsupported configurations refused.  A training forward (train=1) keeps the
gate/up pre-activations; its outputs are the same bits as a plain forward's.
With rank-16 LoRA adapters: the chain rule through W + scale*B A and the
four adapter gradients, against the oracle's, zero for experts no row
reached; zero B gives the frozen-weight d_x bit for bit.  With a 4-bit
base (the GRPO setting), against the oracle on the dequantised weights."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from mixture_experts_decode_router_amd import _lib as L
from mixture_experts_decode_router_amd.layer import MoELayer
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_weights, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q8": ("q64", 64), "q64": ("q64", 64)}


def d_out_for(T, H, seed=17):
    return np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32)


def gpu_backward(lay, x_bits, d_out):
    x = lay.upload_x(x_bits)
    lay.forward(x)
    d_x, d_w = lay.backward(x, torch.from_numpy(d_out).cuda())
    torch.cuda.synchronize()
    return d_x.cpu().numpy(), d_w.cpu().numpy()


def rel(a, ref):
    return float(np.abs(np.asarray(a, np.float64) - ref).max() / np.sqrt(np.mean(ref * ref)))


@pytest.mark.parametrize("name,T", [("tiny", 8), ("tiny", 33), ("q8", None), ("q64", 24)])
def test_backward_matches_oracle(name, T):
    inp = workload(name, T)
    lay = layer(*LAYER_OF[name]).with_options(train=True)
    d_out = d_out_for(inp.T, inp.H)
    say(f"[gpu] backward {name} T={inp.T}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    base = "q64" if name in ("q8", "q64") else name
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights(base))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), b["routing"]["ids"])
    ex, ew = rel(d_x, b["d_x"]), rel(d_w, b["d_w"])
    say(f"[gpu]   d_x max|err|/rms {ex:.3e}, d_w max|err|/rms {ew:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16


def test_backward_deterministic_and_batch_independent():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_options(train=True)
    d_out = d_out_for(64, inp.H, seed=5)
    a = gpu_backward(lay, inp.x, d_out)
    b = gpu_backward(lay, inp.x, d_out)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = gpu_backward(lay, inp.x[:13], d_out[:13])
    assert np.array_equal(c[0], a[0][:13]) and np.array_equal(c[1], a[1][:13])


def test_backward_nf4_deterministic_and_batch_independent():
    inp = workload("q48q", 48)
    lay = layer("q48q", 64).with_options(train=True).with_lora(S.lora_adapters(inp.E, inp.H, inp.I))
    d_out = d_out_for(48, inp.H, seed=7)
    a = gpu_backward_lora(lay, inp.x, d_out)
    b = gpu_backward_lora(lay, inp.x, d_out)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert all(np.array_equal(a[2][n], b[2][n]) for n in LORA_NAMES)
    c = gpu_backward_lora(lay, inp.x[:11], d_out[:11])
    assert np.array_equal(c[0], a[0][:11]) and np.array_equal(c[1], a[1][:11])


def test_backward_unrenormalised_at_prefill_sizes():
    # top-k weights without renormalisation: the logit gradient reaches all E
    # experts through the router's stored partials, also after an MFMA forward
    inp = workload("tiny", 256)
    lay = layer("tiny", 256).with_options(train=True, renorm=False)
    d_out = d_out_for(inp.T, inp.H, seed=31)
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("tiny"), renorm=False)
    ex, ew = rel(d_x, ref["d_x"]), rel(d_w, ref["d_w"])
    say(f"[gpu] unrenormalised backward tiny T={inp.T}: d_x {ex:.3e}, d_w {ew:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16


def test_backward_refuses_unsupported_configurations():
    inp = workload("q64", 64)
    x = torch.zeros(8, inp.H, dtype=torch.int16, device="cuda")
    g = torch.zeros(8, inp.H, dtype=torch.float32, device="cuda")
    for lay in (layer("q64", 64), layer("q64", 64, tiled=False).with_options(train=True),
                layer("q48q", 64, tiled=False).with_options(train=True)):
        lay.forward(x)
        with pytest.raises(L.MoEError) as ei:
            lay.backward(x, g)
        assert ei.value.status == L.MOE_ERR_UNSUPPORTED
    # a 4-bit base is frozen: no expert-weight gradients
    lay = layer("q48q", 64).with_options(train=True)
    lay.forward(x)
    with pytest.raises(L.MoEError) as ei:
        lay.backward(x, g, weight_grads=weight_grad_buffers(lay))
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("T,with_lora", [(48, False), (48, True), (7, True)])
def test_backward_nf4_matches_oracle(T, with_lora):
    # the 4-bit base of the GRPO setting (rank-16 LoRA on 4-bit weights):
    # the oracle runs on the identically dequantised weights, whose fp32
    # codebook entries the kernels take as two bf16 parts (17 significant
    # bits), so the adapter gradients meet the bf16 base's bound (with one
    # bf16 part, the codebook's own rounding showed 4-7 % of rms there)
    inp = workload("q48q", T)
    lay = layer("q48q", 64).with_options(train=True)
    d = S.lora_adapters(inp.E, inp.H, inp.I) if with_lora else None
    if d is not None:
        lay = lay.with_lora(d)
    d_out = d_out_for(inp.T, inp.H, seed=41)
    say(f"[gpu] backward 4-bit T={inp.T} lora={with_lora}")
    x = lay.upload_x(inp.x)
    out = lay.forward(x)
    res = lay.backward(x, torch.from_numpy(d_out).cuda())
    torch.cuda.synchronize()
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("q48q"),
                             lora=None if d is None else O.LoRA(**d))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), b["routing"]["ids"])
    errs = {"d_x": rel(res[0].cpu().numpy(), b["d_x"]), "d_w": rel(res[1].cpu().numpy(), b["d_w"])}
    if d is not None:
        for n in LORA_NAMES:
            errs[n] = rel(res[2][n].cpu().numpy(), b["d_" + n])
    say("[gpu]   max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_NF4 and errs["d_w"] <= TOL_NF4
    if d is not None:
        assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)


@pytest.mark.parametrize("cb", ["normal", "random"])
def test_backward_nf4_skewed_many_rows_per_expert(cb):
    # a 4-bit base with skewed routing, so that one expert gets more than
    # one 16-row work item, and a codebook of arbitrary fp32 values (or the
    # normal-quantile one); rank-16 adapters, against the oracle on the
    # dequantised weights
    book = S.random_codebook(5) if cb == "random" else None
    inp = S.make_small(96, 256, 16, 2, 128, seed=61, wfmt="nf4", bias=True, codebook=book)
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    lay = MoELayer(inp, t_max=96, train=True).with_lora(d)
    d_out = d_out_for(inp.T, inp.H, seed=43)
    say(f"[gpu] backward 4-bit skewed T={inp.T} codebook={cb}")
    d_x, d_w, g = gpu_backward_lora(lay, inp.x, d_out)
    counts = lay.views(inp.T)["counts"].cpu().numpy()
    assert counts.max() > 16
    ref = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp), lora=O.LoRA(**d))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), ref["routing"]["ids"])
    errs = {"d_x": rel(d_x, ref["d_x"]), "d_w": rel(d_w, ref["d_w"])}
    for n in LORA_NAMES:
        errs[n] = rel(g[n], ref["d_" + n])
    say(f"[gpu]   max rows per expert {counts.max()}; max|err|/rms " +
        ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_NF4 and errs["d_w"] <= TOL_NF4
    assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)


@pytest.mark.parametrize("T", [256, 1024])
def test_backward_at_prefill_sizes(T):
    # T*k >= 32*E: the training forward runs the MFMA prefill kernels, which
    # also keep g, u (outputs the same bits as an inference forward); the
    # backward's tiled transposed GEMMs run over the same 128-row items
    # (several per expert at T = 1024) and match the oracle's chain rule,
    # its rows the same bits as a decode-sized call's (16-row GEMVs); also
    # with the expert-weight gradients and with LoRA adapters
    inp = workload("tiny", T)
    d_out = d_out_for(inp.T, inp.H, seed=29)
    inf = layer("tiny", 1024)
    lay = inf.with_options(train=True)
    x = inf.upload_x(inp.x)
    a = inf.forward(x)
    b = lay.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    say(f"[gpu] backward tiny at prefill size T={inp.T}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("tiny"))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), ref["routing"]["ids"])
    ex, ew = rel(d_x, ref["d_x"]), rel(d_w, ref["d_w"])
    say(f"[gpu]   d_x max|err|/rms {ex:.3e}, d_w max|err|/rms {ew:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16
    s_x, s_w = gpu_backward(lay, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])
    # with the expert-weight gradients (the down pass with v in two parts)
    x = lay.upload_x(inp.x)
    lay.forward(x)
    wg = weight_grad_buffers(lay)
    res = lay.backward(x, torch.from_numpy(d_out).cuda(), weight_grads=wg)
    torch.cuda.synchronize()
    ref = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("tiny"), weight_grads=True,
                               wgrad_experts=list(range(inp.E)))
    errs = {"d_x": rel(res[0].cpu().numpy(), ref["d_x"])}
    counts = lay.views(inp.T)["counts"].cpu().numpy()
    for key, dev in (("d_w_gate_up", wg[0]), ("d_w_down", wg[1])):
        assert all(not dev[e].any() for e in range(inp.E) if counts[e] == 0)
        errs[key] = max(rel(dev[e].cpu().numpy(), ref[key][e]) for e in range(inp.E) if counts[e] > 0)
    say("[gpu]   with weight gradients max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16
    assert errs["d_w_gate_up"] <= TOL_LORA_GRAD and errs["d_w_down"] <= TOL_LORA_GRAD
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    ll = lay.with_lora(d)
    d_x, d_w, g = gpu_backward_lora(ll, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("tiny"), lora=O.LoRA(**d))
    errs = {"d_x": rel(d_x, ref["d_x"]), "d_w": rel(d_w, ref["d_w"])}
    for n in LORA_NAMES:
        errs[n] = rel(g[n], ref["d_" + n])
    say("[gpu]   with LoRA max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16 and errs["d_w"] <= TOL_BF16
    assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)
    s_x, s_w, _ = gpu_backward_lora(ll, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])


def test_backward_lora_adapter_gradients_both_prefill_forms():
    # T*k >= 32*E: the adapter gradients are formed per 128-row work item
    # (partial sums in y's memory, then an ordered sum over each expert's
    # items) where every item's partial fits there, else per expert with 8
    # row groups.  tiny at T = 256: with t_max = 1024 both passes take the
    # item form; with t_max = 256 the gate/up pass's partials do not fit and
    # it takes the row-group form.  Both against the oracle; d_x, d_w and the
    # down-adapter gradients (the same form in both) the same bits
    inp = workload("tiny", 256)
    d_out = d_out_for(inp.T, inp.H, seed=31)
    d = S.lora_adapters(inp.E, inp.H, inp.I, seed=5)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("tiny"), lora=O.LoRA(**d))
    res = {}
    for t_max in (1024, 256):
        lay = MoELayer(inp, t_max=t_max, train=True).with_lora(d)
        say(f"[gpu] backward tiny T={inp.T} t_max={t_max} with LoRA")
        res[t_max] = gpu_backward_lora(lay, inp.x, d_out)
        d_x, d_w, g = res[t_max]
        errs = {"d_x": rel(d_x, ref["d_x"]), "d_w": rel(d_w, ref["d_w"])}
        for n in LORA_NAMES:
            errs[n] = rel(g[n], ref["d_" + n])
        say("[gpu]   max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
        assert errs["d_x"] <= TOL_BF16 and errs["d_w"] <= TOL_BF16
        assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)
    a, b = res[1024], res[256]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2]["a_down"], b[2]["a_down"]) and np.array_equal(a[2]["b_down"], b[2]["b_down"])


@pytest.mark.parametrize("T", [300, 700])
def test_backward_bf16_at_prefill_sizes_ragged_tiles(T):
    # bf16 weights at T*k >= 32*E with H = 384 and I = 128: the gate/up pass's
    # second 256-column tile and the down pass's only one are partly past the
    # columns (their copies clamp to the last column block, those columns are
    # never stored), and the last item of each expert is partly past its rows;
    # against the oracle, with and without adapters, and the rows the same
    # bits as a decode-sized call's (16-row GEMVs)
    inp = S.make_small(T, 384, 16, 2, 128, seed=T + 11, bias=True)
    d_out = d_out_for(inp.T, inp.H, seed=53)
    lay = MoELayer(inp, t_max=T, train=True)
    say(f"[gpu] backward bf16 H=384 I=128 at prefill size T={T}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), ref["routing"]["ids"])
    ex, ew = rel(d_x, ref["d_x"]), rel(d_w, ref["d_w"])
    say(f"[gpu]   d_x {ex:.3e}, d_w {ew:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16
    s_x, s_w = gpu_backward(lay, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])
    d = S.lora_adapters(inp.E, inp.H, inp.I, seed=T)
    ll = lay.with_lora(d)
    d_x, d_w, g = gpu_backward_lora(ll, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp), lora=O.LoRA(**d))
    errs = {"d_x": rel(d_x, ref["d_x"]), "d_w": rel(d_w, ref["d_w"])}
    for n in LORA_NAMES:
        errs[n] = rel(g[n], ref["d_" + n])
    say("[gpu]   with LoRA max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16 and errs["d_w"] <= TOL_BF16
    assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)
    s_x, s_w, _ = gpu_backward_lora(ll, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])


def test_training_forward_gives_the_same_output():
    inp = workload("q64", 64)
    base = layer("q64", 64)
    tr = base.with_options(train=True)
    x = base.upload_x(inp.x)
    a = base.forward(x)
    b = tr.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)



LORA_NAMES = ("a_gate_up", "b_gate_up", "a_down", "b_down")
# Adapter gradients: every factor is fp32 (U = A x, z = B^T v, h = silu(g) u
# from the kept g, u) except d_h, whose GEMV takes v as two bf16 parts (about
# 16 bits); the weights are exact bf16 with fp32 accumulation.  Elementwise
# relative error is then ~1e-5; these rank-1 (per row) outer products have
# max/rms ratios up to ~20, so max|err|/rms ~2e-4; 2e-3 leaves a factor 10.
TOL_LORA_GRAD = 2e-3


def gpu_backward_lora(lay, x_bits, d_out):
    x = lay.upload_x(x_bits)
    lay.forward(x)
    d_x, d_w, g = lay.backward(x, torch.from_numpy(d_out).cuda())
    torch.cuda.synchronize()
    return d_x.cpu().numpy(), d_w.cpu().numpy(), {n: v.cpu().numpy() for n, v in g.items()}


@pytest.mark.parametrize("name,T", [("tiny", 8), ("tiny", 33), ("q8", None), ("q64", 24)])
def test_backward_lora_matches_oracle(name, T):
    inp = workload(name, T)
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    lay = layer(*LAYER_OF[name]).with_options(train=True).with_lora(d)
    d_out = d_out_for(inp.T, inp.H, seed=23)
    say(f"[gpu] backward with LoRA {name} T={inp.T}")
    d_x, d_w, g = gpu_backward_lora(lay, inp.x, d_out)
    base = "q64" if name in ("q8", "q64") else name
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights(base), lora=O.LoRA(**d))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), b["routing"]["ids"])
    errs = {"d_x": rel(d_x, b["d_x"]), "d_w": rel(d_w, b["d_w"])}
    for n in LORA_NAMES:
        assert g[n].shape == d[n].shape
        errs[n] = rel(g[n], b["d_" + n])
    say("[gpu]   max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16 and errs["d_w"] <= TOL_BF16
    assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)
    # experts no row reached: exactly zero gradients
    hit = np.zeros(inp.E, bool)
    hit[b["routing"]["ids"].ravel()] = True
    for n in LORA_NAMES:
        assert not g[n][~hit].any()
        assert np.abs(g[n][hit]).max() > 0


def test_backward_lora_deterministic():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_options(train=True).with_lora(S.lora_adapters(inp.E, inp.H, inp.I))
    d_out = d_out_for(64, inp.H, seed=29)
    a = gpu_backward_lora(lay, inp.x, d_out)
    b = gpu_backward_lora(lay, inp.x, d_out)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert all(np.array_equal(a[2][n], b[2][n]) for n in LORA_NAMES)
    # a row's d_x depends on its token only; the adapter gradients sum over the batch
    c = gpu_backward_lora(lay, inp.x[:13], d_out[:13])
    assert np.array_equal(c[0], a[0][:13]) and np.array_equal(c[1], a[1][:13])


def test_backward_lora_zero_b_is_the_frozen_backward():
    """B = 0: the adapters add exactly nothing to g, u or y (so d_w is the
    frozen backward's, bit for bit), z = B^T v = 0 makes d_A exactly zero,
    d_B and d_x are still the oracle's (d_x within the tolerance: with
    adapters the down GEMV carries v in two bf16 parts)."""
    inp = workload("q64", 16)
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    d["b_gate_up"][:] = 0
    d["b_down"][:] = 0
    base = layer("q64", 64).with_options(train=True)
    lay = base.with_lora(d)
    d_out = d_out_for(16, inp.H, seed=31)
    ref = gpu_backward(base, inp.x, d_out)
    d_x, d_w, g = gpu_backward_lora(lay, inp.x, d_out)
    assert np.array_equal(d_w, ref[1])
    assert not g["a_gate_up"].any() and not g["a_down"].any()
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("q64"), lora=O.LoRA(**d))
    errs = {"d_x": rel(d_x, b["d_x"]), "d_x frozen": rel(ref[0], b["d_x"]),
            "b_down": rel(g["b_down"], b["d_b_down"]), "b_gate_up": rel(g["b_gate_up"], b["d_b_gate_up"])}
    say("[gpu]   zero B: max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16 and errs["d_x frozen"] <= TOL_BF16
    assert errs["b_down"] <= TOL_LORA_GRAD and errs["b_gate_up"] <= TOL_LORA_GRAD


def weight_grad_buffers(lay):
    return (torch.full((lay.E, 2 * lay.I, lay.H), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((lay.E, lay.H, lay.I), float("nan"), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("name,T,with_lora", [("tiny", 8, False), ("tiny", 33, True), ("q8", None, False),
                                              ("q64", 24, True)])
def test_backward_weight_grads_match_oracle(name, T, with_lora):
    """Expert-weight gradients (fp32, every expert: zeros where no row went)
    against the oracle's; at the Qwen shape on a sample of experts (the most
    and the least loaded active ones and one more) plus every inactive one."""
    inp = workload(name, T)
    d = S.lora_adapters(inp.E, inp.H, inp.I) if with_lora else None
    lay = layer(*LAYER_OF[name]).with_options(train=True)
    if d is not None:
        lay = lay.with_lora(d)
    d_out = d_out_for(inp.T, inp.H, seed=37)
    say(f"[gpu] backward with weight gradients {name} T={inp.T} lora={with_lora}")
    x = lay.upload_x(inp.x)
    lay.forward(x)
    wg = weight_grad_buffers(lay)
    res = lay.backward(x, torch.from_numpy(d_out).cuda(), weight_grads=wg)
    torch.cuda.synchronize()
    counts = lay.views(inp.T)["counts"].cpu().numpy()
    active = np.flatnonzero(counts)
    small = inp.E <= 16
    experts = list(range(inp.E)) if small else sorted({int(active[np.argmax(counts[active])]),
                                                       int(active[np.argmin(counts[active])]), int(active[0])})
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights("q64" if name != "tiny" else name),
                             lora=None if d is None else O.LoRA(**d), weight_grads=True, wgrad_experts=experts)
    errs = {"d_x": rel(res[0].cpu().numpy(), b["d_x"])}
    for key, dev in (("d_w_gate_up", wg[0]), ("d_w_down", wg[1])):
        for e in experts:
            got = dev[e].cpu().numpy()
            ref = b[key][e]
            if counts[e] == 0:
                assert not got.any(), (key, e)
            else:
                errs[f"{key}[{e}]"] = rel(got, ref)
    inactive = np.flatnonzero(counts == 0)
    for dev in wg:
        assert not bool(torch.isnan(dev).any())
        if len(inactive):
            assert not bool(dev[torch.from_numpy(inactive).cuda()].any())
    say("[gpu]   max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_BF16
    assert all(v <= TOL_LORA_GRAD for k, v in errs.items() if k != "d_x")
    if d is not None:   # the adapter gradients are unchanged by also forming the weight gradients
        ref_l = gpu_backward_lora(lay, inp.x, d_out)
        for n in LORA_NAMES:
            assert np.array_equal(res[2][n].cpu().numpy(), ref_l[2][n])


def test_backward_weight_grads_wide_intermediate():
    """I > H: the down weight gradient forms h = silu(g) u from the kept
    g, u itself (no room for an fp32 h in y's memory); every expert
    against the oracle, several 32-row chunks per expert."""
    inp = S.make_small(80, 256, 16, 4, 384, seed=71, bias=True)
    lay = MoELayer(inp, t_max=80, train=True)
    d_out = d_out_for(inp.T, inp.H, seed=47)
    say(f"[gpu] backward with weight gradients, I > H, T={inp.T}")
    x = lay.upload_x(inp.x)
    lay.forward(x)
    wg = weight_grad_buffers(lay)
    res = lay.backward(x, torch.from_numpy(d_out).cuda(), weight_grads=wg)
    torch.cuda.synchronize()
    counts = lay.views(inp.T)["counts"].cpu().numpy()
    assert counts.max() > 32
    b = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp), weight_grads=True,
                             wgrad_experts=list(range(inp.E)))
    errs = {"d_x": rel(res[0].cpu().numpy(), b["d_x"])}
    for key, dev in (("d_w_gate_up", wg[0]), ("d_w_down", wg[1])):
        for e in range(inp.E):
            got = dev[e].cpu().numpy()
            if counts[e] == 0:
                assert not got.any(), (key, e)
            else:
                errs[f"{key}[{e}]"] = rel(got, b[key][e])
    worst = max((v, k) for k, v in errs.items() if k != "d_x")
    say(f"[gpu]   d_x {errs['d_x']:.3e}; worst weight gradient {worst[1]} {worst[0]:.3e}")
    assert errs["d_x"] <= TOL_BF16 and worst[0] <= TOL_LORA_GRAD


def test_backward_weight_grads_deterministic():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_options(train=True)
    d_out = torch.from_numpy(d_out_for(64, inp.H, seed=41)).cuda()
    x = lay.upload_x(inp.x)
    outs = []
    for _ in range(2):
        lay.forward(x)
        wg = weight_grad_buffers(lay)
        d_x, d_w = lay.backward(x, d_out, weight_grads=wg)
        outs.append((d_x, d_w, wg))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2][0], outs[1][2][0]) and torch.equal(outs[0][2][1], outs[1][2][1])


@pytest.mark.parametrize("name,T", [("tiny", 8), ("tiny", 33), ("q8", None), ("q64", 24)])
def test_backward_unrenormalised_matches_oracle(name, T):
    """Top-k weights without renormalisation: the logit gradient reaches all
    E experts, so d_x carries the router rows of every expert."""
    inp = workload(name, T)
    lay = layer(*LAYER_OF[name]).with_options(renorm=False, train=True)
    d_out = d_out_for(inp.T, inp.H, seed=43)
    say(f"[gpu] backward without renormalisation {name} T={inp.T}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    base = "q64" if name in ("q8", "q64") else name
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights(base), renorm=False)
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), b["routing"]["ids"])
    r = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights(base))
    ex, ew = rel(d_x, b["d_x"]), rel(d_w, b["d_w"])
    gap = rel(r["d_x"], b["d_x"])
    say(f"[gpu]   d_x max|err|/rms {ex:.3e}, d_w {ew:.3e}; renormalised d_x differs by {gap:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16
    assert gap > 10 * ex   # the test separates the two forms


@pytest.mark.parametrize("T,cb", [(600, "normal"), (1100, "random")])
def test_backward_nf4_at_prefill_sizes(T, cb):
    # a 4-bit base at T*k >= 32*E: the training forward runs the 4-bit MFMA
    # prefill kernels (outputs the same bits as an inference forward) and the
    # backward's 4-bit tiled transposed GEMMs run over the same 128-row items
    # (several per expert at T = 1100; H = 384 leaves a ragged 256-column
    # tile), against the oracle on the dequantised weights, with and without
    # adapters; rows are the same bits as a decode-sized call's (16-row GEMVs)
    book = S.random_codebook(11) if cb == "random" else None
    inp = S.make_small(T, 384, 16, 2, 256, seed=T + 3, wfmt="nf4", bias=True, codebook=book)
    d_out = d_out_for(inp.T, inp.H, seed=47)
    inf = MoELayer(inp, t_max=T)
    lay = MoELayer(inp, t_max=T, train=True)
    x = inf.upload_x(inp.x)
    a = inf.forward(x)
    b = lay.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    say(f"[gpu] backward 4-bit at prefill size T={T} codebook={cb}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), ref["routing"]["ids"])
    counts = lay.views(inp.T)["counts"].cpu().numpy()
    ex, ew = rel(d_x, ref["d_x"]), rel(d_w, ref["d_w"])
    say(f"[gpu]   max rows per expert {counts.max()}; d_x {ex:.3e}, d_w {ew:.3e}")
    assert ex <= TOL_NF4 and ew <= TOL_NF4
    s_x, s_w = gpu_backward(lay, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])
    d = S.lora_adapters(inp.E, inp.H, inp.I, seed=T)
    ll = lay.with_lora(d)
    d_x, d_w, g = gpu_backward_lora(ll, inp.x, d_out)
    ref = O.backward_per_token(inp, d_out.astype(np.float64), O.ExpertWeights(inp), lora=O.LoRA(**d))
    errs = {"d_x": rel(d_x, ref["d_x"]), "d_w": rel(d_w, ref["d_w"])}
    for n in LORA_NAMES:
        errs[n] = rel(g[n], ref["d_" + n])
    say("[gpu]   with LoRA max|err|/rms " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["d_x"] <= TOL_NF4 and errs["d_w"] <= TOL_NF4
    assert all(errs[n] <= TOL_LORA_GRAD for n in LORA_NAMES)
    s_x, s_w, _ = gpu_backward_lora(ll, inp.x[:24], d_out[:24])
    assert np.array_equal(s_x, d_x[:24]) and np.array_equal(s_w, d_w[:24])
