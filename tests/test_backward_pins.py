"""Pins of the oracle's backward (frozen weights, fixed routing): torch
autograd in fp64 on an independent dense formulation, a finite-difference
check, and the zero-gradient case."""
import numpy as np
import torch

import oracle as O
import synthetic as S


def dense_torch_forward(inp, x, ids, round_logits=True):
    """Every expert on every token, masked to the oracle's choice, weights
    from torch's softmax over the chosen logits; differentiable in x."""
    wr = torch.from_numpy(O.bf16_bits_to_f64(inp.w_router))
    # the routing weights are taken on fp32 logits (fp32 dot, plus the fp32
    # bias in fp32); the rounding enters as a constant offset, so the
    # gradient flows through in fp64
    l64 = x @ wr.T
    l32 = l64.detach().float()
    if inp.bias is not None:
        l32 = l32 + torch.from_numpy(np.asarray(inp.bias, np.float32))
    l = l64 + (l32.double() - l64.detach()) if round_logits else l64
    mask = torch.zeros_like(l, dtype=torch.bool).scatter_(1, torch.from_numpy(ids.astype(np.int64)), True)
    g = torch.softmax(l.masked_fill(~mask, float("-inf")), dim=1)
    out = torch.zeros(x.shape[0], inp.H, dtype=torch.float64)
    for e in range(inp.E):
        gu = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up[e]))
        wd = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down[e]))
        h = torch.nn.functional.silu(x @ gu[: inp.I].T) * (x @ gu[inp.I:].T)
        out = out + g[:, e:e + 1] * (h @ wd.T)
    return out, g


def test_backward_matches_torch_autograd():
    for inp in (S.make("tiny"), S.make_small(6, 128, 8, 3, 64, seed=41, bias=True)):
        b = O.backward_per_token(inp, np.random.default_rng(3).standard_normal((inp.T, inp.H)))
        d_out = np.random.default_rng(3).standard_normal((inp.T, inp.H))
        x = torch.from_numpy(O.bf16_bits_to_f64(inp.x)).requires_grad_(True)
        out, g = dense_torch_forward(inp, x, b["routing"]["ids"])
        g.retain_grad()
        (out * torch.from_numpy(d_out)).sum().backward()
        ref = x.grad.numpy()
        assert np.abs(b["d_x"] - ref).max() <= 1e-12 * np.sqrt(np.mean(ref * ref))
        # the routing-weight gradient is d(out . d_out)/d g at the chosen experts
        dg = np.take_along_axis(g.grad.numpy(), b["routing"]["ids"].astype(np.int64), 1)
        np.testing.assert_allclose(b["d_w"], dg, rtol=1e-12, atol=1e-14)


def test_backward_finite_differences():
    """Central differences of L = sum(out * d_out) along a random direction
    (small enough that no routing decision changes), on the smooth form of
    the block (logits not rounded to fp32, which moves the result by ~1e-8
    relative)."""
    inp = S.make("tiny")
    rng = np.random.default_rng(9)
    d_out = rng.standard_normal((inp.T, inp.H))
    b = O.backward_per_token(inp, d_out)
    ids = b["routing"]["ids"]
    v = rng.standard_normal((inp.T, inp.H))
    x0 = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    eps = 1e-6

    def loss(x):
        out, _ = dense_torch_forward(inp, x, ids, round_logits=False)
        return float((out * torch.from_numpy(d_out)).sum())

    fd = (loss(x0 + eps * torch.from_numpy(v)) - loss(x0 - eps * torch.from_numpy(v))) / (2 * eps)
    assert abs(fd - float(np.sum(b["d_x"] * v))) <= 1e-5 * abs(fd)


def test_backward_zero_upstream_gives_zero():
    inp = S.make("tiny")
    b = O.backward_per_token(inp, np.zeros((inp.T, inp.H)))
    assert not b["d_x"].any() and not b["d_w"].any() and not b["d_logits"].any()


def test_backward_with_lora_matches_torch_autograd():
    """Adapter gradients and d_x through W + s B A against torch autograd on
    the dense formulation with the adapters as leaf tensors."""
    inp = S.make_small(5, 128, 8, 2, 64, seed=43)
    d = S.lora_adapters(inp.E, inp.H, inp.I, seed=2)
    lora = O.LoRA(**d)
    d_out = np.random.default_rng(8).standard_normal((inp.T, inp.H))
    b = O.backward_per_token(inp, d_out, lora=lora)
    ids = b["routing"]["ids"]
    x = torch.from_numpy(O.bf16_bits_to_f64(inp.x)).requires_grad_(True)
    P = {n: torch.from_numpy(np.asarray(d[n], np.float64)).requires_grad_(True)
         for n in ("a_gate_up", "b_gate_up", "a_down", "b_down")}
    s = float(d["scale"])
    wr = torch.from_numpy(O.bf16_bits_to_f64(inp.w_router))
    l64 = x @ wr.T
    l = l64 + (l64.detach().float().double() - l64.detach())
    mask = torch.zeros_like(l, dtype=torch.bool).scatter_(1, torch.from_numpy(ids.astype(np.int64)), True)
    gw = torch.softmax(l.masked_fill(~mask, float("-inf")), dim=1)
    out = torch.zeros(inp.T, inp.H, dtype=torch.float64)
    for e in range(inp.E):
        gu = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up[e])) + s * P["b_gate_up"][e] @ P["a_gate_up"][e]
        wd = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down[e])) + s * P["b_down"][e] @ P["a_down"][e]
        h = torch.nn.functional.silu(x @ gu[: inp.I].T) * (x @ gu[inp.I:].T)
        out = out + gw[:, e:e + 1] * (h @ wd.T)
    (out * torch.from_numpy(d_out)).sum().backward()
    rms = lambda a: float(np.sqrt(np.mean(a * a)))  # noqa: E731
    assert np.abs(b["d_x"] - x.grad.numpy()).max() <= 1e-12 * rms(x.grad.numpy())
    for n in P:
        ref = P[n].grad.numpy()
        assert np.abs(b["d_" + n] - ref).max() <= 1e-12 * rms(ref), n



def test_backward_weight_grads_match_torch_autograd():
    """The expert-weight gradients against torch autograd on the dense
    formulation with every expert's stacked gate/up and down matrices as
    leaf tensors, without and with LoRA adapters (W + s B A: the gradient in
    W is the same expression)."""
    inp = S.make_small(5, 128, 8, 2, 64, seed=47, bias=True)
    d_out = np.random.default_rng(13).standard_normal((inp.T, inp.H))
    for d in (None, S.lora_adapters(inp.E, inp.H, inp.I, seed=5)):
        lora = None if d is None else O.LoRA(**d)
        b = O.backward_per_token(inp, d_out, lora=lora, weight_grads=True)
        ids = b["routing"]["ids"]
        x = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
        wr = torch.from_numpy(O.bf16_bits_to_f64(inp.w_router))
        l64 = x @ wr.T
        l32 = l64.float() + torch.from_numpy(np.asarray(inp.bias, np.float32))
        mask = torch.zeros_like(l64, dtype=torch.bool).scatter_(1, torch.from_numpy(ids.astype(np.int64)), True)
        gw = torch.softmax(l32.double().masked_fill(~mask, float("-inf")), dim=1)
        WG = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up)).requires_grad_(True)
        WD = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down)).requires_grad_(True)
        out = torch.zeros(inp.T, inp.H, dtype=torch.float64)
        for e in range(inp.E):
            gu, wd = WG[e], WD[e]
            if d is not None:
                s = float(d["scale"])
                gu = gu + s * torch.from_numpy(np.asarray(d["b_gate_up"][e], np.float64)) @ \
                    torch.from_numpy(np.asarray(d["a_gate_up"][e], np.float64))
                wd = wd + s * torch.from_numpy(np.asarray(d["b_down"][e], np.float64)) @ \
                    torch.from_numpy(np.asarray(d["a_down"][e], np.float64))
            h = torch.nn.functional.silu(x @ gu[: inp.I].T) * (x @ gu[inp.I:].T)
            out = out + gw[:, e:e + 1] * (h @ wd.T)
        (out * torch.from_numpy(d_out)).sum().backward()
        for name, leaf in (("d_w_gate_up", WG), ("d_w_down", WD)):
            ref = leaf.grad.numpy()
            assert b[name].shape == ref.shape
            assert np.abs(b[name] - ref).max() <= 1e-12 * np.sqrt(np.mean(ref * ref)), name
        # experts no token chose get exactly zero
        miss = np.setdiff1d(np.arange(inp.E), ids.ravel())
        assert not b["d_w_gate_up"][miss].any() and not b["d_w_down"][miss].any()


def test_weight_grads_expert_subset_equals_full():
    """The per-expert form (for large shapes) gives the full arrays' slices."""
    inp = S.make("tiny")
    d = np.random.default_rng(1).standard_normal((inp.T, inp.H))
    a = O.backward_per_token(inp, d, weight_grads=True)
    b = O.backward_per_token(inp, d, weight_grads=True, wgrad_experts=[0, 3, 5])
    for e in (0, 3, 5):
        assert np.array_equal(a["d_w_gate_up"][e], b["d_w_gate_up"][e])
        assert np.array_equal(a["d_w_down"][e], b["d_w_down"][e])


def test_backward_unrenormalised_matches_torch_autograd():
    """Top-k weights without renormalisation (the full softmax at the chosen
    experts): d_x and the logit gradient over all E experts against torch
    autograd on the dense formulation with the unmasked softmax."""
    for inp in (S.make("tiny"), S.make_small(6, 128, 8, 3, 64, seed=53, bias=True)):
        d_out = np.random.default_rng(17).standard_normal((inp.T, inp.H))
        b = O.backward_per_token(inp, d_out, renorm=False)
        ids = b["routing"]["ids"]
        x = torch.from_numpy(O.bf16_bits_to_f64(inp.x)).requires_grad_(True)
        wr = torch.from_numpy(O.bf16_bits_to_f64(inp.w_router))
        l64 = x @ wr.T
        l32 = l64.detach().float()
        if inp.bias is not None:
            l32 = l32 + torch.from_numpy(np.asarray(inp.bias, np.float32))
        l = l64 + (l32.double() - l64.detach())
        l.retain_grad()
        mask = torch.zeros_like(l, dtype=torch.bool).scatter_(1, torch.from_numpy(ids.astype(np.int64)), True)
        g = torch.softmax(l, dim=1) * mask
        out = torch.zeros(inp.T, inp.H, dtype=torch.float64)
        for e in range(inp.E):
            gu = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up[e]))
            wd = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down[e]))
            h = torch.nn.functional.silu(x @ gu[: inp.I].T) * (x @ gu[inp.I:].T)
            out = out + g[:, e:e + 1] * (h @ wd.T)
        (out * torch.from_numpy(d_out)).sum().backward()
        ref = x.grad.numpy()
        assert np.abs(b["d_x"] - ref).max() <= 1e-12 * np.sqrt(np.mean(ref * ref))
        assert b["d_logits"].shape == (inp.T, inp.E)
        np.testing.assert_allclose(b["d_logits"], l.grad.numpy(), rtol=0,
                                   atol=1e-12 * np.abs(l.grad.numpy()).max())
        # the renormalised backward differs (its logit gradient lives on the k chosen only)
        r = O.backward_per_token(inp, d_out)
        assert np.abs(r["d_x"] - b["d_x"]).max() > 1e-6 * np.sqrt(np.mean(ref * ref))
