"""The layer's options against the oracle: top-k weights without
renormalisation (the full softmax taken at the chosen experts) and a bf16
output (the fp32 result rounded to nearest even, bit for bit)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_weights, rel_err, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q64": ("q64", 64), "q48q": ("q48q", 64), "q4096": ("q4096", 4096)}


@pytest.mark.parametrize("name", ["tiny", "q64", "q4096"])
def test_route_unrenormalised_matches_oracle(name):
    inp = workload(name)
    base = layer(*LAYER_OF[name])
    lay = base.with_options(renorm=False)
    say(f"[gpu] route without renormalisation {name} T={inp.T}")
    x = lay.upload_x(inp.x)
    ids, w, _ = lay.route(x, inp.T)
    ids_r, w_r, _ = base.route(x, inp.T)
    torch.cuda.synchronize()
    ids, w, ids_r, w_r = ids.cpu().numpy(), w.cpu().numpy(), ids_r.cpu().numpy(), w_r.cpu().numpy()
    ids_o, w_o, _ = O.route(inp.x, inp.w_router, inp.k, inp.bias, renorm=False)
    assert np.array_equal(ids, ids_o)
    assert np.array_equal(ids, ids_r)
    # the experts not chosen enter the denominator with their bounded MFMA
    # logits (errors ~1e-6 of the logit scale), hence rtol 1e-4
    np.testing.assert_allclose(w, w_o, rtol=1e-4, atol=1e-7)
    s = w.astype(np.float64).sum(axis=1)
    assert np.all(s <= 1.0 + 1e-5)
    np.testing.assert_allclose(w / s[:, None], w_r, rtol=1e-4, atol=1e-7)


@pytest.mark.parametrize("name", ["q64", "q48q"])
def test_forward_unrenormalised_matches_oracle(name):
    inp = workload(name)
    lay = layer(*LAYER_OF[name]).with_options(renorm=False)
    say(f"[gpu] forward without renormalisation {name}")
    out = lay.forward(lay.upload_x(inp.x))
    torch.cuda.synchronize()
    ref, _ = O.forward_batched(inp, oracle_weights(name), renorm=False)
    err = rel_err(out.cpu().numpy(), ref)
    tol = TOL_NF4 if inp.wfmt == "nf4" else TOL_BF16
    say(f"[gpu]   max|err|/rms = {err:.3e} (tolerance {tol})")
    assert err <= tol


@pytest.mark.parametrize("name", ["tiny", "q64", "q48q", "q4096"])
def test_bf16_output_is_fp32_output_rounded(name):
    """The bf16 output is the fp32 output rounded to nearest even (torch's
    float -> bfloat16 conversion), bit for bit, on the skinny, 4-bit and
    MFMA paths."""
    inp = workload(name)
    base = layer(*LAYER_OF[name])
    lay = base.with_options(out_bf16=True)
    say(f"[gpu] bf16 output {name} T={inp.T}")
    x = base.upload_x(inp.x)
    a = base.forward(x)
    b = lay.forward(x)
    torch.cuda.synchronize()
    assert b.dtype == torch.bfloat16 and b.shape == a.shape
    assert torch.equal(b.view(torch.int16), a.to(torch.bfloat16).view(torch.int16))


def test_bf16_output_graph_replay_equals_eager():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_options(out_bf16=True)
    stream = torch.cuda.Stream()
    x_static = torch.zeros(64, lay.H, dtype=torch.int16, device="cuda")
    out_static = torch.zeros(64, lay.H, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    say("[gpu] bf16 output graph capture")
    lay.capture([8, 64], x_static, out_static, stream)
    try:
        for T in (64, 5, 8):
            x = lay.upload_x(inp.x[:T])
            with torch.cuda.stream(stream):
                out_static.fill_(7.0)
                x_static[:T].copy_(x)
                lay.replay(T, stream)
                eager = lay.forward(x.clone(), stream=stream)
            stream.synchronize()
            assert torch.equal(out_static[:T].view(torch.int16), eager.view(torch.int16)), T
            assert bool((out_static[T:] == 7.0).all()), T
    finally:
        lay.release_graph()


def test_all_options_together_match_oracle_and_replay():
    """Pre-block step + LoRA adapters + weights without renormalisation + bf16
    output in one call, against the oracle on the kernel's x; a graph replay
    gives the same bits."""
    import synthetic as S
    inp = workload("q64", 64)
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    lay = layer("q64", 64).with_lora(d).with_options(out_bf16=True, renorm=False)
    p = S.prenorm_inputs(64, inp.H)
    res, dlt, gam = (lay.upload_x(p[n]) for n in ("residual", "delta", "gamma"))
    say("[gpu] pre-block + LoRA + softmax weights + bf16 out")
    out, x_out, r_out = lay.forward_prenorm(res, dlt, gam, float(p["eps"]), 64)
    torch.cuda.synchronize()
    xb = x_out.cpu().numpy().view(np.uint16)
    ref, rr = O.forward_batched(inp.with_x(xb), oracle_weights("q64"), renorm=False, lora=O.LoRA(**d))
    v = lay.views(64)
    assert np.array_equal(v["ids"].cpu().numpy(), rr["ids"])
    np.testing.assert_allclose(v["w"].cpu().numpy(), rr["w"], rtol=1e-4, atol=1e-7)
    err = rel_err(out.float().cpu().numpy(), ref)
    say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert out.dtype == torch.bfloat16 and err <= TOL_BF16
    stream = torch.cuda.Stream()
    xs = torch.zeros(64, inp.H, dtype=torch.int16, device="cuda")
    rs = torch.zeros(64, inp.H, dtype=torch.int16, device="cuda")
    os_ = torch.zeros(64, inp.H, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    lay.capture_prenorm([64], res, dlt, gam, float(p["eps"]), rs, xs, os_, stream)
    try:
        lay.replay(64, stream)
        stream.synchronize()
        assert torch.equal(xs, x_out) and torch.equal(rs, r_out)
        assert torch.equal(os_.view(torch.int16), out.view(torch.int16))
    finally:
        lay.release_graph()
