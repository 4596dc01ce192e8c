"""The pre-block step (residual add + RMSNorm) fused into the router pass,
against the fp64 oracle: r bit-exact; x the correctly rounded bf16 of the
oracle's value except where that value lies within fp32 rounding of a
midpoint between two bf16 numbers (then either neighbour); routing of the
kernel's x bit-exact; the whole block bit-identical to the unfused call on
the same x."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_weights, rel_err, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q64": ("q64", 64), "q48q": ("q48q", 64), "q4096": ("q4096", 4096)}


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def dev(a, lay):
    return None if a is None else lay.upload_x(a)


def check_x(x_bits, x64, H):
    """x_bits == RNE(x64) except within delta of a bf16 midpoint, where the
    neighbour on the other side is allowed.  delta bounds the relative fp32
    error of the kernel's r * scale * gamma: the row's sum of squares is a
    chain of H/16 fp32 fmas per thread plus a 16-lane butterfly, the scale
    adds four roundings (divide, add, sqrt, reciprocal), the products two."""
    want = O.f64_to_bf16_rne(x64)
    bad = x_bits != want
    delta = (H / 16 + 16) * 2.0 ** -24
    if bad.any():
        step = np.abs(x_bits[bad].astype(np.int32) - want[bad].astype(np.int32))
        assert np.all(step == 1), "x differs by more than one bf16 step"
        mid = 0.5 * (O.bf16_bits_to_f64(x_bits[bad]) + O.bf16_bits_to_f64(want[bad]))
        v = x64[bad]
        assert np.all(np.abs(v - mid) <= delta * np.abs(v)), "x differs away from a rounding midpoint"
    return int(bad.sum())


def run_prenorm(name, T=None, with_delta=True, with_res_out=True, seed=None):
    inp = workload(name, T)
    lay = layer(*LAYER_OF[name])
    p = S.prenorm_inputs(inp.T, inp.H, seed)
    delta = p["delta"] if with_delta else None
    out, x_out, r_out = lay.forward_prenorm(dev(p["residual"], lay), dev(delta, lay), dev(p["gamma"], lay),
                                            float(p["eps"]), inp.T, write_residual=with_res_out)
    torch.cuda.synchronize()
    views = {k: v.clone() for k, v in lay.views(inp.T).items()}
    return inp, lay, p, delta, out.clone(), x_out.clone(), None if r_out is None else r_out.clone(), views


@pytest.mark.parametrize("name,T", [("tiny", 8), ("tiny", 33), ("q64", 64), ("q64", 5), ("q48q", 48),
                                    ("q4096", 4096)])
def test_prenorm_matches_oracle(name, T):
    inp, lay, p, delta, out, x_out, r_out, views = run_prenorm(name, T)
    say(f"[gpu] prenorm {name} T={T}")
    r_bits, x64 = O.residual_rmsnorm(p["residual"], delta, p["gamma"], p["eps"])
    assert np.array_equal(bits(r_out), r_bits)
    xb = bits(x_out)
    n_off = check_x(xb, x64, inp.H)
    say(f"[gpu]   x elements one bf16 step from the correctly rounded value (at a midpoint): {n_off}")
    # the kernel's x routes exactly like the oracle on the same x
    ids_o, w_o, _ = O.route(xb, inp.w_router, inp.k, inp.bias)
    assert np.array_equal(views["ids"].cpu().numpy(), ids_o)
    np.testing.assert_allclose(views["w"].cpu().numpy(), w_o, rtol=2e-5, atol=1e-6)
    # the fused call is the unfused block on that x, bit for bit
    ref = lay.forward(x_out.clone())
    torch.cuda.synchronize()
    assert torch.equal(ref, out)
    if T <= 64:
        base = "q64" if name == "q64" else name
        ref_out, _ = O.forward_batched(inp.with_x(xb), oracle_weights(base))
        err = rel_err(out.cpu().numpy(), ref_out)
        tol = TOL_NF4 if inp.wfmt == "nf4" else TOL_BF16
        say(f"[gpu]   max|err|/rms = {err:.3e} (tolerance {tol})")
        assert err <= tol


def test_prenorm_without_delta_or_residual_out():
    inp, lay, p, delta, out, x_out, r_out, views = run_prenorm("q64", 16, with_delta=False, with_res_out=False)
    assert r_out is None
    _, x64 = O.residual_rmsnorm(p["residual"], None, p["gamma"], p["eps"])
    check_x(bits(x_out), x64, inp.H)


def test_prenorm_rows_do_not_depend_on_the_batch():
    """A row's x, r and output are the same bits in a batch of 64 and of 13."""
    a = run_prenorm("q64", 64)
    lay = a[1]
    p = a[2]
    out, x_out, r_out = lay.forward_prenorm(dev(p["residual"][:13], lay), dev(p["delta"][:13], lay),
                                            dev(p["gamma"], lay), float(p["eps"]), 13)
    torch.cuda.synchronize()
    assert torch.equal(x_out, a[5][:13])
    assert torch.equal(r_out, a[6][:13])
    assert torch.equal(out, a[4][:13])


def test_prenorm_graph_replay_equals_eager():
    inp = workload("q64", 64)
    lay = layer("q64", 64)
    p = S.prenorm_inputs(64, inp.H)
    stream = torch.cuda.Stream()
    res_s, del_s = dev(p["residual"], lay), dev(p["delta"], lay)
    gam_s = dev(p["gamma"], lay)
    x_s = torch.zeros(64, inp.H, dtype=torch.int16, device="cuda")
    r_s = torch.zeros(64, inp.H, dtype=torch.int16, device="cuda")
    out_s = torch.zeros(64, inp.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    say("[gpu] prenorm graph capture")
    lay.capture_prenorm([8, 64], res_s, del_s, gam_s, float(p["eps"]), r_s, x_s, out_s, stream)
    try:
        for T in (64, 5, 8):
            with torch.cuda.stream(stream):
                x_s.fill_(7)
                r_s.fill_(7)
                out_s.fill_(7.0)
                lay.replay(T, stream)
                e_out, e_x, e_r = lay.forward_prenorm(res_s[:T], del_s[:T], gam_s, float(p["eps"]), T,
                                                      stream=stream)
            stream.synchronize()
            assert torch.equal(out_s[:T], e_out), T
            assert torch.equal(x_s[:T], e_x), T
            assert torch.equal(r_s[:T], e_r), T
            assert bool((x_s[T:] == 7).all()) and bool((r_s[T:] == 7).all()) and bool((out_s[T:] == 7.0).all()), T
    finally:
        lay.release_graph()
