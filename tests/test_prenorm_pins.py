"""Pins of the oracle's pre-block step (residual add + RMSNorm feeding the
router) and of its fp64 -> bf16 rounding, against torch, closed forms and the
definition of round-to-nearest-even."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S


def bits_to_f64(b):
    return O.bf16_bits_to_f64(np.asarray(b, dtype=np.uint16))


# ---------------------------------------------------------------- rounding
def test_rne_hand_cases():
    """bf16 has 7 fraction bits: at 1.0 the spacing is 2^-7, the midpoints
    1 + 2^-8 (tie -> even 1.0) and 1 + 3*2^-8 (tie -> even 1 + 2^-6)."""
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, -2.5, 3.0, 0.0, -0.0])
    b = O.f64_to_bf16_rne(v)
    assert bits_to_f64(b).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 3.0, 0.0, 0.0]
    assert b[-2:].tolist() == [0x0000, 0x8000]


def test_rne_equals_fp32_path_on_fp32_values():
    """For values exactly representable in fp32 one rounding to bf16 is the
    same from fp64 or fp32 (the fp32 path is pinned to torch's cast)."""
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    assert np.array_equal(O.f64_to_bf16_rne(a.astype(np.float64)), S.f32_to_bf16_bits(a))


def test_rne_is_nearest_with_ties_to_even():
    """Definition: no bf16 value is nearer, and on an exact tie the even
    neighbour wins.  Values with bits below fp32 precision included (where
    rounding through fp32 first would go wrong)."""
    rng = np.random.default_rng(6)
    base = rng.standard_normal(20000) * np.exp(rng.uniform(-10, 10, 20000))
    # midpoints of bf16 neighbours, nudged by tiny amounts below fp32 resolution
    mids = (bits_to_f64(S.f32_to_bf16_bits(base.astype(np.float32)))
            * (1 + 2.0 ** -8 * rng.choice([-1, 1], 20000)))
    nudge = mids * rng.choice([-1.0, 0.0, 1.0], 20000) * 2.0 ** -35
    v = np.concatenate([base, mids, mids + nudge])
    b = O.f64_to_bf16_rne(v)
    x = bits_to_f64(b)
    up = bits_to_f64(b + np.uint16(1))
    dn = bits_to_f64(b - np.uint16(1))
    d, du, dd = np.abs(v - x), np.abs(v - up), np.abs(v - dn)
    assert np.all(d <= du) and np.all(d <= dd)
    tie = (d == du) | (d == dd)
    assert np.all((b[tie] & 1) == 0)


# ---------------------------------------------------------------- residual + RMSNorm
def test_residual_add_matches_torch_bf16_add():
    """torch adds two bf16 tensors in fp32 and rounds once to bf16, which
    equals the exact sum rounded (an fp32 sum of two bf16 values that is not
    exact lies far from any bf16 midpoint)."""
    p = S.prenorm_inputs(16, 512, seed=11)
    r_bits, _ = O.residual_rmsnorm(p["residual"], p["delta"], p["gamma"], p["eps"])
    t = (torch.from_numpy(p["residual"].view(np.int16)).view(torch.bfloat16)
         + torch.from_numpy(p["delta"].view(np.int16)).view(torch.bfloat16))
    assert np.array_equal(r_bits, t.view(torch.int16).numpy().view(np.uint16))


def test_rmsnorm_matches_torch_rms_norm():
    p = S.prenorm_inputs(16, 512, seed=12)
    r_bits, x = O.residual_rmsnorm(p["residual"], p["delta"], p["gamma"], p["eps"])
    ref = torch.nn.functional.rms_norm(torch.from_numpy(bits_to_f64(r_bits)), (512,),
                                       weight=torch.from_numpy(bits_to_f64(p["gamma"])),
                                       eps=float(p["eps"]))
    np.testing.assert_allclose(x, ref.numpy(), rtol=1e-14, atol=0)


def test_rmsnorm_constant_row_closed_form():
    """A row of one value c: x = c / sqrt(c^2 + eps) * gamma; at c^2 = eps the
    factor is 1/sqrt(2), so an ignored eps would show."""
    H = 256
    gamma = S.f32_to_bf16_bits(np.linspace(-2, 2, H).astype(np.float32))
    for c in (1.0, -3.0, 2.0 ** -10):
        res = S.f32_to_bf16_bits(np.full((1, H), c, dtype=np.float32))
        eps = np.float32(2.0 ** -20)   # = c^2 for the last c, exact in fp32
        r_bits, x = O.residual_rmsnorm(res, None, gamma, eps)
        assert np.array_equal(r_bits, res)
        expect = c / math.sqrt(c * c + float(eps)) * bits_to_f64(gamma)
        np.testing.assert_allclose(x[0], expect, rtol=1e-15, atol=0)
    assert abs(x[0][-1] / bits_to_f64(gamma)[-1] - 1 / math.sqrt(2)) < 1e-15


def test_rmsnorm_scale_invariant_without_eps():
    """Doubling r doubles the numerator and the root mean square exactly."""
    p = S.prenorm_inputs(4, 256, seed=13)
    r_bits, x = O.residual_rmsnorm(p["residual"], p["delta"], p["gamma"], 0.0)
    r2 = S.f32_to_bf16_bits((2.0 * bits_to_f64(r_bits)).astype(np.float32))
    _, x2 = O.residual_rmsnorm(r2, None, p["gamma"], 0.0)
    assert np.array_equal(x, x2)
