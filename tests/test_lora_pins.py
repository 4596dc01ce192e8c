"""Pins of the oracle's LoRA deltas: a hand-worked closed form, the merged-
weight identity W + scale*B A (distributivity, formed independently), zero B
leaving the block bit-for-bit unchanged, and batched = per token."""
import math

import numpy as np

import oracle as O
import synthetic as S
from tests.test_oracle_pins import hand_inputs


def rank1_lora(E, H, I, s):
    """A_gu = [1, 0, ...] (picks x[0]), B_gu adds it to every gate row and
    nothing to the up rows; the down adapter reads h[0] and adds it to
    output column 1."""
    a_gu = np.zeros((E, 1, H), np.float32)
    a_gu[:, 0, 0] = 1
    b_gu = np.zeros((E, 2 * I, 1), np.float32)
    b_gu[:, :I, 0] = 1
    a_d = np.zeros((E, 1, I), np.float32)
    a_d[:, 0, 0] = 1
    b_d = np.zeros((E, H, 1), np.float32)
    b_d[:, 1, 0] = 1
    return O.LoRA(a_gu, b_gu, a_d, b_d, s)


def test_lora_hand_closed_form():
    """Token 0 of the hand block (x = [1, 1/2], ids [0, 1], w = [e, 1]/(e+1))
    with scale 2: expert 0 gate = 1 + 2*1 = 3, up = 1, h0 = silu(3);
    y0 = [h0, -h0] + 2*[0, h0] = [h0, h0].  Expert 1 gate = -1 + 2 = 1,
    up = 2, h1 = 2 silu(1); y1 = [h1/2, h1/4] + [0, 2 h1]."""
    inp = hand_inputs()
    out, r = O.forward_per_token(inp, exact_router=True, lora=rank1_lora(4, 2, 1, 2.0))
    e = math.e
    w0, w1 = e / (e + 1), 1 / (e + 1)
    h0 = 3 / (1 + math.exp(-3))
    h1 = 2 * (1 / (1 + math.exp(-1)))
    np.testing.assert_array_equal(r["ids"], [[0, 1], [0, 1]])
    np.testing.assert_allclose(out[0], [w0 * h0 + w1 * h1 / 2, w0 * h0 + w1 * (h1 / 4 + 2 * h1)],
                               rtol=0, atol=1e-15)
    assert out[1].tolist() == [0.0, 0.0]     # x = 0: every delta is 0


def merged_weights(inp, lora):
    W = O.ExpertWeights(inp)
    M = O.ExpertWeights(inp)
    for e in range(inp.E):
        wg, wu, wd = W.get(e)
        a_gu, b_g, b_u, a_d, b_d = lora.get(e, inp.I)
        M._cache[e] = (wg + lora.scale * (b_g @ a_gu), wu + lora.scale * (b_u @ a_gu), wd + lora.scale * (b_d @ a_d))
    return M


def test_lora_equals_merged_weights():
    for inp in (S.make("tiny"), S.make_small(9, 128, 8, 3, 64, seed=31, wfmt="nf4")):
        lora = O.LoRA(**S.lora_adapters(inp.E, inp.H, inp.I, seed=7))
        a, _ = O.forward_per_token(inp, lora=lora)
        b, _ = O.forward_per_token(inp, merged_weights(inp, lora))
        assert O.rms(a - O.forward_per_token(inp)[0]) > 0.05 * O.rms(a)   # the delta matters
        assert np.abs(a - b).max() <= 1e-12 * O.rms(a)


def test_lora_zero_b_is_exactly_the_base_block():
    inp = S.make("tiny")
    d = S.lora_adapters(inp.E, inp.H, inp.I)
    d["b_gate_up"][:] = 0
    d["b_down"][:] = 0
    a, _ = O.forward_per_token(inp, lora=O.LoRA(**d))
    b, _ = O.forward_per_token(inp)
    assert np.array_equal(a, b)


def test_lora_batched_matches_per_token():
    inp = S.make("q8")
    lora = O.LoRA(**S.lora_adapters(inp.E, inp.H, inp.I))
    W = O.ExpertWeights(inp)
    a, _ = O.forward_per_token(inp, W, lora=lora)
    b, _ = O.forward_batched(inp, W, lora=lora)
    assert np.abs(a - b).max() <= 1e-12 * O.rms(a)
