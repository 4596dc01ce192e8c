"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
closed forms, library routines, brute force and invariants.

The pages give no numeric worked example of the MoE block, so every pin here is
one of: a hand-derived closed form, a special case that reduces to a library
routine (scipy softmax, numpy stable argsort / bincount / cumsum, torch silu),
brute force over tiny inputs, or an invariant of the block's definition.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
import synthetic as S


def bf(vals):
    """Exactly representable floats -> bf16 bits (asserts exactness)."""
    a = np.asarray(vals, dtype=np.float32)
    bits = S.f32_to_bf16_bits(a)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, a), "value not bf16-representable"
    return bits


def hand_inputs():
    """E=4, k=2, H=2, I=1, two tokens (second one all zero)."""
    x = bf([[1.0, 0.5], [0.0, 0.0]])
    # logits for token 0: e0 = 1+1 = 2, e1 = 0.5+0.5 = 1, e2 = 0.25+0.25 = 0.5, e3 = 1
    wr = bf([[1.0, 2.0], [0.5, 1.0], [0.25, 0.5], [1.0, 0.0]])
    # gate rows (I=1) then up rows, per expert: [E][2I][H]
    wgu = bf([
        [[1.0, 0.0], [0.0, 2.0]],     # e0: g = 1,  u = 1
        [[0.0, -2.0], [2.0, 0.0]],    # e1: g = -1, u = 2
        [[1.0, 1.0], [1.0, 1.0]],     # e2 (never chosen for token 0)
        [[3.0, 0.0], [0.0, 3.0]],     # e3 (ties e1 but loses on index)
    ])
    wd = bf([
        [[1.0], [-1.0]],              # e0: y = [h, -h]
        [[0.5], [0.25]],              # e1: y = [h/2, h/4]
        [[1.0], [1.0]],
        [[1.0], [1.0]],
    ])
    return S.MoEInputs("hand", 2, 2, 4, 2, 1, "bf16", x, wr, None, wgu, wd)


def test_hand_worked_block_closed_form():
    """Closed form, derived by hand:
    token 0 logits [2, 1, 0.5, 1]; top-2 = e0, then the tie e1/e3 goes to e1.
    w = [e^2, e^1] / (e^2 + e^1) = [e/(e+1), 1/(e+1)].
    e0: h = silu(1)*1 = e/(e+1); y0 = [h, -h].
    e1: h = silu(-1)*2 = -2/(1+e); y1 = [h/2, h/4].
    out = w0*y0 + w1*y1 = [(e-1)/(e+1), -(e^2 + 1/2)/(e+1)^2].
    token 1 (x = 0): all logits 0 -> ids [0, 1], w = [1/2, 1/2], out = 0.
    """
    inp = hand_inputs()
    out, r = O.forward_per_token(inp, exact_router=True)
    e = math.e
    np.testing.assert_array_equal(r["ids"], [[0, 1], [0, 1]])
    np.testing.assert_allclose(r["w"][0], [e / (e + 1), 1 / (e + 1)], rtol=0, atol=1e-15)
    assert r["w"][1].tolist() == [0.5, 0.5]
    np.testing.assert_allclose(out[0], [(e - 1) / (e + 1), -(e * e + 0.5) / (e + 1) ** 2],
                               rtol=0, atol=1e-15)
    assert out[1].tolist() == [0.0, 0.0]
    out_b, _ = O.forward_batched(inp)
    np.testing.assert_allclose(out_b, out, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- router
def test_router_fast_path_equals_exact_sum_tiny():
    """numpy fp64 matmul then fp32 rounding == math.fsum (correctly rounded)
    then fp32 rounding, on every logit of the tiny workload."""
    inp = S.make("tiny")
    a = O.router_logits(inp.x, inp.w_router)
    b = O.router_logits(inp.x, inp.w_router, exact=True)
    assert np.array_equal(a, b)


def _exact_f32(q):
    """The fp32 value nearest to the rational q (ties to even mantissa),
    decided by exact rational distances (no intermediate rounding)."""
    from fractions import Fraction
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - q), int(np.array(c).view(np.uint32)) & 1))


@pytest.mark.parametrize("name", ["tiny", "q8", "q64", "q48q", "q4096"])
def test_router_logits_that_decide_routing_are_correctly_rounded(name):
    """Every logit among a token's top k+1 (the ones whose order and
    membership decide the routing) equals the fp32 value nearest to the exact
    dot product.  The oracle rounds its fp64 matmul to fp32; that fp64 sum is
    within (H-1) 2^-53 sum|x w| of the exact one, so the fp32 rounding can
    differ only where the fp64 value lies that close to a midpoint between
    two fp32 numbers: those logits are re-formed exactly in rationals
    (bf16 products are exact) and rounded to nearest, ties to even.  Adjacent
    top-(k+1) pairs within 2 fp32 ulp of each other are re-formed the same
    way whatever their distance from a midpoint."""
    from fractions import Fraction
    x_bits, wr_bits, _, k = S.router_inputs(name)
    x, wr = O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(wr_bits)
    H = x.shape[1]
    l64 = x @ wr.T
    l32 = O.router_logits(x_bits, wr_bits)
    S_abs = np.abs(x) @ np.abs(wr).T
    err64 = (H - 1) * 2.0 ** -53 * S_abs * 1.01
    top = np.argsort(-l32.astype(np.float64), axis=1, kind="stable")[:, :k + 1]
    ulp = lambda v: np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)  # noqa: E731
    # distance of the fp64 value from the nearest fp32 rounding boundary
    lo = np.nextafter(l32, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(l32, np.float32(np.inf)).astype(np.float64)
    c = l32.astype(np.float64)
    dist = np.minimum(np.abs(l64 - (c + lo) / 2), np.abs(l64 - (c + hi) / 2))
    redo = set()
    for t in range(l32.shape[0]):
        row = top[t]
        for e in row:
            if dist[t, e] <= err64[t, e]:
                redo.add((t, int(e)))
        vals = l32[t, row].astype(np.float64)
        for j in range(k):
            if vals[j] - vals[j + 1] <= 2 * ulp(vals[j]):
                redo.add((t, int(row[j])))
                redo.add((t, int(row[j + 1])))
    for t, e in sorted(redo):
        q = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], wr[e])), Fraction(0))
        assert _exact_f32(q) == l32[t, e], (name, t, e)
    print(f"{name}: {len(redo)} logits re-formed exactly")


def test_exact_f32_rounding_helper():
    """The helper's rounding against cases with a known answer: values on
    an fp32 number, just above and below a midpoint, and exactly on a
    midpoint (ties to even, both directions)."""
    from fractions import Fraction
    one = Fraction(1)
    u = Fraction(1, 2 ** 23)                                   # ulp of 1.0f
    assert _exact_f32(one) == np.float32(1.0)
    assert _exact_f32(one + u / 2) == np.float32(1.0)          # tie -> even (1.0)
    assert _exact_f32(one + u / 2 + Fraction(1, 2 ** 80)) == np.nextafter(np.float32(1), np.float32(2))
    assert _exact_f32(one + 3 * u / 2) == np.float32(1.0) + np.float32(2 * 2.0 ** -23)  # tie -> even (1 + 2u)
    assert _exact_f32(-(one + u / 2 - Fraction(1, 2 ** 80))) == np.float32(-1.0)


def test_router_bias_added_in_fp32():
    inp = S.make_small(6, 64, 8, 2, 64, seed=5, bias=True)
    plain = O.router_logits(inp.x, inp.w_router)
    biased = O.router_logits(inp.x, inp.w_router, inp.bias)
    assert biased.dtype == np.float32
    assert np.array_equal(biased, np.float32(plain) + inp.bias)


def brute_topk(lrow, k):
    """Brute force over all k-subsets: the chosen set maximises the logits
    lexicographically with ties to lower index; ordering by Python tuple sort."""
    E = len(lrow)
    best = None
    for sub in itertools.combinations(range(E), k):
        key = sorted(((-float(lrow[e]), e) for e in sub))
        if best is None or key < best:
            best = key
    return [e for _, e in best]


@pytest.mark.parametrize("E", [2, 3, 4, 5, 6])
def test_topk_bruteforce_all_tie_patterns(E):
    """Every logit vector over {0, 1, 2}^E (dense with ties), every k."""
    rows = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=E)), dtype=np.float32)
    for k in range(1, E + 1):
        ids = O.topk_lowest_index(rows, k)
        for r, row in enumerate(rows):
            assert ids[r].tolist() == brute_topk(row, k), (row, k)


def test_topk_selection_property_random():
    """For random fp32 logits with planted ties: chosen beats every unchosen
    (strictly, or equal with lower index), and chosen are best-first."""
    rng = np.random.default_rng(3)
    l = rng.integers(-20, 20, size=(500, 32)).astype(np.float32) / 8
    k = 5
    ids = O.topk_lowest_index(l, k)
    for t in range(l.shape[0]):
        chosen = ids[t].tolist()
        rest = set(range(32)) - set(chosen)
        for j, e in enumerate(chosen):
            for f in rest:
                assert l[t, e] > l[t, f] or (l[t, e] == l[t, f] and e < f)
            if j:
                p = chosen[j - 1]
                assert l[t, p] > l[t, e] or (l[t, p] == l[t, e] and p < e)


def test_zero_input_routes_to_first_k_with_equal_weights():
    for k in (2, 8):
        x = np.zeros((3, 64), dtype=np.uint16)
        wr = S.make_small(1, 64, 16, k, 64, seed=1).w_router
        ids, w, l = O.route(x, wr, k)
        assert (l == 0).all()
        np.testing.assert_array_equal(ids, np.tile(np.arange(k), (3, 1)))
        assert (w == 1.0 / k).all()          # exact: k is a power of two


def test_identical_router_rows_lower_index_wins():
    inp = S.make_small(16, 64, 8, 2, 64, seed=11)
    wr = inp.w_router.copy()
    wr[5] = wr[2]                       # experts 2 and 5 always tie
    l = O.router_logits(inp.x, wr)
    ids = O.topk_lowest_index(l, 8)     # all experts ordered
    for t in range(16):
        row = ids[t].tolist()
        assert row.index(2) < row.index(5)


def test_weights_sum_to_one_and_are_positive():
    for name in ("tiny", "q8"):
        inp = S.make(name)
        ids, w, l = O.route(inp.x, inp.w_router, inp.k, inp.bias)
        assert np.all(w > 0)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_k_equals_E_is_plain_softmax():
    inp = S.make("tiny")
    ids, w, l = O.route(inp.x, inp.w_router, inp.E)
    ref = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-13, atol=0)


def test_k_one_weight_is_one():
    inp = S.make("tiny")
    ids, w, l = O.route(inp.x, inp.w_router, 1)
    assert (w == 1.0).all()
    np.testing.assert_array_equal(ids[:, 0], np.argmax(l, axis=1))


def test_unrenormalised_hand_closed_form():
    """The variant without top-k renormalisation, by hand on the same inputs:
    token 0 softmax denominator Z = e^2 + 2e + e^(1/2); w = [e^2, e] / Z.
    y0 = [h0, -h0] with h0 = e/(e+1); y1 = [h1/2, h1/4] with h1 = -2/(1+e).
    token 1: four equal logits, w = [1/4, 1/4], out = 0."""
    inp = hand_inputs()
    out, r = O.forward_per_token(inp, exact_router=True, renorm=False)
    e = math.e
    Z = e * e + 2 * e + math.sqrt(e)
    w0, w1 = e * e / Z, e / Z
    np.testing.assert_array_equal(r["ids"], [[0, 1], [0, 1]])
    np.testing.assert_allclose(r["w"][0], [w0, w1], rtol=0, atol=1e-15)
    assert r["w"][1].tolist() == [0.25, 0.25]
    h0, h1 = e / (e + 1), -2 / (1 + e)
    np.testing.assert_allclose(out[0], [w0 * h0 + w1 * h1 / 2, -w0 * h0 + w1 * h1 / 4], rtol=0, atol=1e-15)
    assert out[1].tolist() == [0.0, 0.0]
    out_b, _ = O.forward_batched(inp, renorm=False)
    np.testing.assert_allclose(out_b, out, rtol=0, atol=1e-15)


def test_unrenormalised_weights_are_softmax_mass_of_the_chosen():
    """w_j = p[id_j] from scipy's softmax; the weights sum to 1 minus the mass
    of the experts not chosen; dividing by their sum gives the renormalised
    weights; k = E gives the whole softmax (sum 1)."""
    for name in ("tiny", "q8"):
        inp = S.make(name)
        ids, w, l = O.route(inp.x, inp.w_router, inp.k, inp.bias, renorm=False)
        ids_r, w_r, _ = O.route(inp.x, inp.w_router, inp.k, inp.bias)
        np.testing.assert_array_equal(ids, ids_r)
        p = scipy.special.softmax(l.astype(np.float64), axis=1)
        np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13, atol=0)
        rest = p.sum(axis=1) - np.take_along_axis(p, ids.astype(np.int64), 1).sum(axis=1)
        assert np.all(w.sum(axis=1) <= 1.0 + 1e-15)
        np.testing.assert_allclose(w.sum(axis=1), 1.0 - rest, rtol=0, atol=1e-13)
        np.testing.assert_allclose(w / w.sum(axis=1, keepdims=True), w_r, rtol=1e-13, atol=0)
    inp = S.make("tiny")
    ids, w, l = O.route(inp.x, inp.w_router, inp.E, renorm=False)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- bucketing
def check_bucketing(ids, E):
    T, k = ids.shape
    counts, offsets, perm, pos = O.permute(ids, E)
    flat = ids.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k
    np.testing.assert_array_equal(offsets[1:], np.cumsum(counts))
    assert offsets[0] == 0 and offsets[E] == T * k
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    assert sorted(perm.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(pos[perm], np.arange(T * k))
    tok = perm // k
    assert np.array_equal(np.bincount(tok, minlength=T), np.full(T, k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    return counts, offsets, perm, pos


def test_bucketing_random_and_adversarial():
    rng = np.random.default_rng(0)
    E, k = 16, 4
    for T in (1, 3, 17, 64):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        check_bucketing(ids, E)
    # every token on the same k experts; most experts empty
    check_bucketing(np.tile(np.array([9, 3, 12, 0], dtype=np.int32), (33, 1)), E)


def test_bucketing_zero_input_closed_form():
    """X = 0 routes every token to experts 0..k-1 in that order, so
    perm[e*T + t] = t*k + e for e < k."""
    T, E, k = 12, 16, 2
    x = np.zeros((T, 64), dtype=np.uint16)
    wr = S.make_small(1, 64, E, k, 64, seed=1).w_router
    ids, _, _ = O.route(x, wr, k)
    counts, offsets, perm, pos = check_bucketing(ids, E)
    for e in range(k):
        for t in range(T):
            assert perm[e * T + t] == t * k + e


def test_bucketing_tiny_and_q8():
    for name in ("tiny", "q8"):
        inp = S.make(name)
        ids, _, _ = O.route(inp.x, inp.w_router, inp.k)
        check_bucketing(ids, inp.E)


# ---------------------------------------------------------------- experts
def test_single_expert_reduces_to_swiglu_mlp():
    """E = k = 1: the block is one SwiGLU MLP with weight 1 (torch fp64 silu)."""
    inp = S.make_small(7, 64, 1, 1, 32, seed=4)
    out, r = O.forward_per_token(inp)
    assert (r["w"] == 1.0).all()
    x = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    gu = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up[0]))
    wd = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down[0]))
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(x, gu[:32])) * torch.nn.functional.linear(x, gu[32:]),
        wd)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-15)


def test_down_weights_scale_output_exactly():
    """Doubling W_down doubles the output exactly (fp64, power of two)."""
    inp = S.make("tiny")
    out, _ = O.forward_per_token(inp)
    W = O.ExpertWeights(inp)
    for e in range(inp.E):
        wg, wu, wd = W.get(e)
        W._cache[e] = (wg, wu, 2.0 * wd)
    out2, _ = O.forward_per_token(inp, W)
    assert np.array_equal(out2, 2.0 * out)


def dense_masked_reference(inp):
    """Every expert on every token (torch fp64), masked by torch.topk of the
    logits and weighted by the softmax renormalised over the mask."""
    l = torch.from_numpy(O.router_logits(inp.x, inp.w_router, inp.bias).astype(np.float64))
    top = torch.topk(l, inp.k, dim=1).indices
    mask = torch.zeros_like(l).scatter_(1, top, 1.0)
    p = torch.softmax(l, dim=1) * mask
    g = p / p.sum(dim=1, keepdim=True)
    x = torch.from_numpy(O.bf16_bits_to_f64(inp.x))
    out = torch.zeros(inp.T, inp.H, dtype=torch.float64)
    for e in range(inp.E):
        gu = torch.from_numpy(O.bf16_bits_to_f64(inp.w_gate_up[e]))
        wd = torch.from_numpy(O.bf16_bits_to_f64(inp.w_down[e]))
        h = torch.nn.functional.silu(x @ gu[: inp.I].T) * (x @ gu[inp.I:].T)
        out += g[:, e:e + 1] * (h @ wd.T)
    return out.numpy()


@pytest.mark.parametrize("name", ["tiny", "tiny_bias"])
def test_per_token_loop_matches_dense_masked_formulation(name):
    inp = S.make("tiny") if name == "tiny" else S.make_small(8, 256, 16, 2, 128, seed=21, bias=True)
    out, _ = O.forward_per_token(inp)
    ref = dense_masked_reference(inp)
    assert np.abs(out - ref).max() <= 1e-12 * O.rms(ref)


@pytest.mark.parametrize("name", ["tiny", "q8"])
def test_batched_matches_per_token(name):
    inp = S.make(name)
    W = O.ExpertWeights(inp)
    a, _ = O.forward_per_token(inp, W)
    b, rb = O.forward_batched(inp, W)
    assert np.abs(a - b).max() <= 1e-12 * O.rms(a)
    check_bucketing(rb["ids"], inp.E)


def test_nf4_batched_matches_per_token_small():
    inp = S.make_small(5, 128, 8, 2, 64, seed=9, wfmt="nf4")
    W = O.ExpertWeights(inp)
    a, _ = O.forward_per_token(inp, W)
    b, _ = O.forward_batched(inp, W)
    assert np.abs(a - b).max() <= 1e-12 * O.rms(a)


def test_oracle_reproduces_golden_tiny():
    """Regression pin: the committed fixture (written by
    tests/golden/make_golden.py from the oracle alone) still matches."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    g = json.load(open(path))
    inp = S.make("tiny")
    out, r = O.forward_per_token(inp, exact_router=True)
    counts, offsets, perm, _ = O.permute(r["ids"], inp.E)
    assert r["ids"].tolist() == g["ids"]
    assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"] and perm.tolist() == g["perm"]
    np.testing.assert_allclose(r["w"], g["weights"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(out[0, :16], g["out_first_row_first_16"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(out.sum(axis=1), g["out_row_sums"], rtol=1e-12, atol=1e-15)


def test_oracle_reproduces_golden_variants():
    """Regression pin for the variants (written by tests/golden/make_golden.py
    from the oracle alone): weights without renormalisation, LoRA adapters,
    the pre-block step."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_variants.json")))
    inp = S.make("tiny")
    out_s, rs = O.forward_per_token(inp, exact_router=True, renorm=False)
    np.testing.assert_allclose(rs["w"], g["softmax_weights"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(out_s.sum(axis=1), g["softmax_out_row_sums"], rtol=1e-12, atol=1e-15)
    lora = O.LoRA(**S.lora_adapters(inp.E, inp.H, inp.I))
    out_l, _ = O.forward_per_token(inp, exact_router=True, lora=lora)
    np.testing.assert_allclose(out_l[0, :16], g["lora_out_first_row_first_16"], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(out_l.sum(axis=1), g["lora_out_row_sums"], rtol=1e-12, atol=1e-15)
    p = S.prenorm_inputs(8, 256)
    r_bits, x64 = O.residual_rmsnorm(p["residual"], p["delta"], p["gamma"], p["eps"])
    assert r_bits[0, :16].tolist() == g["prenorm_r_bits_row0_first_16"]
    assert O.f64_to_bf16_rne(x64)[0, :16].tolist() == g["prenorm_x_bits_row0_first_16"]
    np.testing.assert_allclose(x64.sum(axis=1), g["prenorm_x_row_sums"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose((x64 * x64).sum(axis=1), g["prenorm_x_row_sumsq"], rtol=1e-13, atol=0)
