"""Router parity (HIP vs fp64 oracle): top-k ids bit-exact, weights within
fp32 rounding, every logit within the error bound the kernel's selection
relies on, and near-ties that only an exact re-formation can order."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from mixture_experts_decode_router_amd.layer import MoELayer
from tests.gpu_util import layer, say, topk_gap_audit, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q8": ("q64", 64), "q64": ("q64", 64), "q48q": ("q48q", 64),
            "q4096": ("q4096", 4096)}


def route_bound(x_bits, wr_bits, bias):
    """The selection's error bound on each approximate logit, from the exact
    sum S = sum_h |x w| (fp64) and the chain depth of the kernel's fp32
    sums: 32 additions inside one MFMA, one per 32-k step of a K split, the
    ks split partials (ks: the largest power of two <= 16 with H a multiple
    of 256 ks), 8 more, doubled, times 2^-24; plus 2.5e-7 (|l| + |bias|) for
    the fp32 rounding of the logit and of the bias addition."""
    H = x_bits.shape[1]
    ks = 1
    while ks * 2 <= 16 and H % (ks * 2 * 256) == 0:
        ks *= 2
    gamma = 2.0 * (32 + (H // ks) // 32 + ks + 8) * 2.0 ** -24
    x, wr = O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(wr_bits)
    S_abs = np.abs(x) @ np.abs(wr).T
    l_dot = O.router_logits(x_bits, wr_bits).astype(np.float64)
    b = 0.0 if bias is None else np.abs(np.asarray(bias, np.float64))[None, :]
    return gamma * S_abs + 2.5e-7 * (np.abs(l_dot) + b)


def check_route(lay, inp, x_bits=None):
    x_bits = inp.x if x_bits is None else x_bits
    T = x_bits.shape[0]
    x = lay.upload_x(x_bits)
    ids, w, lg = lay.route(x, T, with_logits=True)
    torch.cuda.synchronize()
    ids, w, lg = ids.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()
    ids_o, w_o, l_o = O.route(x_bits, inp.w_router, inp.k, inp.bias)
    mism = np.nonzero((ids != ids_o).any(axis=1))[0]
    assert mism.size == 0, f"ids differ on tokens {mism[:10]}: gpu {ids[mism[:3]]} oracle {ids_o[mism[:3]]}"
    np.testing.assert_allclose(w, w_o, rtol=2e-5, atol=1e-6)
    # every logit (approximate, or re-formed and rounded where the bound
    # left the choice open) lies within the bound the selection takes for it
    beta = route_bound(x_bits, inp.w_router, inp.bias)
    err = np.abs(lg.astype(np.float64) - l_o.astype(np.float64))
    ratio = float((err / beta).max())
    say(f"[gpu]   max |logit - oracle fp32 logit| / bound = {ratio:.3e}")
    assert np.all(err <= beta), np.unravel_index(np.argmax(err / beta), err.shape)
    return ids, w, lg, l_o


@pytest.mark.parametrize("name", ["tiny", "q8", "q64", "q48q", "q4096"])
def test_route_matches_oracle(name):
    inp = workload(name)
    lay = layer(*LAYER_OF[name])
    if name == "q4096":
        # the q4096 layer carries the router bias
        assert inp.bias is not None
    say(f"[gpu] route {name} T={inp.T}")
    ids, w, lg, l_o = check_route(lay, inp)
    say(f"[gpu]   min top-{inp.k + 1} gap {topk_gap_audit(l_o, inp.k):.3e}, "
        f"max|logit err| {np.abs(lg - l_o).max():.3e}")


@pytest.mark.parametrize("T", [1, 3, 16, 17, 33, 64])
def test_route_ragged_tiles(T):
    inp = workload("tiny", T)
    say(f"[gpu] route tiny T={T}")
    check_route(layer("tiny", 64), inp)


def test_route_zero_input_ties_to_lowest_indices():
    inp = workload("q64")
    lay = layer("q64", 64)
    x = np.zeros((5, inp.H), dtype=np.uint16)
    say("[gpu] route zero input")
    ids, w, lg, _ = check_route(lay, inp, x)
    assert (ids == np.arange(inp.k)).all()
    assert (w == np.float32(1.0 / inp.k)).all()
    assert (lg == 0).all()


def test_route_duplicate_router_rows_lower_index_first():
    base = S.make_small(40, 512, 16, 16, 128, seed=77)
    wr = base.w_router.copy()
    wr[9] = wr[3]
    wr[14] = wr[3]
    inp = S.MoEInputs("dup", base.T, base.H, base.E, base.k, base.I, "bf16", base.x, wr, None,
                      base.w_gate_up, base.w_down)
    lay = MoELayer(inp, t_max=64)
    say("[gpu] route duplicate rows (k = E)")
    ids, _, _, _ = check_route(lay, inp)
    for row in ids.tolist():
        assert row.index(3) < row.index(9) < row.index(14)


def test_route_near_tie_decided_by_reformation():
    """Two router rows equal except for one element, one bf16 step apart:
    their logits differ by |x[h0]| times that step, far below the bound, so
    only the exact re-formation can order them (k = E puts both among the
    chosen of every token).  Tokens with x[h0] of either sign give both
    orders; tokens with x[h0] = 0 tie exactly and the lower index wins."""
    base = S.make_small(48, 512, 16, 16, 128, seed=78)
    wr = base.w_router.copy()
    h0 = 100
    wr[4, h0] = 0x3980                    # 2^-12
    wr[11] = wr[4]
    wr[11, h0] = 0x3981                   # the next bf16 number: 2^-12 + 2^-19
    x = base.x.copy()
    x[:8, h0] = 0                         # exact ties on the first tokens
    sign = np.random.default_rng(3).integers(0, 2, size=40)
    x[8:, h0] = np.where(sign == 1, 0x3F80, 0xBF80)   # +-1: the logits differ by +-2^-19
    inp = S.MoEInputs("near_tie", base.T, base.H, base.E, base.k, base.I, "bf16", x, wr, None,
                      base.w_gate_up, base.w_down)
    _, _, l_o = O.route(x, wr, inp.k)
    d = l_o[:, 11].astype(np.float64) - l_o[:, 4]
    beta = route_bound(x, wr, None)
    assert np.all(np.abs(d) < beta[:, 4])          # inside the bound: undecidable without re-forming
    assert (d > 0).sum() >= 5 and (d < 0).sum() >= 5 and (d == 0).sum() >= 8
    lay = MoELayer(inp, t_max=64)
    say("[gpu] route near-tie rows")
    ids, _, _, _ = check_route(lay, inp)
    for t, row in enumerate(ids.tolist()):
        first = 11 if d[t] > 0 else 4
        assert row.index(first) < row.index(15 - first)


@pytest.mark.parametrize("shape", [
    dict(T=70, H=512, E=256, k=16, I=128),    # E = 256, k = 16
    dict(T=20, H=4096, E=64, k=6, I=128),     # long rows (8 chunks per lane)
    dict(T=9, H=128, E=16, k=1, I=128),       # k = 1, shortest rows
])
def test_route_other_shapes(shape):
    inp = S.make_small(shape["T"], shape["H"], shape["E"], shape["k"], shape["I"], seed=5, bias=True)
    say(f"[gpu] route shape {shape}")
    check_route(MoELayer(inp, t_max=shape["T"]), inp)


def test_route_is_deterministic():
    inp = workload("q64")
    lay = layer("q64", 64)
    x = lay.upload_x(inp.x)
    a = [t.clone() for t in lay.route(x, with_logits=True)]
    for _ in range(3):
        b = lay.route(x, with_logits=True)
        for u, v in zip(a, b):
            assert torch.equal(u, v)


def test_route_large_batch_equals_small_batches_bit_for_bit():
    """At T=4096 one workgroup sums all K splits itself; at T=64 the splits are
    stored and summed by the selection kernel.  Same split-order sums, so the
    same ids, weights and logits, bit for bit."""
    inp = workload("q4096")
    lay = layer("q4096", 4096)
    say("[gpu] route T=4096 vs 64-token slices")
    ids, w, lg = lay.route(lay.upload_x(inp.x), with_logits=True)
    for lo in (0, 1984, 4032):
        ids_s, w_s, lg_s = lay.route(lay.upload_x(inp.x[lo:lo + 64]), with_logits=True)
        assert torch.equal(ids[lo:lo + 64], ids_s), lo
        assert torch.equal(w[lo:lo + 64], w_s), lo
        assert torch.equal(lg[lo:lo + 64], lg_s), lo
