"""Router parity (HIP vs fp64 oracle): top-k ids bit-exact, weights within
fp32 rounding, chosen logits equal to the oracle's fp32 logits."""
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
    # every logit is within the proven bound of the exact fp32 logit (the
    # bound is ~1e-3 of |logit| scale here; typical errors are ~1e-6)
    assert np.abs(lg.astype(np.float64) - l_o).max() <= 1e-3 * max(1.0, np.abs(l_o).max())
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
