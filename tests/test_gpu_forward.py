"""Whole-block parity (HIP vs fp64 oracle): routing arrays in the workspace
bit-exact, outputs within max|err| <= 2e-2 * rms (bf16 weights) or
5e-2 * rms (4-bit weights, oracle on the same dequantised weights)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from mixture_experts_decode_router_amd.layer import MoELayer
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_forward, oracle_weights, rel_err, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q8": ("q64", 64), "q64": ("q64", 64), "q48q": ("q48q", 64),
            "q4096": ("q4096", 4096)}


def run_forward(lay, x_bits):
    x = lay.upload_x(x_bits)
    out = lay.forward(x)
    torch.cuda.synchronize()
    return out, lay.views(x_bits.shape[0])


def check_views(views, ref):
    assert np.array_equal(views["ids"].cpu().numpy(), ref["ids"])
    assert np.array_equal(views["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(views["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(views["perm"].cpu().numpy(), ref["perm"])
    assert np.array_equal(views["pos"].cpu().numpy(), ref["pos"])
    np.testing.assert_allclose(views["w"].cpu().numpy(), ref["w"], rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("name", ["tiny", "q8", "q64", "q48q", "q4096"])
def test_forward_matches_oracle(name):
    inp = workload(name)
    lay = layer(*LAYER_OF[name])
    say(f"[gpu] forward {name} T={inp.T} wfmt={inp.wfmt}")
    out, views = run_forward(lay, inp.x)
    ref_out, ref = oracle_forward(name)
    check_views(views, ref)
    err = rel_err(out.cpu().numpy(), ref_out)
    tol = TOL_NF4 if inp.wfmt == "nf4" else TOL_BF16
    say(f"[gpu]   max|err|/rms = {err:.3e} (tolerance {tol})")
    assert err <= tol


@pytest.mark.parametrize("name", ["q64", "q48q"])
def test_forward_row_major_weights(name):
    """Same parity with the expert weights left row-major (no packing)."""
    inp = workload(name)
    lay = layer(name, 64, tiled=False)
    say(f"[gpu] forward {name} row-major weights")
    out, views = run_forward(lay, inp.x)
    ref_out, ref = oracle_forward(name)
    check_views(views, ref)
    tol = TOL_NF4 if inp.wfmt == "nf4" else TOL_BF16
    assert rel_err(out.cpu().numpy(), ref_out) <= tol
    tiled = layer(name, 64).forward(layer(name, 64).upload_x(inp.x))
    assert torch.equal(out, tiled)   # same arithmetic, only the weight layout differs


@pytest.mark.parametrize("T", list(S.SWEEP_T))
def test_forward_decode_sweep(T):
    inp = workload("q64", T)
    say(f"[gpu] forward sweep T={T}")
    out, views = run_forward(layer("q64", 64), inp.x)
    ref_out, ref = oracle_forward("q64", T)
    check_views(views, ref)
    assert rel_err(out.cpu().numpy(), ref_out) <= TOL_BF16


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_forward_decode_sweep_4bit(T):
    """4-bit Qwen layer at decode sizes: the down kernel's grid of (E + T k /
    16) x 16 workgroups stays within the small-grid bound (1024) up to T = 7,
    so T = 1 and 4 take its three-block iterations; T = 8, 16 (and q48q) the
    one-block form."""
    inp = workload("q48q", T)
    say(f"[gpu] forward 4-bit sweep T={T}")
    out, views = run_forward(layer("q48q", 64), inp.x)
    ref_out, ref = oracle_forward("q48q", T)
    check_views(views, ref)
    assert rel_err(out.cpu().numpy(), ref_out) <= TOL_NF4


@pytest.mark.parametrize("tiled", [True, False])
@pytest.mark.parametrize("case", [
    dict(T=1, H=256, E=16, k=2, I=128, wfmt="bf16"),
    dict(T=17, H=256, E=16, k=16, I=128, wfmt="bf16"),     # k = E: every expert
    dict(T=33, H=512, E=32, k=1, I=256, wfmt="bf16"),      # k = 1
    dict(T=40, H=4096, E=16, k=4, I=384, wfmt="bf16"),     # longest rows
    dict(T=50, H=1024, E=32, k=4, I=2560, wfmt="bf16"),    # long intermediate
    dict(T=37, H=384, E=32, k=4, I=256, wfmt="nf4"),       # H an odd number of 128-blocks
    dict(T=21, H=4096, E=16, k=3, I=2560, wfmt="nf4"),
    dict(T=300, H=256, E=16, k=2, I=128, wfmt="bf16"),     # many rows per expert (several items)
    dict(T=24, H=512, E=256, k=8, I=128, wfmt="bf16"),     # largest expert count
    dict(T=9, H=256, E=48, k=6, I=128, wfmt="bf16"),       # E not a multiple of 64
    dict(T=13, H=512, E=256, k=16, I=256, wfmt="nf4"),     # largest E and k, 4-bit
    dict(T=4, H=256, E=16, k=16, I=128, wfmt="bf16"),      # small batch bucketed by the router: 64 slots
    dict(T=3, H=512, E=256, k=8, I=128, wfmt="bf16"),      # ... with the largest expert count
    dict(T=7, H=256, E=48, k=6, I=128, wfmt="bf16"),       # ... eight-wave select, E not a multiple of 64
    dict(T=11, H=256, E=16, k=3, I=128, wfmt="bf16"),     # direct form, 33 slots (ragged scan tail)
    dict(T=64, H=256, E=16, k=16, I=128, wfmt="bf16"),    # 1024 slots: the direct form's largest (row-major)
    dict(T=29, H=512, E=16, k=2, I=256, wfmt="nf4", cb="random"),  # codebook of arbitrary fp32 values
    dict(T=6, H=256, E=16, k=4, I=384, wfmt="nf4", cb="random"),   # ... small grid (three-block down)
])
def test_forward_edge_shapes(case, tiled):
    book = S.random_codebook(case["T"]) if case.get("cb") == "random" else None
    inp = S.make_small(case["T"], case["H"], case["E"], case["k"], case["I"], seed=case["T"],
                       wfmt=case["wfmt"], bias=case["k"] == 4, codebook=book)
    say(f"[gpu] forward edge {case} tiled={tiled}")
    lay = MoELayer(inp, t_max=case["T"], tiled=tiled)
    out, views = run_forward(lay, inp.x)
    ref_out, ref = O.forward_batched(inp)
    check_views(views, ref)
    tol = TOL_NF4 if case["wfmt"] == "nf4" else TOL_BF16
    err = rel_err(out.cpu().numpy(), ref_out)
    say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("case", [
    dict(T=600, H=384, E=16, k=2, I=256),     # down: last 256-row weight tile half past H
    dict(T=1100, H=512, E=16, k=1, I=384),    # k = 1, three gate/up tiles
    dict(T=520, H=256, E=16, k=4, I=128),     # shortest K (down K = 128: two stages)
    dict(T=640, H=256, E=256, k=16, I=128),   # largest E and k on the MFMA kernels
    dict(T=600, H=384, E=16, k=2, I=256, wfmt="nf4"),    # 4-bit: H an odd number of 128-blocks
    dict(T=520, H=256, E=16, k=4, I=128, wfmt="nf4"),    # 4-bit: shortest K
    dict(T=640, H=256, E=256, k=16, I=128, wfmt="nf4"),  # 4-bit: largest E and k
    dict(T=700, H=512, E=32, k=2, I=384, wfmt="nf4", cb="random"),  # 4-bit: arbitrary fp32 codebook
])
def test_forward_prefill_mfma_shapes(case):
    """Shapes that take the LDS-tiled MFMA kernels (>= 32 routed rows per expert)."""
    wfmt = case.get("wfmt", "bf16")
    book = S.random_codebook(case["T"]) if case.get("cb") == "random" else None
    inp = S.make_small(case["T"], case["H"], case["E"], case["k"], case["I"], seed=case["T"],
                       wfmt=wfmt, bias=True, codebook=book)
    say(f"[gpu] forward prefill-path {case}")
    lay = MoELayer(inp, t_max=case["T"])
    out, views = run_forward(lay, inp.x)
    ref_out, ref = O.forward_batched(inp)
    check_views(views, ref)
    err = rel_err(out.cpu().numpy(), ref_out)
    say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= (TOL_NF4 if wfmt == "nf4" else TOL_BF16)


def test_forward_prefill_one_hot_expert_set():
    """Every token identical: k experts get all T rows (many 128-row items each)."""
    inp = S.make_small(700, 256, 16, 2, 128, seed=7, wfmt="bf16", bias=False)
    inp.x[:] = inp.x[3]
    say("[gpu] forward prefill-path, all rows identical")
    lay = MoELayer(inp, t_max=700)
    out, views = run_forward(lay, inp.x)
    ref_out, ref = O.forward_batched(inp)
    check_views(views, ref)
    assert (views["counts"].cpu().numpy() > 0).sum() == 2
    assert rel_err(out.cpu().numpy(), ref_out) <= TOL_BF16
    o = out.cpu()
    assert torch.equal(o, o[:1].expand_as(o))   # identical rows give identical bits


def test_forward_zero_input_gives_zero():
    inp = workload("q64")
    lay = layer("q64", 64)
    say("[gpu] forward zero input")
    out, views = run_forward(lay, np.zeros((7, inp.H), dtype=np.uint16))
    assert torch.count_nonzero(out) == 0
    assert (views["ids"].cpu().numpy() == np.arange(inp.k)).all()


def test_forward_deterministic_and_row_independent():
    inp = workload("q64")
    lay = layer("q64", 64)
    say("[gpu] forward determinism / row permutation")
    x = lay.upload_x(inp.x)
    a = lay.forward(x).clone()
    for _ in range(5):
        assert torch.equal(lay.forward(x), a)
    rng = np.random.default_rng(4)
    p = rng.permutation(inp.T)
    b = lay.forward(lay.upload_x(inp.x[p]))
    assert torch.equal(b, a[torch.from_numpy(p).cuda()])


def test_prefill_rows_match_decode_rows_bit_for_bit():
    """T=4096 runs the LDS-tiled MFMA kernels, T=16 the skinny ones: the same
    token gets the same bits either way."""
    inp = workload("q4096")
    lay = layer("q4096", 4096)
    say("[gpu] prefill vs decode path rows")
    a = lay.forward(lay.upload_x(inp.x))
    for lo in (0, 2000, 4080):
        b = lay.forward(lay.upload_x(inp.x[lo:lo + 16]))
        assert torch.equal(a[lo:lo + 16], b), lo


def test_prefill_rows_match_decode_rows_4bit():
    """4-bit Qwen layer at T=1024 (the LDS-tiled 4-bit MFMA kernels) against
    the same tokens in batches of 16 (the 16-row 4-bit kernels): the same
    bits, and parity with the oracle on sampled rows."""
    inp = S.make("q48q", 1024)
    lay = MoELayer(inp, t_max=1024)
    say("[gpu] 4-bit prefill vs decode path rows")
    a = lay.forward(lay.upload_x(inp.x))
    for lo in (0, 500, 1008):
        b = lay.forward(lay.upload_x(inp.x[lo:lo + 16]))
        assert torch.equal(a[lo:lo + 16], b), lo
    rows = np.array([0, 1, 333, 777, 1023])
    sub = dataclasses.replace(inp, x=inp.x[rows], T=len(rows))
    ref_out, _ = O.forward_batched(sub, oracle_weights("q48q"))
    err = rel_err(a.cpu().numpy()[rows], ref_out)
    say(f"[gpu]   sampled rows max|err|/rms = {err:.3e}")
    assert err <= TOL_NF4


def test_forward_row_subset_is_bit_identical():
    """A token's output does not depend on which other tokens share the batch."""
    inp = workload("q64")
    lay = layer("q64", 64)
    a = lay.forward(lay.upload_x(inp.x))
    b = lay.forward(lay.upload_x(inp.x[:13]))
    assert torch.equal(a[:13], b)
    c = lay.forward(lay.upload_x(inp.x[40:41]))
    assert torch.equal(a[40:41], c)


@pytest.mark.parametrize("tiled", [True, False])
def test_direct_form_many_rows_per_expert(tiled):
    """Direct form (2E <= T k <= 1024 slots, no work list): every token
    identical, so k experts get all 40 rows (a two-block pass, then a
    one-block pass).  Parity with the oracle, routing arrays as the bucketing
    kernel writes them, and each row bit-identical to the same token alone
    (T = 1 runs the work-list kernels)."""
    inp = S.make_small(40, 256, 32, 8, 256, seed=11, wfmt="bf16", bias=True)
    inp.x[:] = inp.x[5]
    say(f"[gpu] direct form, 40 identical rows tiled={tiled}")
    lay = MoELayer(inp, t_max=40, tiled=tiled)
    out, views = run_forward(lay, inp.x)
    ref_out, ref = O.forward_batched(inp)
    check_views(views, ref)
    assert (views["counts"].cpu().numpy() == 40).sum() == 8
    assert rel_err(out.cpu().numpy(), ref_out) <= TOL_BF16
    one = lay.forward(lay.upload_x(inp.x[:1]))
    assert torch.equal(out, one.expand_as(out))
