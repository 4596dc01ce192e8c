"""LoRA adapters fused into the decode expert GEMMs, against the fp64 oracle
with the same adapters: routing bit-exact, outputs within the bf16 / 4-bit
tolerances; zero B gives the base block's bits; graph replays equal eager;
at prefill sizes the MFMA kernels add the adapter terms with the same
arithmetic as the 16-row kernels, so rows do not depend on the batch."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from mixture_experts_decode_router_amd import _lib as L
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_weights, rel_err, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q8": ("q64", 64), "q64": ("q64", 64), "q48q": ("q48q", 64)}


def adapters(inp, seed=None):
    return S.lora_adapters(inp.E, inp.H, inp.I, seed=seed)


def check_views(views, ref):
    for k in ("ids", "counts", "offsets", "perm", "pos"):
        assert np.array_equal(views[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("name,T,tiled", [("tiny", 8, True), ("tiny", 33, False), ("q8", None, True),
                                          ("q64", None, True), ("q64", None, False), ("q48q", None, True),
                                          ("q48q", 20, False)])
def test_lora_forward_matches_oracle(name, T, tiled):
    inp = workload(name, T)
    d = adapters(inp)
    lay = layer(*LAYER_OF[name], tiled=tiled).with_lora(d)
    say(f"[gpu] LoRA forward {name} T={inp.T} tiled={tiled}")
    out = lay.forward(lay.upload_x(inp.x))
    torch.cuda.synchronize()
    base = "q64" if name in ("q8", "q64") else name
    ref_out, ref = O.forward_batched(inp, oracle_weights(base), lora=O.LoRA(**d))
    check_views(lay.views(inp.T), ref)
    err = rel_err(out.cpu().numpy(), ref_out)
    tol = TOL_NF4 if inp.wfmt == "nf4" else TOL_BF16
    base_out, _ = O.forward_batched(inp, oracle_weights(base), routing=ref)
    say(f"[gpu]   max|err|/rms = {err:.3e} (tolerance {tol}); LoRA moves out by "
        f"{O.rms(ref_out - base_out) / O.rms(ref_out):.2f} rms")
    assert err <= tol


@pytest.mark.parametrize("name", ["q64", "q48q"])
def test_lora_zero_b_equals_base_block(name):
    inp = workload(name)
    d = adapters(inp)
    d["b_gate_up"][:] = 0
    d["b_down"][:] = 0
    base = layer(*LAYER_OF[name])
    lay = base.with_lora(d)
    x = base.upload_x(inp.x)
    a = base.forward(x)
    b = lay.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_lora_rows_do_not_depend_on_the_batch():
    inp = workload("q64")
    lay = layer("q64", 64).with_lora(adapters(inp))
    a = lay.forward(lay.upload_x(inp.x))
    b = lay.forward(lay.upload_x(inp.x[:13]))
    torch.cuda.synchronize()
    assert torch.equal(a[:13], b)


def test_lora_graph_replay_equals_eager():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_lora(adapters(inp))
    stream = torch.cuda.Stream()
    x_s = torch.zeros(64, inp.H, dtype=torch.int16, device="cuda")
    out_s = torch.zeros(64, inp.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    lay.capture([8, 64], x_s, out_s, stream)
    try:
        for T in (64, 5):
            x = lay.upload_x(inp.x[:T])
            with torch.cuda.stream(stream):
                out_s.fill_(3.0)
                x_s[:T].copy_(x)
                lay.replay(T, stream)
                eager = lay.forward(x.clone(), stream=stream)
            stream.synchronize()
            assert torch.equal(out_s[:T], eager), T
            assert bool((out_s[T:] == 3.0).all()), T
    finally:
        lay.release_graph()


def test_lora_graph_replay_at_prefill_size_equals_eager():
    inp = workload("tiny", 256)
    lay = layer("tiny", 256).with_lora(adapters(inp))
    stream = torch.cuda.Stream()
    x_s = torch.zeros(256, inp.H, dtype=torch.int16, device="cuda")
    out_s = torch.zeros(256, inp.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    lay.capture([16, 256], x_s, out_s, stream)
    try:
        for T in (256, 200, 9):
            x = lay.upload_x(inp.x[:T])
            for _ in range(2):
                with torch.cuda.stream(stream):
                    out_s.fill_(3.0)
                    x_s[:T].copy_(x)
                    lay.replay(T, stream)
                    eager = lay.forward(x.clone(), stream=stream)
                stream.synchronize()
                assert torch.equal(out_s[:T], eager), T
                assert bool((out_s[T:] == 3.0).all()), T
    finally:
        lay.release_graph()


@pytest.mark.parametrize("T", [256, 1024])
def test_lora_at_prefill_sizes(T):
    # T*k >= 32*E: the MFMA prefill kernels run, adding the adapter terms in
    # their epilogues (several 128-row items per expert at T = 1024), against
    # the oracle; each row is the same bits as a decode-sized call's (16-row
    # kernels); zero B gives the base MFMA kernels' bits
    inp = workload("tiny", T)
    d = adapters(inp)
    base = layer("tiny", 1024)
    say(f"[gpu] LoRA forward tiny at prefill size T={inp.T}")
    lay = base.with_lora(d)
    x = lay.upload_x(inp.x)
    out = lay.forward(x)
    torch.cuda.synchronize()
    ref_out, ref = O.forward_batched(inp, oracle_weights("tiny"), lora=O.LoRA(**d))
    check_views(lay.views(inp.T), ref)
    err = rel_err(out.cpu().numpy(), ref_out)
    say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= TOL_BF16
    small = lay.forward(lay.upload_x(inp.x[:16]))
    torch.cuda.synchronize()
    assert torch.equal(small, out[:16])
    d0 = adapters(inp)
    d0["b_gate_up"][:] = 0
    d0["b_down"][:] = 0
    xb = base.upload_x(inp.x)
    a = base.forward(xb)
    b = base.with_lora(d0).forward(xb)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("T", [600, 1100])
def test_lora_at_prefill_sizes_4bit(T):
    # 4-bit base at T*k >= 32*E: the 4-bit LDS-tiled MFMA kernels add the
    # adapter terms in their epilogues, against the oracle on the dequantised
    # weights; rows equal a decode-sized call's (the 16-row 4-bit kernels);
    # zero B gives the base kernels' bits
    from mixture_experts_decode_router_amd.layer import MoELayer
    inp = S.make_small(T, 384, 16, 2, 256, seed=T + 1, wfmt="nf4", bias=True)
    d = S.lora_adapters(inp.E, inp.H, inp.I, seed=T)
    base = MoELayer(inp, t_max=T)
    say(f"[gpu] LoRA forward 4-bit at prefill size T={T}")
    lay = base.with_lora(d)
    out = lay.forward(lay.upload_x(inp.x))
    torch.cuda.synchronize()
    ref_out, ref = O.forward_batched(inp, lora=O.LoRA(**d))
    check_views(lay.views(T), ref)
    err = rel_err(out.cpu().numpy(), ref_out)
    say(f"[gpu]   max|err|/rms = {err:.3e}")
    assert err <= TOL_NF4
    small = lay.forward(lay.upload_x(inp.x[:16]))
    torch.cuda.synchronize()
    assert torch.equal(small, out[:16])
    d0 = S.lora_adapters(inp.E, inp.H, inp.I, seed=T)
    d0["b_gate_up"][:] = 0
    d0["b_down"][:] = 0
    xb = base.upload_x(inp.x)
    a = base.forward(xb)
    b = base.with_lora(d0).forward(xb)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
