"""Backward of the block (frozen weights, the forward's routing) against the
fp64 oracle's chain rule: input and routing-weight gradients within the bf16
tolerance; the same bits on every run and whatever the batch; the
unsupported configurations refused.  A training forward (train=1) keeps the
gate/up pre-activations; its outputs are the same bits as a plain forward's."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from mixture_experts_decode_router_amd import _lib as L
from mixture_experts_decode_router_amd.layer import MoELayer
from tests.gpu_util import TOL_BF16, layer, oracle_weights, say, workload

pytestmark = pytest.mark.gpu

LAYER_OF = {"tiny": ("tiny", 64), "q8": ("q64", 64), "q64": ("q64", 64)}


def d_out_for(T, H, seed=17):
    return np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32)


def gpu_backward(lay, x_bits, d_out):
    x = lay.upload_x(x_bits)
    lay.forward(x)
    d_x, d_w = lay.backward(x, torch.from_numpy(d_out).cuda())
    torch.cuda.synchronize()
    return d_x.cpu().numpy(), d_w.cpu().numpy()


def rel(a, ref):
    return float(np.abs(np.asarray(a, np.float64) - ref).max() / np.sqrt(np.mean(ref * ref)))


@pytest.mark.parametrize("name,T", [("tiny", 8), ("tiny", 33), ("q8", None), ("q64", 24)])
def test_backward_matches_oracle(name, T):
    inp = workload(name, T)
    lay = layer(*LAYER_OF[name]).with_options(train=True)
    d_out = d_out_for(inp.T, inp.H)
    say(f"[gpu] backward {name} T={inp.T}")
    d_x, d_w = gpu_backward(lay, inp.x, d_out)
    base = "q64" if name in ("q8", "q64") else name
    b = O.backward_per_token(inp, d_out.astype(np.float64), oracle_weights(base))
    assert np.array_equal(lay.views(inp.T)["ids"].cpu().numpy(), b["routing"]["ids"])
    ex, ew = rel(d_x, b["d_x"]), rel(d_w, b["d_w"])
    say(f"[gpu]   d_x max|err|/rms {ex:.3e}, d_w max|err|/rms {ew:.3e}")
    assert ex <= TOL_BF16 and ew <= TOL_BF16


def test_backward_deterministic_and_batch_independent():
    inp = workload("q64", 64)
    lay = layer("q64", 64).with_options(train=True)
    d_out = d_out_for(64, inp.H, seed=5)
    a = gpu_backward(lay, inp.x, d_out)
    b = gpu_backward(lay, inp.x, d_out)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = gpu_backward(lay, inp.x[:13], d_out[:13])
    assert np.array_equal(c[0], a[0][:13]) and np.array_equal(c[1], a[1][:13])


def test_backward_refuses_unsupported_configurations():
    inp = workload("q64", 64)
    x = torch.zeros(8, inp.H, dtype=torch.int16, device="cuda")
    g = torch.zeros(8, inp.H, dtype=torch.float32, device="cuda")
    for lay in (layer("q64", 64), layer("q64", 64, tiled=False).with_options(train=True),
                layer("q64", 64).with_options(renorm=False, train=True), layer("q48q", 64).with_options(train=True),
                layer("q64", 64).with_options(train=True).with_lora(S.lora_adapters(inp.E, inp.H, inp.I))):
        lay.forward(x)
        with pytest.raises(L.MoEError) as ei:
            lay.backward(x, g)
        assert ei.value.status == L.MOE_ERR_UNSUPPORTED


def test_training_forward_gives_the_same_output():
    inp = workload("q64", 64)
    base = layer("q64", 64)
    tr = base.with_options(train=True)
    x = base.upload_x(inp.x)
    a = base.forward(x)
    b = tr.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)

