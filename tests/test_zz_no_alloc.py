"""moe_forward_noalloc (no workspace argument: the library's static device
scratch) against moe_forward on the same inputs: bit-identical outputs on
two calls in a row, the second with fewer tokens, and a config too large
for the scratch refused before any launch."""
import numpy as np
import pytest
import torch

from mixture_experts_decode_router_amd import _lib as L
from tests.gpu_util import TOL_BF16, TOL_NF4, layer, oracle_forward, rel_err, say, workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["q64", "q48q"])
def test_noalloc_forward_equals_forward(name):
    lay = layer(name, 64)
    for T in (64, 9):
        inp = workload(name, T)
        say(f"[gpu] no-alloc forward {name} T={T}")
        x = lay.upload_x(inp.x)
        ref = lay.forward(x)
        out = torch.full((T, lay.H), float("nan"), dtype=torch.float32, device="cuda")
        L.moe_forward_noalloc(lay.cfg, lay.w, x, T, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), T
        ref_out, _ = oracle_forward(name, T)
        tol = TOL_NF4 if name == "q48q" else TOL_BF16
        assert rel_err(out.cpu().numpy(), ref_out) <= tol


def test_noalloc_refuses_a_config_beyond_the_scratch():
    lay = layer("q64", 64)
    big = L.moe_config(lay.cfg.hidden, lay.cfg.inter, lay.cfg.n_experts, lay.cfg.top_k, 4096, lay.cfg.wfmt)
    x = torch.zeros(8, lay.H, dtype=torch.int16, device="cuda")
    out = torch.zeros(8, lay.H, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.moe_forward_noalloc(big, lay.w, x, 8, out)
    assert e.value.status == L.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()   # nothing was launched
