"""The tiled weight layout written by moe_pack_weights, checked against an
independent numpy formulation of the same layout (reshape + transpose)."""
import numpy as np
import pytest
import torch

import synthetic as S
from mixture_experts_decode_router_amd import _lib as L
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def tiled_bf16(w):
    """[E][R][K] -> chunk order (rt, ks, g, r) of 8 elements each."""
    E, R, K = w.shape
    return w.reshape(E, R // 16, 16, K // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(E, R, K)


def tiled_codes(q):
    """[E][R][K/2] bytes -> chunk order (rt, kb, g, r) of 16 bytes each; inside
    a chunk, 4-byte word st holds the codes of k in [128kb + 32st + 8g, +8)."""
    E, R, B = q.shape
    # row bytes of one 128-k block: (st, g, 4 bytes)
    return q.reshape(E, R // 16, 16, B // 64, 4, 4, 4).transpose(0, 1, 3, 5, 2, 4, 6).reshape(E, R, B)


def tiled_scales(s):
    """[E][R][K/64] -> order (rt, kb, r, h)."""
    E, R, NB = s.shape
    return s.reshape(E, R // 16, 16, NB // 2, 2).transpose(0, 1, 3, 2, 4).reshape(E, R, NB)


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("wfmt", ["bf16", "nf4"])
def test_pack_matches_numpy_layout(wfmt):
    inp = S.make_small(4, 384, 32, 4, 256, seed=8, wfmt=wfmt)
    say(f"[gpu] pack {wfmt}")
    cfg = L.moe_config(inp.H, inp.I, inp.E, inp.k, 4, L.MOE_W_BF16 if wfmt == "bf16" else L.MOE_W_NF4_B64)
    names = ("w_gate_up", "w_down") if wfmt == "bf16" else ("q_gate_up", "s_gate_up", "q_down", "s_down")
    src_t = {n: dev(getattr(inp, n)) for n in names}
    dst_t = {n: torch.empty_like(v) for n, v in src_t.items()}

    def weights(d):
        return L.moe_weights(*[d[f].data_ptr() if f in d else None for f, _ in L.moe_weights._fields_])

    L.moe_pack_weights(cfg, weights(src_t), weights(dst_t))
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in dst_t.items()}
    if wfmt == "bf16":
        assert np.array_equal(got["w_gate_up"].view(np.uint16), tiled_bf16(inp.w_gate_up))
        assert np.array_equal(got["w_down"].view(np.uint16), tiled_bf16(inp.w_down))
    else:
        assert np.array_equal(got["q_gate_up"], tiled_codes(inp.q_gate_up))
        assert np.array_equal(got["q_down"], tiled_codes(inp.q_down))
        assert np.array_equal(got["s_gate_up"], tiled_scales(inp.s_gate_up))
        assert np.array_equal(got["s_down"], tiled_scales(inp.s_down))
