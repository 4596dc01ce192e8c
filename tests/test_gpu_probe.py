"""The measurement probes read and compute what they claim: the read probe
loads every word of its buffer exactly once (the XOR of its per-wave
results equals the XOR of the buffer), the gather probe copies every word
once when its copies cover the buffer once (either lane order), and the
MFMA probe's per-lane sums are finite, positive and the same on every run."""
import numpy as np
import pytest
import torch

from mixture_experts_decode_router_amd import _lib as L
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,n_wg", [(16, 1), (4096 * 16 + 48, 3), (64 << 20, 2048)])
def test_read_probe_touches_every_word_once(nbytes, n_wg):
    words = np.random.default_rng(nbytes).integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(n_wg * 4, dtype=torch.int32, device="cuda")
    say(f"[gpu] read probe {nbytes} B over {n_wg} workgroups")
    L.moe_probe_read(src, nbytes, sink, n_wg)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("nbytes,row_bytes,n_wg", [(16 * 64, 64, 1), (64 * 4096, 4096, 2), (16 << 20, 4096, 16)])
def test_gather_probe_copies_every_word_once(order, nbytes, row_bytes, n_wg):
    words = np.random.default_rng(nbytes + order).integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64)
    words = words.astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    tiles = nbytes // 1024
    iters = tiles // (4 * n_wg)
    assert iters * 4 * n_wg == tiles or (tiles < 4 * n_wg and tiles == 1)
    if tiles < 4 * n_wg:  # one tile, one wave
        iters = 1
    sink = torch.zeros(n_wg * 4, dtype=torch.int32, device="cuda")
    say(f"[gpu] gather probe {nbytes} B rows {row_bytes} order {order} over {n_wg} workgroups")
    L.moe_probe_gather(src, nbytes, row_bytes, order, iters, sink, n_wg)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    if tiles < 4 * n_wg:  # every wave copied tile 0: the XOR of an odd count of copies is the tile's
        assert n_wg * 4 % 2 == 0
        assert np.bitwise_xor.reduce(got) == 0 and got[0] == np.bitwise_xor.reduce(words)
    else:
        assert np.bitwise_xor.reduce(got) == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_probe_is_repeatable(shape):
    sink = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    L.moe_probe_mfma(sink, 8, 16, shape)
    a = sink.clone()
    L.moe_probe_mfma(sink, 8, 16, shape)
    torch.cuda.synchronize()
    assert torch.equal(a, sink) and bool(torch.isfinite(a).all()) and bool((a > 0).all())


def test_probes_refuse_bad_arguments():
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    for args in ((buf, 20, buf, 1), (buf, 0, buf, 1), (buf, 16, buf, 0)):
        with pytest.raises(L.MoEError) as e:
            L.moe_probe_read(*args)
        assert e.value.status == L.MOE_ERR_INVALID_ARG
    with pytest.raises(L.MoEError):
        L.moe_probe_mfma(buf, 1, 1, 2)
    big = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    for args in ((big, 1 << 18, 96, 0, 1, buf, 1), (big, 1 << 18, 4096, 2, 1, buf, 1),
                 (big, 3 << 16, 4096, 0, 1, buf, 1), (big, 1 << 18, 4096, 0, 0, buf, 1),
                 (big, 1 << 18, 4096, 0, 1, buf, 0), (big, 8 * 4096, 4096, 0, 1, buf, 1)):
        with pytest.raises(L.MoEError) as e:
            L.moe_probe_gather(*args)
        assert e.value.status == L.MOE_ERR_INVALID_ARG
