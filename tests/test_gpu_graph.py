"""hipGraph capture per batch-size bucket: replay is bit-identical to eager
(the captured-equals-eager invariant of the bucketed decode capture), across
all buckets, partial buckets, re-capture, and the refusal paths."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic as S
from mixture_experts_decode_router_amd import _lib as L
from tests.gpu_util import TOL_BF16, layer, oracle_forward, rel_err, say, workload

pytestmark = pytest.mark.gpu

BUCKETS = list(S.SWEEP_T)  # [1, 2, 4, 8] + 16-steps up to 64


@pytest.fixture(scope="module")
def captured():
    lay = layer("q64", 64)
    stream = torch.cuda.Stream()
    x_static = torch.zeros(64, lay.H, dtype=torch.int16, device="cuda")
    out_static = torch.zeros(64, lay.H, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    say("[gpu] capture 8 buckets")
    lay.capture(BUCKETS, x_static, out_static, stream)
    yield lay, stream, x_static, out_static
    lay.release_graph()


def test_bucket_choice(captured):
    lay = captured[0]
    assert [L.moe_graph_bucket_for(lay.graph, t) for t in (1, 2, 3, 5, 8, 9, 17, 33, 49, 64, 65)] == \
        [1, 2, 4, 8, 8, 16, 32, 48, 64, 64, -1]


@pytest.mark.parametrize("T", BUCKETS)
def test_replay_equals_eager_and_oracle(captured, T):
    lay, stream, x_static, out_static = captured
    inp = workload("q64", T)
    say(f"[gpu] replay bucket T={T}")
    x = lay.upload_x(inp.x)
    with torch.cuda.stream(stream):
        x_static[:T].copy_(x)
        lay.replay(T, stream)
        eager = lay.forward(x.clone(), stream=stream)
    stream.synchronize()
    assert torch.equal(out_static[:T], eager)
    ref_out, _ = oracle_forward("q64", T)
    assert rel_err(out_static[:T].cpu().numpy(), ref_out) <= TOL_BF16


@pytest.mark.parametrize("T", [5, 13, 40])
def test_partial_bucket_masks_rows_past_T(captured, T):
    """replay(T) runs the smallest bucket >= T; a device live count keeps rows
    T.. out of routing, bucketing and the output (they are left untouched)."""
    lay, stream, x_static, out_static = captured
    inp = workload("q64", 64)
    b = L.moe_graph_bucket_for(lay.graph, T)
    say(f"[gpu] partial bucket T={T} (bucket {b})")
    with torch.cuda.stream(stream):
        x_static.copy_(lay.upload_x(inp.x))
        out_static.fill_(12345.0)
        lay.replay(T, stream)
        v = lay.views(b)
        counts = v["counts"].clone()
        got = out_static.clone()
        eager = lay.forward(lay.upload_x(inp.x[:T]), stream=stream)
    stream.synchronize()
    assert torch.equal(got[:T], eager)
    assert int(counts.sum()) == T * lay.k
    assert bool((got[T:b] == 12345.0).all())


def test_live_count_follows_each_replay(captured):
    """Alternating partial and full replays of one bucket: each sees its own T."""
    lay, stream, x_static, out_static = captured
    inp = workload("q64", 64)
    with torch.cuda.stream(stream):
        x_static.copy_(lay.upload_x(inp.x))
        full = lay.forward(lay.upload_x(inp.x), stream=stream)
        for T in (64, 50, 64, 33, 64):
            lay.replay(T, stream)
            torch.cuda.current_stream().synchronize()
            assert torch.equal(out_static[:T], full[:T]), T
    stream.synchronize()


def test_replay_ignores_what_the_workspace_held_before(captured):
    """Every replay writes its own live row count (the graph's first node),
    so a workspace overwritten between two replays of the same partial T
    (here filled with 0xFF bytes) gives the same result; so does a second
    graph set on the same workspace replayed in between with another T."""
    lay, stream, x_static, out_static = captured
    inp = workload("q64", 64)
    say("[gpu] replays around a workspace fill")
    other = L.moe_graph_capture(lay.cfg, lay.w, [64], x_static, out_static, lay.workspace, lay.ws_bytes, stream)
    try:
        with torch.cuda.stream(stream):
            x_static.copy_(lay.upload_x(inp.x))
            eager = lay.forward(lay.upload_x(inp.x[:40]), stream=stream)
            lay.replay(40, stream)
            first = out_static[:40].clone()
            lay.workspace.fill_(255)
            out_static.fill_(-7.0)
            lay.replay(40, stream)
            second = out_static.clone()
            L.moe_graph_replay(other, 64, stream)
            lay.replay(40, stream)
            third = out_static[:40].clone()
        stream.synchronize()
    finally:
        L.moe_graph_destroy(other)
    assert torch.equal(first, eager)
    assert torch.equal(second[:40], eager)
    assert bool((second[40:48] == -7.0).all())
    assert torch.equal(third, eager)


def test_replays_are_repeatable(captured):
    lay, stream, x_static, out_static = captured
    inp = workload("q64", 64)
    with torch.cuda.stream(stream):
        x_static.copy_(lay.upload_x(inp.x))
        lay.replay(64, stream)
        first = out_static.clone()
        for _ in range(10):
            lay.replay(64, stream)
            torch.cuda.current_stream().synchronize()
            assert torch.equal(out_static, first)
    stream.synchronize()


def test_replay_beyond_largest_bucket_is_rejected(captured):
    lay, stream, _, _ = captured
    with pytest.raises(L.MoEError) as e:
        lay.replay(65, stream)
    assert e.value.status == L.MOE_ERR_INVALID_ARG


def test_recapture_after_destroy():
    lay = layer("q64", 64)
    inp = workload("q64", 8)
    stream = torch.cuda.Stream()
    xs = torch.zeros(64, lay.H, dtype=torch.int16, device="cuda")
    os_ = torch.zeros(64, lay.H, dtype=torch.float32, device="cuda")
    for rnd in range(2):
        g = L.moe_graph_capture(lay.cfg, lay.w, [8, 64], xs, os_, lay.workspace, lay.ws_bytes, stream)
        with torch.cuda.stream(stream):
            xs[:8].copy_(lay.upload_x(inp.x))
            L.moe_graph_replay(g, 8, stream)
            eager = lay.forward(lay.upload_x(inp.x), stream=stream)
        stream.synchronize()
        assert torch.equal(os_[:8], eager), rnd
        L.moe_graph_destroy(g)


def test_capture_refused_on_null_stream():
    lay = layer("q64", 64)
    xs = torch.zeros(64, lay.H, dtype=torch.int16, device="cuda")
    os_ = torch.zeros(64, lay.H, dtype=torch.float32, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.moe_graph_capture(lay.cfg, lay.w, [1, 2], xs, os_, lay.workspace, lay.ws_bytes, 0)
    assert e.value.status == L.MOE_ERR_NOT_CAPTURABLE


def test_synchronising_call_refused_while_capturing():
    lay = layer("q64", 64)
    hip = ctypes.CDLL("libamdhip64.so")
    stream = torch.cuda.Stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    torch.cuda.synchronize()
    assert hip.hipStreamBeginCapture(sh, 0) == 0  # hipStreamCaptureModeGlobal
    try:
        with pytest.raises(L.MoEError) as e:
            lay.read_counts(stream=stream.cuda_stream)
        assert e.value.status == L.MOE_ERR_CAPTURE_VIOLATION
    finally:
        g = ctypes.c_void_p()
        assert hip.hipStreamEndCapture(sh, ctypes.byref(g)) == 0
        if g.value:
            hip.hipGraphDestroy(g)
    # and the same call works once the stream is not capturing
    lay.forward(lay.upload_x(workload("q64", 8).x), stream=stream)
    counts = lay.read_counts(stream=stream.cuda_stream)
    assert counts.sum() == 8 * lay.k
