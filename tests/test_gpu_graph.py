"""Replays of HIP graphs captured from index_topk and attend calls give the
eager results bit for bit, also with eager work and synchronisations between
the replays (the benchmark times decode steps as graph replays)."""
import numpy as np
import pytest
import torch

import synth
from synth import device as sd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _inputs(seed, B, N, D, H, Di, W):
    key = lambda t: synth.stream_key(seed, t)
    return dict(
        qidx=sd.new((B, Di), synth.KIND_INT_BF16, key(synth.T_QIDX), a=8),
        kidx=sd.new((B, N, Di), synth.KIND_INT_BF16, key(synth.T_KIDX), a=8),
        cache=sd.new((B, N, D), synth.KIND_NORMAL_BF16, key(synth.T_CACHE)),
        win=sd.new((B, W, D), synth.KIND_NORMAL_BF16, key(synth.T_WIN)),
        Q=sd.new((B, H, D), synth.KIND_NORMAL_BF16, key(synth.T_Q)),
        pos=torch.full((B,), 4 * N + 7, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("dense", [False, True])
def test_graph_replays_match_eager(cskv, dense):
    B, N, D, H, Di, W, k = 4, 6000, 512, 64, 128, 128, 512
    x = _inputs(71, B, N, D, H, Di, W)
    other = _inputs(72, B, N, D, H, Di, W)
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")

    def step(inp, ids_buf, out_buf):
        sel = None
        if not dense:
            cskv.index_topk(inp["qidx"], inp["kidx"], k, ids=ids_buf)
            sel = ids_buf
        cskv.attend(inp["Q"], inp["cache"], sel, inp["win"], softmax_scale=D ** -0.5, rope_dims=64,
                    q_pos=inp["pos"], out=out_buf)

    step(x, ids, out)                      # eager, also sizes the workspaces
    torch.cuda.synchronize()
    ref_ids, ref_out = ids.clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, ids, out)
    ids2 = torch.empty_like(ids)
    out2 = torch.empty_like(out)
    for r in range(4):
        ids.fill_(-7)
        out.zero_()
        g.replay()
        step(other, ids2, out2)           # eager work between the replays
        torch.cuda.synchronize()
        if not dense:
            assert torch.equal(ids, ref_ids), r
        assert torch.equal(out, ref_out), r


def test_graph_replays_after_other_shapes_on_the_capture_stream(cskv):
    """Between replays, eager calls on the capture stream itself: index_topk
    with another batch size (a workspace layout of its own) and an attend
    large enough to grow the stream's attend workspace (the captured buffer is
    retired, not freed). Every replay still gives the eager result."""
    B, N, D, H, Di, W, k = 4, 6000, 512, 64, 128, 128, 512
    x = _inputs(73, B, N, D, H, Di, W)
    big = _inputs(74, 7, 3 * N, D, H, Di, W)
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def step():
        cskv.index_topk(x["qidx"], x["kidx"], k, ids=ids)
        cskv.attend(x["Q"], x["cache"], ids, x["win"], softmax_scale=D ** -0.5, rope_dims=64, q_pos=x["pos"],
                    out=out)

    with torch.cuda.stream(s):
        step()                                 # eager on the capture stream: sizes its workspaces
    torch.cuda.synchronize()
    ref_ids, ref_out = ids.clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    ids_big = torch.empty((7, k), dtype=torch.int32, device="cuda")
    for r in range(4):
        ids.fill_(-7)
        out.zero_()
        g.replay()
        with torch.cuda.stream(s):
            cskv.index_topk(big["qidx"], big["kidx"], k, ids=ids_big)          # another layout
            cskv.attend(big["Q"], big["cache"], None, big["win"], softmax_scale=D ** -0.5, rope_dims=64,
                        q_pos=big["pos"], splits=40 + r)                        # grows the attend workspace
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids), r
        assert torch.equal(out, ref_out), r
