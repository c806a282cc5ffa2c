"""The 61-layer decode step, run through the benchmark's own workload code
(per layer: compress the appended states into the cache, top-k for c4a
layers, then attention), checked layer by layer against the oracle on inputs
the host regenerates from the same streams."""
import argparse
import dataclasses

import numpy as np
import pytest
import torch

import bench
import synth
from oracle import formats as F
from oracle import method as M
from synth import configs
from synth import device as sd
from tests.helpers import row_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _run(cfg, cskv):
    args = argparse.Namespace(chunk=0, splits=0)
    wl = bench.Mixed61(cfg, args, torch, cskv, sd, synth)
    wl.setup(1)
    wl.step_layers()
    torch.cuda.synchronize()
    return wl


def _bf16_rows(key, b, n_rows, D, rows):
    """Rows `rows` of sequence b of a [B, n_rows, D] N(0,1) bf16 tensor."""
    if isinstance(rows, range):
        return synth.normal_bf16(key, (b * n_rows + rows.start) * D, len(rows) * D).reshape(len(rows), D)
    return np.stack([synth.normal_bf16(key, (b * n_rows + int(r)) * D, D) for r in rows])


def _check_layer(wl, layer, b, full_cache_rows=None):
    """Oracle for sequence b of one layer: the cache rows the step reads are the
    drawn prefix plus the entries compressed from the appended span."""
    c = wl.cfg
    lay = next(x for x in wl.layers if x["layer"] == layer)
    assert lay["kind"] == c.layer_kind(layer)
    kind = lay["kind"]
    key = lambda tensor: wl.key(0, tensor, layer)
    D, H, W = c.D, c.H, c.W
    span_T = 132 if kind == "c4a" else 128
    span = synth.normal_bf16(key(synth.T_S), b * span_T * D, span_T * D).reshape(span_T, D)
    gate = synth.normal_f32(key(synth.T_GATE), b * span_T, span_T)
    Q = F.bf16_to_f64(synth.normal_bf16(key(synth.T_Q), b * H * D, H * D).reshape(H, D))
    new = M.compress(kind, F.bf16_to_f64(span), gate.astype(np.float64))
    new_bf16 = F.bf16_to_f64(F.f32_to_bf16(new.astype(np.float32)))   # the cache stores bf16
    first = lay["first"]
    N = wl.N4 if kind == "c4a" else wl.N128
    window = F.bf16_to_f64(span[span_T - W:])
    O_gpu = lay["O"][b].cpu().numpy()
    if kind == "c4a":
        Di = c.Di
        # a layer that reuses ids attends over the selection of the layer it names
        src = lay.get("reuse")
        src = layer if src is None else src
        ikey = lambda tensor: wl.key(0, tensor, src)  # noqa: E731
        q = F.bf16_to_f64(synth.int_bf16(ikey(synth.T_QIDX), b * Di, Di, c.idx_range))
        kk = F.bf16_to_f64(synth.int_bf16(ikey(synth.T_KIDX), b * N * Di, N * Di, c.idx_range).reshape(N, Di))
        ids = M.topk_ids(M.index_scores(q, kk), c.k)
        src_lay = next(x for x in wl.layers if x["layer"] == src)
        assert np.array_equal(src_lay["ids"][b].cpu().numpy(), ids), (layer, b)
        # only the selected rows are needed: drawn rows, or rows the span rewrote
        cache = np.zeros((N, D))
        drawn = [r for r in ids if r < first or r >= first + new.shape[0]]
        if drawn:
            cache[drawn] = F.bf16_to_f64(_bf16_rows(key(synth.T_CACHE), b, N, D, drawn))
        cache[first:first + new.shape[0]] = new_bf16
        ref = M.attend(Q, cache, ids, window, c.tau, c.R, c.rope_base, c.q_pos)
    else:
        cache = F.bf16_to_f64(_bf16_rows(key(synth.T_CACHE), b, N, D, range(N)))
        cache[first:first + new.shape[0]] = new_bf16
        ref = M.attend(Q, cache, None, window, c.tau, c.R, c.rope_base, c.q_pos)
    err = row_rel_err(O_gpu, ref)
    assert err <= 2e-2, (layer, kind, b, err)


def test_mixed_step_small(cskv):
    """Four layers (c128a, c4a, c128a, c4a) of 2 sequences x 8192 tokens."""
    cfg = dataclasses.replace(configs.MIXED_61, name="mixed_small", number=50, B=2, L=8192, layers=4)
    wl = _run(cfg, cskv)
    for layer in range(cfg.layers):
        for b in range(cfg.B):
            _check_layer(wl, layer, b)


@pytest.mark.slow
def test_mixed_step_full_size_first_layers(cskv):
    """The 61-layer workload's first two layers (one c128a, one c4a) at full size
    (64 sequences x 262144 tokens), in the benchmark's launch configuration, with
    the same input streams; sampled sequences are checked."""
    cfg = dataclasses.replace(configs.MIXED_61, layers=2)
    wl = _run(cfg, cskv)
    for layer in (0, 1):
        for b in (0, cfg.B - 1):
            _check_layer(wl, layer, b)


@pytest.mark.slow
def test_mixed_step_full_size_late_layers(cskv):
    """The last two layers of the 61-layer workload (59: c4a, 60: c128a) at full
    size, each with its own input streams (built alone: the step's layers share
    no data), on first, middle and last sequences."""
    cfg = dataclasses.replace(configs.MIXED_61, only_layers=(59, 60))
    wl = _run(cfg, cskv)
    for layer in (59, 60):
        for b in (0, cfg.B // 2, cfg.B - 1):
            _check_layer(wl, layer, b)


def test_mixed_step_reusing_ids(cskv):
    """Eight layers with id reuse: c4a layers 3 and 7 skip their indexer and
    attend over the selections of layers 1 and 5."""
    cfg = dataclasses.replace(configs.MIXED_61_REUSE, name="mixed_reuse_small", number=51, B=2, L=8192, layers=8)
    wl = _run(cfg, cskv)
    assert [l for l in range(cfg.layers) if cfg.reuses(l) is not None] == [3, 7]
    assert wl.n_dominant() == 2
    for layer in range(cfg.layers):
        for b in range(cfg.B):
            _check_layer(wl, layer, b)
