"""Attention in two parts: the window-only partial (cskv_attend_window_partial)
and the attend over the selected entries that merges it
(cskv_attend_with_partial), against the oracle's partial attention and
log-sum-exp merge; the partial computed on a second stream while the indexer
runs on the first."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import method as M
from tests.helpers import row_rel_err, sorted_ids, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _bf16(seed, tensor, shape):
    return synth.normal_bf16(synth.stream_key(seed, tensor), 0, int(np.prod(shape))).reshape(shape)


def _split_partial(buf, B, H, D):
    """(values [B, H, D], m [B, H], l [B, H]) of a partial buffer."""
    a = buf.detach().cpu().numpy()
    vals = a[:B * H * D].reshape(B, H, D)
    ml = a[B * H * D:B * H * (D + 2)].reshape(B, H, 2)
    return vals, ml[..., 0], ml[..., 1]


def _oracle(Q, cache, ids, win, tau, R, pos, n_window=None):
    out = []
    for b in range(Q.shape[0]):
        w = None if win is None else win[b][: (win.shape[1] if n_window is None else int(n_window[b]))]
        out.append(M.attend(Q[b], cache[b], None if ids is None else ids[b], w, tau, R, 10000.0, pos[b]))
    return np.stack(out)


@pytest.mark.parametrize("B,H,W,fp8", [
    (3, 64, 128, False),   # the c4a layer's window
    (2, 20, 37, False),    # heads not a multiple of 16, a ragged tile
    (2, 64, 128, True),    # fp8 window rows with row scales
    (2, 64, 0, False),     # no window: every sum is 0
])
def test_window_partial_matches_oracle(cskv, B, H, W, fp8):
    D, tau = 512, 1 / np.sqrt(512)
    seed = 800 + B + H + W
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    if fp8:
        wc = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
        wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
        win64 = F.decode_fp8_rows(wc, wsc)
        part = cskv.attend_window_partial(to_dev_bf16(Q), to_dev(wc), window_scale=to_dev(wsc), softmax_scale=tau)
    else:
        win = _bf16(seed, synth.T_WIN, (B, W, D))
        win64 = F.bf16_to_f64(win)
        part = cskv.attend_window_partial(to_dev_bf16(Q), to_dev_bf16(win), softmax_scale=tau)
    torch.cuda.synchronize()
    vals, m, l = _split_partial(part, B, H, D)
    for b in range(B):
        O, lse = M.attention_partial(F.bf16_to_f64(Q[b]), win64[b], tau)
        if W == 0:
            assert np.all(l[b] == 0) and np.all(vals[b] == 0)
            continue
        assert row_rel_err(vals[b], O) <= (6e-2 if fp8 else 2e-2)
        # m is a reference within 64 (log2 units) of the largest logit; m + log2 l is the log-sum-exp
        assert np.all(l[b] > 0)
        np.testing.assert_allclose(m[b] + np.log2(l[b]), lse, atol=2e-3 * max(1.0, np.abs(lse).max()))


@pytest.mark.parametrize("B,H,N,k,W,R,splits", [
    (3, 64, 3000, 512, 128, 64, 0),   # the c4a layer shape, automatic splits
    (3, 64, 3000, 512, 128, 64, 1),   # one split: the attend kernel merges the partial itself
    (2, 20, 900, 100, 7, 0, 3),       # heads not a multiple of 16, no rotation
    (2, 64, 600, 64, 0, 64, 0),       # an empty window partial
])
def test_merged_attend_matches_oracle(cskv, B, H, N, k, W, R, splits):
    D, tau = 512, 1 / np.sqrt(512)
    seed = 900 + B + H + k
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cache = _bf16(seed, synth.T_CACHE, (B, N, D))
    win = _bf16(seed, synth.T_WIN, (B, W, D))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k, n_valid=k - (9 if b == 1 else 0)) for b in range(B)])
    pos = np.array([(1 << 20) - 1 - 977 * b for b in range(B)], dtype=np.int64)
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), ids, F.bf16_to_f64(win), tau, R, pos)
    Qd = to_dev_bf16(Q)
    part = cskv.attend_window_partial(Qd, to_dev_bf16(win), softmax_scale=tau)
    O = cskv.attend(Qd, to_dev_bf16(cache), to_dev(ids), None, softmax_scale=tau, rope_dims=R,
                    q_pos=to_dev(pos), splits=splits, partial=part)
    assert row_rel_err(O.cpu().numpy(), ref) <= 2e-2


def test_merged_attend_fp8_and_ragged_window(cskv):
    """fp8 cache and window rows; ragged n_window in the partial; one sequence
    whose ids are all -1 (only the partial's keys count) and one with an
    empty window (only the entries count)."""
    B, H, D, N, k, W, R = 3, 64, 512, 2000, 256, 128, 64
    seed, tau = 47, 1 / np.sqrt(512)
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cc = synth.fp8_codes(synth.stream_key(seed, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
    cs = synth.pos_scale(synth.stream_key(seed, synth.T_CACHE_SCALE), 0, B * N).reshape(B, N)
    wc = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)])
    ids[1] = -1
    nwin = np.array([W, 77, 0], dtype=np.int32)
    pos = np.array([123456, 99, 5], dtype=np.int64)
    ref = _oracle(F.bf16_to_f64(Q), F.decode_fp8_rows(cc, cs), ids, F.decode_fp8_rows(wc, wsc), tau, R, pos, nwin)
    Qd = to_dev_bf16(Q)
    part = cskv.attend_window_partial(Qd, to_dev(wc), window_scale=to_dev(wsc), n_window=to_dev(nwin),
                                      softmax_scale=tau)
    for splits in (0, 1):
        O = cskv.attend(Qd, to_dev(cc), to_dev(ids), None, cache_scale=to_dev(cs), softmax_scale=tau,
                        rope_dims=R, q_pos=to_dev(pos), splits=splits, partial=part)
        assert row_rel_err(O.cpu().numpy(), ref) <= 6e-2, splits


def test_partial_overlaps_the_indexer_on_a_second_stream(cskv):
    """The decode step with the window partial on a side stream while
    index_topk runs on the main stream: ids bit-exact, O equal to the oracle
    over the selected entries and the window in one softmax, and equal (to
    rounding) to the one-call attend; repeated several times on the same
    buffers and workspaces."""
    B, H, D, N, Di, k, W, R = 4, 64, 512, 20000, 128, 512, 128, 64
    seed, tau = 51, 1 / np.sqrt(512)
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cache = _bf16(seed, synth.T_CACHE, (B, N, D))
    win = _bf16(seed, synth.T_WIN, (B, W, D))
    q_idx = synth.int_bf16(synth.stream_key(seed, synth.T_QIDX), 0, B * Di, 8).reshape(B, Di)
    k_idx = synth.int_bf16(synth.stream_key(seed, synth.T_KIDX), 0, B * N * Di, 8).reshape(B, N, Di)
    pos = np.array([4 * N + 7 + b for b in range(B)], dtype=np.int64)
    ref_ids = np.stack([M.topk_ids(M.index_scores(F.bf16_to_f64(q_idx[b]), F.bf16_to_f64(k_idx[b])), k)
                        for b in range(B)])
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), ref_ids, F.bf16_to_f64(win), tau, R, pos)
    Qd, cd, wd = to_dev_bf16(Q), to_dev_bf16(cache), to_dev_bf16(win)
    qd, kd, pd = to_dev_bf16(q_idx), to_dev_bf16(k_idx), to_dev(pos)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    O_one = cskv.attend(Qd, cd, cskv.index_topk(qd, kd, k), wd, softmax_scale=tau, rope_dims=R, q_pos=pd)
    for _ in range(3):
        ready = torch.cuda.Event()
        ready.record(main)
        with torch.cuda.stream(side):
            side.wait_event(ready)
            part = cskv.attend_window_partial(Qd, wd, softmax_scale=tau)
            done = torch.cuda.Event()
            done.record(side)
        ids = cskv.index_topk(qd, kd, k)
        main.wait_event(done)
        part.record_stream(main)
        O = cskv.attend(Qd, cd, ids, None, softmax_scale=tau, rope_dims=R, q_pos=pd, partial=part)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref_ids)
        assert row_rel_err(O.cpu().numpy(), ref) <= 2e-2
        np.testing.assert_allclose(O.cpu().numpy(), O_one.cpu().numpy(), rtol=0, atol=2e-2 * np.abs(ref).max())
