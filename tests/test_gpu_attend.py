"""attend parity: GPU output against the oracle's float64 attention + inverse
RoPE on identical input bytes (row-relative <= 2e-2 bf16, <= 6e-2 fp8)."""
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


def _oracle(Q, cache, ids, win, tau, R, base, pos, n_entries=None):
    B = Q.shape[0]
    return np.stack([M.attend(Q[b], cache[b], None if ids is None else ids[b],
                              None if win is None else win[b], tau, R, base, pos[b],
                              None if n_entries is None else int(n_entries[b])) for b in range(B)])


@pytest.mark.parametrize("B,H,D,N,k,W,R", [
    (1, 8, 128, 511, 64, 32, 32),      # the tiny workload's shape
    (3, 64, 512, 3000, 512, 128, 64),  # the c4a layer shape
    (2, 20, 512, 900, 100, 7, 0),      # heads not a multiple of 16, no rotation
    (2, 64, 128, 300, 37, 0, 16),      # no window
])
def test_sparse_bf16_matches_oracle(cskv, B, H, D, N, k, W, R):
    seed = B * 100 + H
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cache = _bf16(seed, synth.T_CACHE, (B, N, D))
    win = _bf16(seed, synth.T_WIN, (B, W, D))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k, n_valid=k - (3 if b == 1 else 0)) for b in range(B)])
    pos = np.array([1000 + 977 * b for b in range(B)], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), ids, F.bf16_to_f64(win), tau, R, 10000.0, pos)
    for splits in (0, 1, 3):
        O = cskv.attend(to_dev_bf16(Q), to_dev_bf16(cache), to_dev(ids), to_dev_bf16(win) if W else None,
                        softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos), splits=splits)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= 2e-2, (splits, err)


@pytest.mark.parametrize("splits", [0, 1, 5, 40])
def test_dense_bf16_matches_oracle(cskv, splits):
    B, H, D, N, W, R = 3, 64, 512, 1500, 128, 64
    Q = _bf16(1, synth.T_Q, (B, H, D))
    cache = _bf16(1, synth.T_CACHE, (B, N, D))
    win = _bf16(1, synth.T_WIN, (B, W, D))
    nv = np.array([1500, 33, 0], dtype=np.int32)
    pos = np.array([(1 << 20) - 1, 5, 0], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), None, F.bf16_to_f64(win), tau, R, 10000.0, pos, nv)
    O = cskv.attend(to_dev_bf16(Q), to_dev_bf16(cache), None, to_dev_bf16(win), softmax_scale=tau,
                    rope_dims=R, q_pos=to_dev(pos), n_entries=to_dev(nv), splits=splits)
    assert row_rel_err(O.cpu().numpy(), ref) <= 2e-2


def test_fp8_cache_and_window_match_oracle(cskv):
    B, H, D, N, k, W, R = 2, 64, 512, 2000, 512, 128, 64
    seed = 44
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cc = synth.fp8_codes(synth.stream_key(seed, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
    cs = synth.pos_scale(synth.stream_key(seed, synth.T_CACHE_SCALE), 0, B * N).reshape(B, N)
    wc = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)])
    pos = np.array([123456, 7], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    ref = _oracle(F.bf16_to_f64(Q), F.decode_fp8_rows(cc, cs), ids, F.decode_fp8_rows(wc, wsc), tau, R,
                  10000.0, pos)
    for splits in (0, 1):
        O = cskv.attend(to_dev_bf16(Q), to_dev(cc), to_dev(ids), to_dev(wc), cache_scale=to_dev(cs),
                        window_scale=to_dev(wsc), softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos),
                        splits=splits)
        assert row_rel_err(O.cpu().numpy(), ref) <= 6e-2


def test_window_is_a_view_into_a_span(cskv):
    B, H, D, N, k, T, W = 2, 64, 512, 600, 64, 132, 128
    Q = _bf16(2, synth.T_Q, (B, H, D))
    cache = _bf16(2, synth.T_CACHE, (B, N, D))
    span = _bf16(2, synth.T_S, (B, T, D))
    rng = np.random.default_rng(2)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)])
    pos = np.array([5000, 6000], dtype=np.int64)
    span_d = to_dev_bf16(span)
    O = cskv.attend(to_dev_bf16(Q), to_dev_bf16(cache), to_dev(ids), span_d[:, T - W:, :],
                    softmax_scale=0.05, rope_dims=64, q_pos=to_dev(pos))
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), ids, F.bf16_to_f64(span[:, T - W:]), 0.05, 64,
                  10000.0, pos)
    assert row_rel_err(O.cpu().numpy(), ref) <= 2e-2


def test_empty_key_sets(cskv):
    B, H, D = 2, 16, 128
    Q = to_dev_bf16(_bf16(3, synth.T_Q, (B, H, D)))
    cache = to_dev_bf16(_bf16(3, synth.T_CACHE, (B, 10, D)))
    ids = torch.full((B, 4), -1, dtype=torch.int32, device="cuda")
    O = cskv.attend(Q, cache, ids, None, softmax_scale=0.1)
    assert torch.all(O == 0)
    win = _bf16(3, synth.T_WIN, (B, 5, D))
    O = cskv.attend(Q, cache, ids, to_dev_bf16(win), softmax_scale=0.1).cpu().numpy()
    ref = np.stack([M.attention(F.bf16_to_f64(_bf16(3, synth.T_Q, (B, H, D))[b]), F.bf16_to_f64(win[b]), 0.1)
                    for b in range(B)])
    assert row_rel_err(O, ref) <= 2e-2


def test_attend_deterministic(cskv):
    B, H, D, N = 2, 64, 512, 5000
    Q = to_dev_bf16(_bf16(4, synth.T_Q, (B, H, D)))
    cache = to_dev_bf16(_bf16(4, synth.T_CACHE, (B, N, D)))
    win = to_dev_bf16(_bf16(4, synth.T_WIN, (B, 128, D)))
    pos = torch.tensor([1, 2], dtype=torch.int64, device="cuda")
    a = cskv.attend(Q, cache, None, win, softmax_scale=0.04, rope_dims=64, q_pos=pos).cpu().numpy()
    b = cskv.attend(Q, cache, None, win, softmax_scale=0.04, rope_dims=64, q_pos=pos).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("case", ["large", "negative", "mixed"])
@pytest.mark.parametrize("sparse", [False, True])
def test_logits_far_from_zero(cskv, case, sparse):
    """Logit ranges far above or below zero (in log2 units, beyond the 64 of
    headroom around the first pass's reference maximum) take the second pass;
    heads of one sequence may need it while others do not."""
    B, H, D, N, k, W, R = 2, 64, 512, 1200, 256, 40, 64
    seed = {"large": 61, "negative": 62, "mixed": 63}[case]
    Q = F.bf16_to_f64(_bf16(seed, synth.T_Q, (B, H, D)))
    cache = F.bf16_to_f64(_bf16(seed, synth.T_CACHE, (B, N, D)))
    win = F.bf16_to_f64(_bf16(seed, synth.T_WIN, (B, W, D)))
    tau = 1 / np.sqrt(D)
    if case == "large":
        tau = 3.0                          # logits with a spread of hundreds
    else:
        # rows near a common direction u; heads pointing against it see only
        # very negative logits
        cache = 1.0 + 0.1 * cache
        win = 1.0 + 0.1 * win
        # mixed: heads against u, along u, and across it (ordinary logits)
        sign = -np.ones(H) if case == "negative" else np.array([-1.0, 1.0, 0.0])[np.arange(H) % 3]
        Q = sign[None, :, None] + 0.1 * Q
        tau = 0.2
    Qb, cb, wb = (F.f32_to_bf16(x.astype(np.float32)) for x in (Q, cache, win))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)]) if sparse else None
    pos = np.array([77, 1 << 19], dtype=np.int64)
    ref = _oracle(F.bf16_to_f64(Qb), F.bf16_to_f64(cb), ids, F.bf16_to_f64(wb), tau, R, 10000.0, pos)
    for splits in (0, 1, 4):
        O = cskv.attend(to_dev_bf16(Qb), to_dev_bf16(cb), None if ids is None else to_dev(ids), to_dev_bf16(wb),
                        softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos), splits=splits)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= 2e-2, (splits, err)


def test_fp8_logits_far_from_zero(cskv):
    """The second pass on the scaled (fp8) rows path."""
    B, H, D, N, k, W, R = 1, 64, 512, 700, 512, 128, 64
    seed = 64
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cc = synth.fp8_codes(synth.stream_key(seed, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
    cs = synth.pos_scale(synth.stream_key(seed, synth.T_CACHE_SCALE), 0, B * N).reshape(B, N)
    wc = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)])
    pos = np.array([4242], dtype=np.int64)
    tau = 4.0
    ref = _oracle(F.bf16_to_f64(Q), F.decode_fp8_rows(cc, cs), ids, F.decode_fp8_rows(wc, wsc), tau, R,
                  10000.0, pos)
    for splits in (0, 1):
        O = cskv.attend(to_dev_bf16(Q), to_dev(cc), to_dev(ids), to_dev(wc), cache_scale=to_dev(cs),
                        window_scale=to_dev(wsc), softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos),
                        splits=splits)
        assert row_rel_err(O.cpu().numpy(), ref) <= 6e-2


@pytest.mark.parametrize("B,H,k,W,R", [
    (64, 64, 512, 128, 64),   # the c4a layer shape of the 61-layer step (one split per CU at auto splits)
    (64, 64, 300, 40, 64),    # a ragged last tile and a short window
    (256, 16, 100, 0, 0),     # one head group, no window, no rotation
])
def test_sparse_large_batch_matches_oracle(cskv, B, H, k, W, R):
    """Sparse bf16 reads at large batches, automatic splits and one split;
    some sequences end in -1 ids."""
    D, N = 512, 2000
    seed = 700 + B + H
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cache = _bf16(seed, synth.T_CACHE, (B, N, D))
    win = _bf16(seed, synth.T_WIN, (B, W, D))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k, n_valid=k - (5 if b % 7 == 3 else 0)) for b in range(B)])
    pos = np.array([1000 + 977 * b for b in range(B)], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    ref = _oracle(F.bf16_to_f64(Q), F.bf16_to_f64(cache), ids, F.bf16_to_f64(win) if W else None, tau, R,
                  10000.0, pos)
    for splits in (0, 1):
        O = cskv.attend(to_dev_bf16(Q), to_dev_bf16(cache), to_dev(ids), to_dev_bf16(win) if W else None,
                        softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos), splits=splits)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= 2e-2, (splits, err)


def test_sparse_large_batch_far_logits(cskv):
    """The second pass at a large batch: heads against, along and across a
    common row direction, so some heads' logits lie far below zero."""
    B, H, D, N, k, W, R = 64, 64, 512, 1200, 256, 40, 64
    seed = 64
    Q = F.bf16_to_f64(_bf16(seed, synth.T_Q, (B, H, D)))
    cache = 1.0 + 0.1 * F.bf16_to_f64(_bf16(seed, synth.T_CACHE, (B, N, D)))
    win = 1.0 + 0.1 * F.bf16_to_f64(_bf16(seed, synth.T_WIN, (B, W, D)))
    Q = np.array([-1.0, 1.0, 0.0])[np.arange(H) % 3][None, :, None] + 0.1 * Q
    tau = 0.2
    Qb, cb, wb = (F.f32_to_bf16(x.astype(np.float32)) for x in (Q, cache, win))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k) for _ in range(B)])
    pos = np.array([77 + (1 << 14) * b for b in range(B)], dtype=np.int64)
    ref = _oracle(F.bf16_to_f64(Qb), F.bf16_to_f64(cb), ids, F.bf16_to_f64(wb), tau, R, 10000.0, pos)
    O = cskv.attend(to_dev_bf16(Qb), to_dev_bf16(cb), to_dev(ids), to_dev_bf16(wb), softmax_scale=tau,
                    rope_dims=R, q_pos=to_dev(pos))
    assert row_rel_err(O.cpu().numpy(), ref) <= 2e-2


@pytest.mark.parametrize("sparse", [False, True])
def test_far_negative_logits_with_empty_splits(cskv, sparse):
    """Every logit far below zero (about -148 in log2 units) while some splits
    hold no key at all: ragged n_entries (dense) or mostly -1 ids (sparse).
    An empty split's (reference maximum, sum) pair must not enter the merge,
    or its reference of 0 would underflow every real split's weight."""
    B, H, D, N, k, W, R = 2, 64, 512, 1200, 256, 40, 64
    seed = 65
    Q = F.bf16_to_f64(_bf16(seed, synth.T_Q, (B, H, D)))
    cache = 1.0 + 0.1 * F.bf16_to_f64(_bf16(seed, synth.T_CACHE, (B, N, D)))
    win = 1.0 + 0.1 * F.bf16_to_f64(_bf16(seed, synth.T_WIN, (B, W, D)))
    Q = -1.0 + 0.1 * Q
    tau = 0.2
    Qb, cb, wb = (F.f32_to_bf16(x.astype(np.float32)) for x in (Q, cache, win))
    rng = np.random.default_rng(seed)
    pos = np.array([77, 1 << 19], dtype=np.int64)
    if sparse:
        ids = np.stack([sorted_ids(rng, N, k), sorted_ids(rng, N, k, n_valid=30)])
        nv = None
    else:
        ids = None
        nv = np.array([N, 30], dtype=np.int32)
    ref = _oracle(F.bf16_to_f64(Qb), F.bf16_to_f64(cb), ids, F.bf16_to_f64(wb), tau, R, 10000.0, pos, nv)
    assert np.all(np.abs(ref).max(axis=-1) > 0.5)
    for splits in (0, 4, 40):
        O = cskv.attend(to_dev_bf16(Qb), to_dev_bf16(cb), None if ids is None else to_dev(ids), to_dev_bf16(wb),
                        softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos),
                        n_entries=None if nv is None else to_dev(nv), splits=splits)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= 2e-2, (splits, err)


@pytest.mark.parametrize("B,H,k,W,R,fmt", [
    (32, 64, 512, 128, 64, "bf16"),   # the c4a 128K layer
    (8, 64, 512, 128, 64, "fp8"),     # the c4a 1M layer
    (4, 64, 300, 40, 64, "bf16"),     # a ragged last tile
    (16, 40, 100, 7, 0, "bf16"),      # heads not a multiple of 16, no rotation
    (8, 64, 1100, 128, 64, "bf16"),   # more entries than the c4a layers select
    (12, 64, 512, 0, 64, "fp8"),      # no window; a batch that is not a multiple of 8
])
def test_sparse_ragged_windows_match_oracle(cskv, B, H, k, W, R, fmt):
    """Sparse reads at automatic splits and at one split against the oracle,
    with ragged window counts (n_window) and some sequences ending in -1 ids."""
    D, N = 512, 2500
    seed = 900 + B + k
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    rng = np.random.default_rng(seed)
    ids = np.stack([sorted_ids(rng, N, k, n_valid=k - (7 if b % 5 == 2 else 0)) for b in range(B)])
    nw = np.array([W - (13 * b) % (W + 1) for b in range(B)], dtype=np.int32)
    pos = np.array([1000 + 4093 * b for b in range(B)], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    extra = {}
    if fmt == "bf16":
        cache = _bf16(seed, synth.T_CACHE, (B, N, D))
        win = _bf16(seed, synth.T_WIN, (B, W, D))
        c64, w64 = F.bf16_to_f64(cache), F.bf16_to_f64(win)
        cache_d, win_d = to_dev_bf16(cache), to_dev_bf16(win) if W else None
        tol = 2e-2
    else:
        cache = synth.fp8_codes(synth.stream_key(seed, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
        cs = synth.pos_scale(synth.stream_key(seed, synth.T_CACHE_SCALE), 0, B * N).reshape(B, N)
        win = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
        wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
        c64, w64 = F.decode_fp8_rows(cache, cs), F.decode_fp8_rows(win, wsc)
        cache_d, win_d = to_dev(cache), to_dev(win) if W else None
        extra = {"cache_scale": to_dev(cs)}
        if W:
            extra["window_scale"] = to_dev(wsc)
        tol = 6e-2
    Q64 = F.bf16_to_f64(Q)
    ref = np.stack([M.attend(Q64[b], c64[b], ids[b], w64[b, :nw[b]] if nw[b] > 0 else None, tau, R, 10000.0,
                             pos[b]) for b in range(B)])
    for splits in (0, 1):
        O = cskv.attend(to_dev_bf16(Q), cache_d, to_dev(ids), win_d, softmax_scale=tau, rope_dims=R,
                        q_pos=to_dev(pos), n_window=to_dev(nw) if W else None, splits=splits, **extra)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= tol, (splits, err)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_attend_skips_invalid_ids(cskv, fmt):
    """Ids past the cache (and -1 padding) stay out of the softmax for bf16 and
    fp8 rows too, whether they fall in a tile whose 8 rows per wave all come
    from the cache (scalar row addresses) or not, at several split counts."""
    B, H, D, N, k, W, R = 2, 64, 512, 400, 256, 24, 64
    seed = 31
    rng = np.random.default_rng(seed)
    ids = np.full((B, k), -1, dtype=np.int32)
    ids[0, :100] = np.sort(rng.choice(N, size=100, replace=False))
    ids[1, :] = np.sort(rng.choice(N, size=k, replace=False))
    ids[1, 3] = N                          # first id past the cache
    ids[1, 64:72] = N + np.arange(8)       # a whole wave's 8 rows of one tile
    ids[1, 130] = (1 << 31) - 1
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    if fmt == "bf16":
        cache = _bf16(seed, synth.T_CACHE, (B, N, D))
        win = _bf16(seed, synth.T_WIN, (B, W, D))
        c64, w64 = F.bf16_to_f64(cache), F.bf16_to_f64(win)
        args, extra, tol = (to_dev_bf16(cache), to_dev_bf16(win)), {}, 2e-2
    else:
        cache = synth.fp8_codes(synth.stream_key(seed, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
        cs = synth.pos_scale(synth.stream_key(seed, synth.T_CACHE_SCALE), 0, B * N).reshape(B, N)
        win = synth.fp8_codes(synth.stream_key(seed, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
        wsc = synth.pos_scale(synth.stream_key(seed, synth.T_WIN_SCALE), 0, B * W).reshape(B, W)
        c64, w64 = F.decode_fp8_rows(cache, cs), F.decode_fp8_rows(win, wsc)
        args, extra, tol = (to_dev(cache), to_dev(win)), {"cache_scale": to_dev(cs), "window_scale": to_dev(wsc)}, 6e-2
    pos = np.array([321, 1 << 18], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    Q64 = F.bf16_to_f64(Q)
    ref = np.stack([M.attend(Q64[b], c64[b], ids[b][(ids[b] >= 0) & (ids[b] < N)], w64[b], tau, R, 10000.0, pos[b])
                    for b in range(B)])
    for splits in (0, 1, 3):
        O = cskv.attend(to_dev_bf16(Q), args[0], to_dev(ids), args[1], softmax_scale=tau, rope_dims=R,
                        q_pos=to_dev(pos), splits=splits, **extra)
        err = row_rel_err(O.cpu().numpy(), ref)
        assert err <= tol, (splits, err)
