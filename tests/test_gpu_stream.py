"""Streaming decode parity: one state appended per sequence and step through
the C ABI (ragged positions, inactive sequences skipped), against the GPU's
own span compress (bit-identical entries) and the oracle's streaming append;
then a whole streaming decode step (append, index_topk over the ragged entry
counts, attend over the ring with its ragged window) against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import method as M
from tests.helpers import bf16_bits, bf16_f64, row_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _schedule(seed, B, steps, p_active=0.8):
    """pos [steps, B]: each sequence's next token position when it is active
    at a step, -1 when it sits the step out (ragged progress)."""
    rng = np.random.default_rng(seed)
    act = rng.random((steps, B)) < p_active
    act[:, 0] = True                     # one sequence advances every step
    if B > 2:
        act[:, B - 1] = False            # and one never does
    pos = np.full((steps, B), -1, dtype=np.int64)
    n = np.zeros(B, dtype=np.int64)
    for t in range(steps):
        pos[t, act[t]] = n[act[t]]
        n += act[t]
    return pos, n


def _run_stream(cskv, kind, S, g, pos, W, rows, fp8, n_entries=None, n_window=None):
    """Appends, step by step, S[b, pos[t, b]] for every active (t, b)."""
    steps, B = pos.shape
    D = S.shape[2]
    Sd, gd = to_dev_bf16(S), to_dev(g)
    ring = torch.zeros((B, W, D), dtype=torch.bfloat16, device="cuda")
    ring_gate = torch.zeros((B, W), dtype=torch.float32, device="cuda")
    if fp8:
        cache = torch.zeros((B, rows, D), dtype=torch.uint8, device="cuda")
        cscale = torch.zeros((B, rows), dtype=torch.float32, device="cuda")
    else:
        cache = torch.zeros((B, rows, D), dtype=torch.bfloat16, device="cuda")
        cscale = None
    bidx = np.arange(B)
    s_all = to_dev_bf16(S[bidx[None, :], np.maximum(pos, 0)])            # [steps, B, D]
    g_all = to_dev(g[bidx[None, :], np.maximum(pos, 0)].astype(np.float32))
    p_all = to_dev(pos)
    for t in range(steps):
        cskv.append(kind, s_all[t], g_all[t], p_all[t], ring, ring_gate, cache, cscale,
                    n_entries=n_entries, n_window=n_window)
    return ring, ring_gate, cache, cscale


def _tokens(seed, B, T, D):
    S = synth.normal_bf16(synth.stream_key(seed, synth.T_S), 0, B * T * D).reshape(B, T, D)
    g = (synth.normal_f32(synth.stream_key(seed, synth.T_GATE), 0, B * T) * np.float32(2.0)).reshape(B, T)
    return S, g


@pytest.mark.parametrize("kind,D,fp8,W,steps", [("c4a", 512, False, 128, 120), ("c4a", 128, True, 8, 90),
                                                ("c4a", 512, True, 13, 70), ("c128a", 512, False, 128, 330),
                                                ("c128a", 128, True, 200, 300)])
def test_append_matches_span_compress_and_oracle(cskv, kind, D, fp8, W, steps):
    B = 5
    pos, n_tok = _schedule(100 + steps, B, steps)
    S, g = _tokens(7 + D + W, B, steps, D)
    rows = M.entry_count(kind, steps) + 2
    n_ent = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_win = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ring, ring_gate, cache, cscale = _run_stream(cskv, kind, S, g, pos, W, rows, fp8, n_ent, n_win)
    torch.cuda.synchronize()
    ne, nw = n_ent.cpu().numpy(), n_win.cpu().numpy()
    rg = ring_gate.cpu().numpy()
    rb = bf16_bits(ring)
    for b in range(B):
        T = int(n_tok[b])
        n = M.entry_count(kind, T)
        # counts: the oracle's; a sequence that never appended keeps its own
        if T == 0:
            assert ne[b] == -7 and nw[b] == -7
        else:
            assert (ne[b], nw[b]) == M.stream_counts(kind, T - 1, W)
        # the ring holds the newest min(T, W) states and logits, bit for bit
        for p in range(max(0, T - W), T):
            assert np.array_equal(rb[b, p % W], S[b, p])
            assert rg[b, p % W] == g[b, p]
        if n == 0:
            continue
        # the GPU's span compress of the same states writes the same bytes
        if fp8:
            ref_c = torch.zeros((1, n, D), dtype=torch.uint8, device="cuda")
            ref_s = torch.zeros((1, n), dtype=torch.float32, device="cuda")
        else:
            ref_c = torch.zeros((1, n, D), dtype=torch.bfloat16, device="cuda")
            ref_s = None
        cskv.compress(kind, to_dev_bf16(S[b:b + 1, :T]), to_dev(g[b:b + 1, :T]), ref_c, ref_s)
        if fp8:
            assert torch.equal(cache[b, :n], ref_c[0]) and torch.equal(cscale[b, :n], ref_s[0])
            got = F.decode_fp8_rows(cache[b, :n].cpu().numpy(), cscale[b, :n].cpu().numpy())
            tol = 6e-2
        else:
            assert torch.equal(cache[b, :n].view(torch.int16), ref_c[0].view(torch.int16))
            got = bf16_f64(cache[b, :n])
            tol = 2e-2
        # and the oracle's streaming append agrees within the bar
        oring, org = np.zeros((W, D)), np.zeros(W)
        ref = {}
        for p in range(T):
            c, row = M.append(kind, oring, org, F.bf16_to_f64(S[b, p]), float(g[b, p]), p)
            if c is not None:
                ref[c] = row
        assert sorted(ref) == list(range(n))
        assert row_rel_err(got, np.stack([ref[c] for c in range(n)])) <= tol


def test_append_past_the_cache_drops_entries(cskv):
    B, D, W, T, rows = 2, 512, 16, 40, 3
    pos = np.stack([np.arange(T), np.arange(T)], axis=1).astype(np.int64)
    S, g = _tokens(5, B, T, D)
    n_ent = torch.zeros((B,), dtype=torch.int32, device="cuda")
    _, _, cache, _ = _run_stream(cskv, "c4a", S, g, pos, W, rows, False, n_ent)
    torch.cuda.synchronize()
    assert n_ent.cpu().numpy().tolist() == [rows, rows]        # 9 complete, 3 held
    ref = torch.zeros((B, M.entry_count("c4a", T), D), dtype=torch.bfloat16, device="cuda")
    cskv.compress("c4a", to_dev_bf16(S), to_dev(g), ref)
    assert torch.equal(cache.view(torch.int16), ref[:, :rows].contiguous().view(torch.int16))


@pytest.mark.parametrize("kind", ["c4a", "c128a"])
def test_stream_decode_step_matches_oracle(cskv, kind):
    """Ragged batch (one ring not yet full, others wrapped): append the newest
    state, then index_topk over n_entries and attend over the ring with
    n_window, each against the oracle on the GPU's own cache bytes."""
    B, D, H, R, W, Di, k = 4, 512, 64, 64, 128, 128, 64
    lens = np.array([9, 100, 383, 700] if kind == "c4a" else [130, 127, 400, 700], dtype=np.int64)
    steps = int(lens.max())
    pos = np.full((steps, B), -1, dtype=np.int64)
    for b in range(B):                    # sequence b appends its tokens in the last lens[b] steps
        pos[steps - lens[b]:, b] = np.arange(lens[b])
    S, g = _tokens(31, B, steps, D)
    rows = M.entry_count(kind, steps)
    n_ent = torch.zeros((B,), dtype=torch.int32, device="cuda")
    n_win = torch.zeros((B,), dtype=torch.int32, device="cuda")
    ring, _, cache, _ = _run_stream(cskv, kind, S, g, pos, W, rows, False, n_ent, n_win)
    q_pos = to_dev(lens - 1)
    rng = np.random.default_rng(3)
    Q = synth.normal_bf16(synth.stream_key(77, synth.T_Q), 0, B * H * D).reshape(B, H, D)
    tau = 1.0 / np.sqrt(D)
    if kind == "c4a":
        qi = rng.integers(-8, 9, size=(B, Di)).astype(np.float32)
        ki = rng.integers(-8, 9, size=(B, rows, Di)).astype(np.float32)
        ids = cskv.index_topk(to_dev(qi).to(torch.bfloat16), to_dev(ki).to(torch.bfloat16), k, n_entries=n_ent)
    else:
        ids = None
    O = cskv.attend(to_dev_bf16(Q), cache, ids, ring, softmax_scale=float(tau), rope_dims=R, q_pos=q_pos,
                    n_entries=n_ent if ids is None else None, n_window=n_win)
    torch.cuda.synchronize()
    ne, nw = n_ent.cpu().numpy(), n_win.cpu().numpy()
    cache_h, ring_h, O_h = bf16_f64(cache), bf16_f64(ring), O.cpu().numpy()
    ids_h = None if ids is None else ids.cpu().numpy()
    for b in range(B):
        assert (ne[b], nw[b]) == M.stream_counts(kind, int(lens[b]) - 1, W)
        if kind == "c4a":
            ref_ids = M.topk_ids(M.index_scores(qi[b], ki[b]), k, int(ne[b]))
            assert np.array_equal(ids_h[b], ref_ids)
            ref = M.attend(F.bf16_to_f64(Q[b]), cache_h[b], ref_ids, ring_h[b, :nw[b]], tau, R, 10000.0,
                           int(lens[b]) - 1)
        else:
            ref = M.attend(F.bf16_to_f64(Q[b]), cache_h[b], None, ring_h[b, :nw[b]], tau, R, 10000.0,
                           int(lens[b]) - 1, n_entries=int(ne[b]))
        assert row_rel_err(O_h[b], ref) <= 2e-2


@pytest.mark.parametrize("B", [4, 64])
def test_attend_ragged_window_counts(cskv, B):
    """n_window keeps the leading rows of each window (0, partial, all W), at a
    small batch (B = 4: several splits per sequence) and a large one (B = 64:
    one split per sequence, no merge)."""
    H, D, R, W, N, k = 64, 512, 64, 128, 300, 64
    rng = np.random.default_rng(8 + B)
    Q = synth.normal_bf16(synth.stream_key(90 + B, synth.T_Q), 0, B * H * D).reshape(B, H, D)
    cache = synth.normal_bf16(synth.stream_key(91 + B, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
    win = synth.normal_bf16(synth.stream_key(92 + B, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    ids = np.stack([np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32) for _ in range(B)])
    nw = rng.integers(0, W + 1, size=B).astype(np.int32)
    nw[0], nw[1 % B] = 0, W
    nw[2 % B] = -5                        # clamped to 0
    pos = rng.integers(1000, 5000, size=B).astype(np.int64)
    tau = 1.0 / np.sqrt(D)
    O = cskv.attend(to_dev_bf16(Q), to_dev_bf16(cache), to_dev(ids), to_dev_bf16(win), softmax_scale=float(tau),
                    rope_dims=R, q_pos=to_dev(pos), n_window=to_dev(nw)).cpu().numpy()
    for b in sorted(set(range(0, B, max(1, B // 8))) | {1 % B, 2 % B}):
        ref = M.attend(F.bf16_to_f64(Q[b]), F.bf16_to_f64(cache[b]), ids[b],
                       F.bf16_to_f64(win[b, :max(0, min(int(nw[b]), W))]), tau, R, 10000.0, int(pos[b]))
        assert row_rel_err(O[b], ref) <= 2e-2, b
