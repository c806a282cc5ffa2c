"""fp4 attention-cache rows (E2M1 codes, one E4M3 scale byte per 16 channels,
288 B per 512-channel row) through the C ABI: compress and the streaming
append write them, attend widens them exactly; against the oracle's group
codec and attention on the same bytes."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import method as M
from tests.helpers import row_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
D, RB = 512, 288


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _states(seed, B, T):
    S = synth.normal_bf16(synth.stream_key(seed, synth.T_S), 0, B * T * D).reshape(B, T, D)
    g = (synth.normal_f32(synth.stream_key(seed, synth.T_GATE), 0, B * T) * np.float32(2.0)).reshape(B, T)
    return S, g


@pytest.mark.parametrize("kind,T", [("c4a", 1030), ("c128a", 640)])
def test_compress_fp4_rows(cskv, kind, T):
    B = 2
    S, g = _states(70 + T, B, T)
    n = M.entry_count(kind, T)
    rows = torch.zeros((B, n, RB), dtype=torch.uint8, device="cuda")
    assert cskv.compress(kind, to_dev_bf16(S), to_dev(g), rows) == n
    got = rows.cpu().numpy()
    flips = scale_flips = 0
    for b in range(B):
        ref = M.compress(kind, F.bf16_to_f64(S[b]), g[b].astype(np.float64))
        # the group codec on the oracle's entries: the same codes and scales
        # except where the two fp32 sums round differently next to a boundary
        rp, rs = F.encode_fp4_g16(ref.astype(np.float32))
        flips += int(np.sum(F.unpack_fp4(got[b, :, :256]) != F.unpack_fp4(rp)))
        scale_flips += int(np.sum(got[b, :, 256:] != rs))
        # and the decoded rows are within the 4-bit codec's own error of the entries
        dec = F.decode_fp4_rows(got[b], D)
        assert row_rel_err(dec, ref) <= 0.35
        assert np.array_equal(dec, F.decode_fp4_rows(F.fp4_row_bytes(rp, rs), D)) or flips > 0
    assert flips <= 0.01 * B * n * D and scale_flips <= 0.01 * B * n * (D // 16)


@pytest.mark.parametrize("kind,T", [("c4a", 90), ("c128a", 300)])
def test_append_fp4_rows_equal_compress(cskv, kind, T):
    """Appending one state at a time writes the same fp4 rows as compressing
    the whole span (c128a: two complete entries and a partial block)."""
    B, W = 2, 128
    S, g = _states(75, B, T)
    n = M.entry_count(kind, T)
    rows = torch.zeros((B, n, RB), dtype=torch.uint8, device="cuda")
    ring = torch.zeros((B, W, D), dtype=torch.bfloat16, device="cuda")
    rg = torch.zeros((B, W), dtype=torch.float32, device="cuda")
    Sd, gd = to_dev_bf16(S), to_dev(g)
    for p in range(T):
        cskv.append(kind, Sd[:, p].contiguous(), gd[:, p].contiguous(),
                    torch.full((B,), p, dtype=torch.int64, device="cuda"), ring, rg, rows)
    ref = torch.zeros_like(rows)
    cskv.compress(kind, Sd, gd, ref)
    assert torch.equal(rows, ref)


@pytest.mark.parametrize("sparse,win_fp8", [(True, False), (False, False), (True, True)])
def test_attend_fp4_rows_matches_oracle(cskv, sparse, win_fp8):
    B, H, N, W, k, R = 3, 64, 700, 128, 96, 64
    rng = np.random.default_rng(15 + sparse + 2 * win_fp8)
    x = synth.normal_f32(synth.stream_key(71, synth.T_CACHE), 0, B * N * D).reshape(B, N, D) * np.float32(1.5)
    packed, sc = F.encode_fp4_g16(x)
    rows = F.fp4_row_bytes(packed, sc)                           # [B, N, 288]
    Q = synth.normal_bf16(synth.stream_key(72, synth.T_Q), 0, B * H * D).reshape(B, H, D)
    win = synth.normal_bf16(synth.stream_key(73, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    pos = rng.integers(10_000, 1 << 20, size=B).astype(np.int64)
    tau = 1.0 / np.sqrt(D)
    ids = np.stack([np.sort(rng.choice(N, size=k, replace=False)).astype(np.int32) for _ in range(B)]) if sparse else None
    n_ent = np.array([N, 123, 0], dtype=np.int32)
    if win_fp8:
        wc, ws = F.encode_fp8_rows(F.bf16_to_f64(win).astype(np.float32))
        win_dev, wsc_dev, win_ref = to_dev(wc), to_dev(ws), F.decode_fp8_rows(wc, ws)
    else:
        win_dev, wsc_dev, win_ref = to_dev_bf16(win), None, F.bf16_to_f64(win)
    O = cskv.attend(to_dev_bf16(Q), to_dev(rows), None if ids is None else to_dev(ids), win_dev,
                    window_scale=wsc_dev, softmax_scale=float(tau), rope_dims=R, q_pos=to_dev(pos),
                    n_entries=None if sparse else to_dev(n_ent)).cpu().numpy()
    dec = F.decode_fp4_rows(rows, D)
    for b in range(B):
        ref = M.attend(F.bf16_to_f64(Q[b]), dec[b], None if ids is None else ids[b], win_ref[b], tau, R, 10000.0,
                       int(pos[b]), n_entries=None if sparse else int(n_ent[b]))
        assert row_rel_err(O[b], ref) <= 2e-2


@pytest.mark.parametrize("fmt", ["fp4", "mixed"])
def test_attend_raw_rows_skip_invalid_ids(cskv, fmt):
    """-1 padding and ids past the cache read the zero row with a zero flag and
    stay out of the softmax (top-k pads with -1 when a sequence is short)."""
    B, H, N, W, k, R = 2, 64, 300, 16, 80, 64
    rng = np.random.default_rng(21)
    x = synth.normal_f32(synth.stream_key(81, synth.T_CACHE), 0, B * N * D).reshape(B, N, D)
    if fmt == "fp4":
        packed, sc = F.encode_fp4_g16(x)
        rows, cscale, dec = F.fp4_row_bytes(packed, sc), None, F.decode_fp4_g16(packed, sc)
    else:
        codes, rope, scale = F.encode_mixed_rows(x, R)
        rows, cscale, dec = F.mixed_row_bytes(codes, rope), to_dev(scale), F.decode_mixed_rows(codes, rope, scale)
    ids = np.full((B, k), -1, dtype=np.int32)
    ids[0, :50] = np.sort(rng.choice(N, size=50, replace=False))
    ids[1, :k] = np.sort(rng.choice(N, size=k, replace=False))
    ids[1, 7] = N + 5                      # out of range: skipped
    ids[1, 40] = 1 << 30
    Q = synth.normal_bf16(synth.stream_key(82, synth.T_Q), 0, B * H * D).reshape(B, H, D)
    win = synth.normal_bf16(synth.stream_key(83, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
    pos = np.array([5000, 77], dtype=np.int64)
    tau = 1.0 / np.sqrt(D)
    O = cskv.attend(to_dev_bf16(Q), to_dev(rows), to_dev(ids), to_dev_bf16(win), cache_scale=cscale,
                    softmax_scale=float(tau), rope_dims=R, q_pos=to_dev(pos)).cpu().numpy()
    for b in range(B):
        valid = ids[b][(ids[b] >= 0) & (ids[b] < N)]
        ref = M.attend(F.bf16_to_f64(Q[b]), dec[b], valid, F.bf16_to_f64(win[b]), tau, R, 10000.0, int(pos[b]))
        assert row_rel_err(O[b], ref) <= 2e-2
