"""Mixed-precision attention rows (the 64 rotary channels in bf16, the other
448 in fp8 with a per-token scale) through the C ABI: compress and the
streaming append write them, attend reads them; against the oracle's codec and
attention on the same bytes, and against the GPU's own bf16 rows where the
arithmetic is the same."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import method as M
from tests.helpers import bf16_bits, bf16_f64, row_rel_err, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
D, R = 512, 64


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _split(rows_u8):
    """GPU mixed rows [..., 576] -> (codes [..., 448], rotary bf16 bits [..., 64])."""
    rows_u8 = np.ascontiguousarray(rows_u8)
    return rows_u8[..., : D - R], rows_u8[..., D - R:].copy().view("<u2")


def _states(seed, B, T):
    S = synth.normal_bf16(synth.stream_key(seed, synth.T_S), 0, B * T * D).reshape(B, T, D)
    g = (synth.normal_f32(synth.stream_key(seed, synth.T_GATE), 0, B * T) * np.float32(2.0)).reshape(B, T)
    return S, g


@pytest.mark.parametrize("kind,T", [("c4a", 1030), ("c128a", 640)])
def test_compress_mixed_rows(cskv, kind, T):
    B = 3
    S, g = _states(40 + T, B, T)
    S[1, :, : D - R] = 0                   # a sequence whose fp8 part is all zero (scale 1)
    n = M.entry_count(kind, T)
    mix = torch.zeros((B, n, D + R), dtype=torch.uint8, device="cuda")
    msc = torch.zeros((B, n), dtype=torch.float32, device="cuda")
    ref16 = torch.zeros((B, n, D), dtype=torch.bfloat16, device="cuda")
    assert cskv.compress(kind, to_dev_bf16(S), to_dev(g), mix, msc) == n
    cskv.compress(kind, to_dev_bf16(S), to_dev(g), ref16)
    codes, rope = _split(mix.cpu().numpy())
    sc = msc.cpu().numpy()
    # the rotary channels are the bf16 entry's own bits (same fold, same rounding)
    assert np.array_equal(rope, bf16_bits(ref16)[..., D - R:])
    for b in range(B):
        ref = M.compress(kind, F.bf16_to_f64(S[b]), g[b].astype(np.float64))
        dec = F.decode_mixed_rows(codes[b], rope[b], sc[b])
        assert row_rel_err(dec, ref) <= 6e-2
        assert row_rel_err(dec[:, D - R:], ref[:, D - R:]) <= 4e-3
        # the scale covers the fp8 channels only: max |value| of the codes is 448
        if b == 1:
            assert np.all(sc[b] == 1.0) and np.all(codes[b] == 0)
        else:
            np.testing.assert_allclose(np.abs(F.e4m3_decode(codes[b])).max(axis=1), 448.0)


@pytest.mark.parametrize("kind,T", [("c4a", 90), ("c128a", 300)])
def test_append_mixed_rows_equal_compress(cskv, kind, T):
    """Appending one state at a time writes the same mixed rows as compressing
    the whole span (c128a: two complete entries and a partial block)."""
    B, W = 2, 128
    S, g = _states(55, B, T)
    n = M.entry_count(kind, T)
    mix = torch.zeros((B, n, D + R), dtype=torch.uint8, device="cuda")
    msc = torch.zeros((B, n), dtype=torch.float32, device="cuda")
    ring = torch.zeros((B, W, D), dtype=torch.bfloat16, device="cuda")
    rg = torch.zeros((B, W), dtype=torch.float32, device="cuda")
    Sd, gd = to_dev_bf16(S), to_dev(g)
    for p in range(T):
        cskv.append(kind, Sd[:, p].contiguous(), gd[:, p].contiguous(), torch.full((B,), p, dtype=torch.int64,
                    device="cuda"), ring, rg, mix, msc)
    ref = torch.zeros_like(mix)
    rsc = torch.zeros_like(msc)
    cskv.compress(kind, Sd, gd, ref, rsc)
    assert torch.equal(mix, ref) and torch.equal(msc, rsc)


@pytest.mark.parametrize("sparse,win_fp8", [(True, False), (False, False), (True, True)])
def test_attend_mixed_rows_matches_oracle(cskv, sparse, win_fp8):
    B, H, N, W, k = 3, 64, 700, 128, 96
    rng = np.random.default_rng(5 + sparse + 2 * win_fp8)
    x = synth.normal_f32(synth.stream_key(61, synth.T_CACHE), 0, B * N * D).reshape(B, N, D) * np.float32(1.5)
    codes, rope, scale = F.encode_mixed_rows(x, R)
    rows = F.mixed_row_bytes(codes, rope)                       # [B, N, 576]
    Q = synth.normal_bf16(synth.stream_key(62, synth.T_Q), 0, B * H * D).reshape(B, H, D)
    win = synth.normal_bf16(synth.stream_key(63, synth.T_WIN), 0, B * W * D).reshape(B, W, D)
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
                    cache_scale=to_dev(scale), window_scale=wsc_dev, softmax_scale=float(tau), rope_dims=R,
                    q_pos=to_dev(pos), n_entries=None if sparse else to_dev(n_ent)).cpu().numpy()
    dec = F.decode_mixed_rows(codes, rope, scale)
    for b in range(B):
        ref = M.attend(F.bf16_to_f64(Q[b]), dec[b], None if ids is None else ids[b], win_ref[b], tau, R, 10000.0,
                       int(pos[b]), n_entries=None if sparse else int(n_ent[b]))
        assert row_rel_err(O[b], ref) <= 2e-2
