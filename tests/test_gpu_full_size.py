"""Full-size checks in the benchmark's own launch configuration.

* c4a workloads: one decode step (index_topk, then attend) on inputs built
  exactly as the benchmark builds them, caches compressed from the states by
  the library. For sampled sequences the host regenerates what the oracle
  needs: the indexer keys for its own top-k, and the 8 states of each entry it
  selects.
* c128a workloads: the dense attend over a cache of the full shape drawn
  directly (the host cannot regenerate 2^20 states per sequence in a test's
  time), and sampled entries of the caches the benchmark compresses from its
  states, in every row format.
"""
import argparse

import numpy as np
import pytest
import torch

import bench
import synth
from oracle import formats as F
from oracle import method as M
from synth import configs
from synth import device as sd
from tests.helpers import bf16_bits, row_rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _cfg(name):
    return next(w for w in configs.ALL if w.name == name)


def _args():
    return argparse.Namespace(chunk=0, splits=0, repeats=0)


def _c4a_oracle(wl, b):
    """Oracle ids and attention output of sequence b of a c4a workload."""
    c = wl.cfg
    key = lambda tensor: wl.key(0, tensor)  # noqa: E731
    L, D, H, N, Di, W = c.L, c.D, c.H, c.n_entries, c.Di, c.W
    q = F.bf16_to_f64(synth.int_bf16(key(synth.T_QIDX), b * Di, Di, c.idx_range))
    if c.key_dtype == "fp4":
        codes = synth.random_bytes(key(synth.T_KIDX), b * N * Di // 2, N * Di // 2).reshape(N, Di // 2)
        sc = synth.pow2_e4m3(key(synth.T_KIDX_SCALE), b * N * Di // 16, N * Di // 16, -2, 2).reshape(N, Di // 16)
        keys = F.decode_fp4_g16(codes, sc)
    else:
        keys = F.bf16_to_f64(synth.int_bf16(key(synth.T_KIDX), b * N * Di, N * Di, c.idx_range).reshape(N, Di))
    ids = M.topk_ids(M.index_scores(q, keys), c.k)
    # entry e folds states 4e .. 4e+7 of the sequence
    kS, kG = key(synth.T_S), key(synth.T_GATE)
    sel = ids[ids >= 0]
    ent = np.stack([
        M.compress("c4a", F.bf16_to_f64(synth.normal_bf16(kS, (b * L + 4 * int(e)) * D, 8 * D).reshape(8, D)),
                   synth.normal_f32(kG, b * L + 4 * int(e), 8).astype(np.float64))[0]
        for e in sel])
    tail = synth.normal_bf16(kS, (b * L + L - W) * D, W * D).reshape(W, D)
    cache = np.zeros((N, D))
    if c.cache_dtype == "fp8":
        # the cache and the window hold fp8 rows with a row scale
        rc, rs = F.encode_fp8_rows(ent.astype(np.float32))
        cache[sel] = F.decode_fp8_rows(rc, rs)
        wc, ws = F.encode_fp8_rows(F.bf16_to_f64(tail).astype(np.float32))
        win = F.decode_fp8_rows(wc, ws)
    else:
        cache[sel] = F.bf16_to_f64(F.f32_to_bf16(ent.astype(np.float32)))   # the cache stores bf16
        win = F.bf16_to_f64(tail)
    Q = F.bf16_to_f64(synth.normal_bf16(key(synth.T_Q), b * H * D, H * D).reshape(H, D))
    return ids, M.attend(Q, cache, ids, win, c.tau, c.R, c.rope_base, c.q_pos)


@pytest.mark.parametrize("name", ["c4a_128k_bf16", "c4a_1m_fp8_fp4"])
def test_c4a_step_full_size(cskv, name):
    """c4a 128K bf16 (32 x 32,767 entries) and c4a 1M fp8 cache + fp4 keys
    (8 x 262,143 entries): one step; the first, a middle and the last sequence."""
    cfg = _cfg(name)
    wl = bench.C4aLayer(cfg, _args(), torch, cskv, sd, synth)
    wl.setup(1)
    st = wl.sets[0]
    wl.dominant(st)
    wl.rest(st)
    torch.cuda.synchronize()
    ids_gpu = st["ids"].cpu().numpy()
    O = st["O"].cpu().numpy()
    tol = 2e-2 if cfg.cache_dtype == "bf16" else 6e-2
    for b in (0, cfg.B // 2, cfg.B - 1):
        ids, ref = _c4a_oracle(wl, b)
        assert np.array_equal(ids_gpu[b], ids), b
        err = row_rel_err(O[b], ref)
        assert err <= tol, (name, b, err)


def test_c128a_dense_attend_full_size(cskv):
    """Dense attend at the c128a 1M shape (16 sequences x 8,192 entries + 128
    window rows), automatic splits as in the benchmark, over drawn rows."""
    cfg = _cfg("c128a_1m_bf16")
    B, N, D, H, W = cfg.B, cfg.n_entries, cfg.D, cfg.H, cfg.W
    kc = synth.stream_key(cfg.seed, synth.T_CACHE)
    kw = synth.stream_key(cfg.seed, synth.T_WIN)
    kq = synth.stream_key(cfg.seed, synth.T_Q)
    cache = sd.new((B, N, D), synth.KIND_NORMAL_BF16, kc)
    win = sd.new((B, W, D), synth.KIND_NORMAL_BF16, kw)
    Q = sd.new((B, H, D), synth.KIND_NORMAL_BF16, kq)
    pos = torch.full((B,), cfg.q_pos, dtype=torch.int64, device="cuda")
    O = cskv.attend(Q, cache, None, win, softmax_scale=cfg.tau, rope_dims=cfg.R, rope_base=cfg.rope_base,
                    q_pos=pos).cpu().numpy()
    for b in (0, B // 2, B - 1):
        ch = F.bf16_to_f64(synth.normal_bf16(kc, b * N * D, N * D).reshape(N, D))
        wh = F.bf16_to_f64(synth.normal_bf16(kw, b * W * D, W * D).reshape(W, D))
        qh = F.bf16_to_f64(synth.normal_bf16(kq, b * H * D, H * D).reshape(H, D))
        ref = M.attend(qh, ch, None, wh, cfg.tau, cfg.R, cfg.rope_base, cfg.q_pos)
        err = row_rel_err(O[b], ref)
        assert err <= 2e-2, (b, err)


@pytest.mark.parametrize("name", ["c128a_1m_bf16", "c128a_1m_mixed", "c128a_1m_fp4"])
def test_c128a_entries_full_size(cskv, name):
    """The c128a 1M caches the benchmark compresses from 2^20 states per
    sequence, in bf16, mixed and fp4 rows: sampled entries of the first, a
    middle and the last sequence against the oracle's fold of their 128 states, and the
    window rows (the last 128 states, copied)."""
    cfg = _cfg(name)
    wl = bench.C128aLayer(cfg, _args(), torch, cskv, sd, synth)
    wl.setup(1)
    st = wl.sets[0]
    torch.cuda.synchronize()
    B, L, N, D, R, W = cfg.B, cfg.L, cfg.n_entries, cfg.D, cfg.R, cfg.W
    kS, kG = wl.key(0, synth.T_S), wl.key(0, synth.T_GATE)
    for b in (0, B // 2, B - 1):
        rows = bf16_bits(st["cache"][b]) if cfg.cache_dtype == "bf16" else st["cache"][b].cpu().numpy()
        scale = st["cscale"][b].cpu().numpy() if st["cscale"] is not None else None
        for e in (0, 1, N // 2, N - 1):
            S = F.bf16_to_f64(synth.normal_bf16(kS, (b * L + 128 * e) * D, 128 * D).reshape(128, D))
            g = synth.normal_f32(kG, b * L + 128 * e, 128).astype(np.float64)
            ref = M.compress("c128a", S, g)
            if cfg.cache_dtype == "mixed":
                row = rows[e:e + 1]
                codes, rope = row[:, : D - R], row[:, D - R:].copy().view(np.uint16)
                dec = F.decode_mixed_rows(codes, rope, scale[e:e + 1])
                assert row_rel_err(dec, ref) <= 6e-2, (name, b, e)
                assert row_rel_err(dec[:, D - R:], ref[:, D - R:]) <= 4e-3, (name, b, e)
            elif cfg.cache_dtype == "fp4":
                dec = F.decode_fp4_rows(rows[e:e + 1], D)
                assert row_rel_err(dec, ref) <= 0.35, (name, b, e)
                # within one code step of the oracle's own encoding of its entry
                rp, rs = F.encode_fp4_g16(ref.astype(np.float32))
                flips = int(np.sum(F.unpack_fp4(rows[e:e + 1, : D // 2]) != F.unpack_fp4(rp)))
                assert flips <= 8, (name, b, e, flips)
            else:
                got = F.bf16_to_f64(rows[e:e + 1])
                assert row_rel_err(got, ref) <= 4e-3, (name, b, e)
        tail = synth.normal_bf16(kS, (b * L + L - W) * D, W * D).reshape(W, D)
        assert np.array_equal(bf16_bits(st["win"][b]), tail), (name, b)
