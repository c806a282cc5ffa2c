"""index_topk parity: ids must equal the oracle's bit for bit. Indexer values
are small integers (bf16) or fp4 codes with power-of-two scales against
integer queries, so every fp32 partial sum is exact on both sides."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import method as M
from tests.helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def _bf16_case(seed, B, N, Di, a):
    q = synth.int_bf16(synth.stream_key(seed, synth.T_QIDX), 0, B * Di, a).reshape(B, Di)
    kk = synth.int_bf16(synth.stream_key(seed, synth.T_KIDX), 0, B * N * Di, a).reshape(B, N, Di)
    return q, kk


def _oracle_ids(q, kk, k, n_valid=None):
    B = q.shape[0]
    out = []
    for b in range(B):
        s = M.index_scores(F.bf16_to_f64(q[b]), F.bf16_to_f64(kk[b]))
        out.append(M.topk_ids(s, k, None if n_valid is None else int(n_valid[b])))
    return np.stack(out)


@pytest.mark.parametrize("B,N,Di,k,a,chunk", [
    (1, 511, 32, 64, 4, 0),          # the tiny workload's shape
    (3, 5000, 128, 512, 8, 1024),    # several chunks and a ragged tail
    (2, 33000, 128, 512, 8, 0),      # automatic chunking
    (2, 25600, 128, 64, 8, 256),     # three selection levels (100 chunks -> 2 lists -> 1)
    (4, 777, 128, 2048, 8, 256),     # k larger than N: -1 padding
    (2, 4096, 32, 100, 1, 512),      # values in [-1, 1]: massive ties
])
def test_topk_bf16_matches_oracle(cskv, B, N, Di, k, a, chunk):
    q, kk = _bf16_case(B * 1000 + N, B, N, Di, a)
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, chunk=chunk).cpu().numpy()
    assert np.array_equal(ids, _oracle_ids(q, kk, k))


def test_topk_fp4_matches_oracle(cskv):
    B, N, Di, k = 3, 20000, 128, 512
    seed = 77
    q = synth.int_bf16(synth.stream_key(seed, synth.T_QIDX), 0, B * Di, 8).reshape(B, Di)
    codes = synth.random_bytes(synth.stream_key(seed, synth.T_KIDX), 0, B * N * Di // 2).reshape(B, N, Di // 2)
    sc = synth.pow2_e4m3(synth.stream_key(seed, synth.T_KIDX_SCALE), 0, B * N * Di // 16, -2, 2).reshape(B, N, Di // 16)
    for chunk in (0, 2048):
        ids = cskv.index_topk(to_dev_bf16(q), to_dev(codes), k, k_scale=to_dev(sc), chunk=chunk).cpu().numpy()
        for b in range(B):
            s = M.index_scores(F.bf16_to_f64(q[b]), F.decode_fp4_g16(codes[b], sc[b]))
            assert np.array_equal(ids[b], M.topk_ids(s, k)), (chunk, b)


def test_topk_ragged_entry_counts(cskv):
    B, N, Di, k = 6, 9000, 128, 512
    q, kk = _bf16_case(5, B, N, Di, 8)
    nv = np.array([9000, 0, 100, 512, 8191, 4097], dtype=np.int32)
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, n_entries=to_dev(nv), chunk=1024).cpu().numpy()
    assert np.array_equal(ids, _oracle_ids(q, kk, k, nv))


def test_topk_all_equal_and_nan(cskv):
    B, N, Di, k = 2, 3000, 128, 300
    q = np.full((B, Di), F.f32_to_bf16(np.float32(1.0)), dtype=np.uint16)
    kk = np.zeros((B, N, Di), dtype=np.uint16)                      # every score is 0
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, chunk=512).cpu().numpy()
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (B, 1)))
    # NaN keys rank below everything, -inf included
    kk2 = kk.copy()
    kk2[:, :2000, 0] = 0x7FC0                                       # NaN
    kk2[:, 2000:2100, 0] = 0xFF80                                   # -inf
    kk2[:, 2200:, 0] = 0x7FC0                                       # NaN; 2100..2199 score 0
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk2), k, chunk=512).cpu().numpy()
    assert np.array_equal(ids, _oracle_ids(q, kk2, k))
    want = np.concatenate([np.arange(0, 100), np.arange(2000, 2200)]).astype(np.int32)
    assert np.array_equal(ids[0], want)


def test_topk_k_equals_n_and_deterministic(cskv):
    B, N, Di = 2, 1024, 128
    q, kk = _bf16_case(3, B, N, Di, 8)
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), N, chunk=256).cpu().numpy()
    assert np.array_equal(ids, np.tile(np.arange(N, dtype=np.int32), (B, 1)))
    q, kk = _bf16_case(4, B, 40000, Di, 8)
    a = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), 512).cpu().numpy()
    b = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), 512).cpu().numpy()
    assert np.array_equal(a, b)


def test_topk_rejects_bad_arguments(cskv):
    q, kk = _bf16_case(1, 1, 100, 128, 8)
    with pytest.raises(cskv.CskvError):
        cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), 4096)               # k > 2048
    with pytest.raises(cskv.CskvError):
        cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), 10, chunk=300)      # chunk not a multiple of 256
    q64 = np.zeros((1, 64), dtype=np.uint16)
    with pytest.raises(cskv.CskvError):
        cskv.index_topk(to_dev_bf16(q64), to_dev_bf16(np.zeros((1, 10, 64), dtype=np.uint16)), 4)
