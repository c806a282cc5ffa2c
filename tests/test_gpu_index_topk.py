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
    (2, 25600, 128, 64, 8, 256),     # 100 scoring chunks per sequence
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


@pytest.mark.parametrize("case", ["subnormal", "mantissas", "zero_nan"])
def test_topk_fp4_scale_codes(cskv, case):
    """Group-scale codes beyond powers of two, which the kernel decodes with the
    hardware E4M3 converter: subnormals (m * 2^-9), every mantissa of one
    exponent, both signs, zero and NaN (a NaN scale makes the entry's score NaN,
    which ranks below every number). Within a case the scales share one
    exponent range, so the fp32 sums are exact and the ids compare byte for
    byte."""
    B, N, Di, k = 2, 6000, 128, 512
    rng = np.random.default_rng({"subnormal": 11, "mantissas": 12, "zero_nan": 13}[case])
    q = synth.int_bf16(synth.stream_key(91, synth.T_QIDX), 0, B * Di, 8).reshape(B, Di)
    codes = rng.integers(0, 256, size=(B, N, Di // 2), dtype=np.uint8)
    shape = (B, N, Di // 16)
    sign = (rng.integers(0, 2, size=shape) << 7).astype(np.uint8)
    if case == "subnormal":
        sc = rng.integers(0, 8, size=shape).astype(np.uint8) | sign          # exponent field 0
    elif case == "mantissas":
        sc = np.uint8(7 << 3) | rng.integers(0, 8, size=shape).astype(np.uint8) | sign   # 1.0 .. 1.875
    else:
        pick = np.array([0x38, 0x40, 0xB8, 0x00, 0x80, 0x7F, 0xFF], dtype=np.uint8)   # 1, 2, -1, +-0, NaN
        sc = pick[rng.choice(len(pick), size=shape, p=[0.4, 0.3, 0.2, 0.04, 0.04, 0.01, 0.01])]
    for chunk in (0, 1024):
        ids = cskv.index_topk(to_dev_bf16(q), to_dev(codes), k, k_scale=to_dev(sc), chunk=chunk).cpu().numpy()
        for b in range(B):
            s = M.index_scores(F.bf16_to_f64(q[b]), F.decode_fp4_g16(codes[b], sc[b]))
            assert np.array_equal(ids[b], M.topk_ids(s, k)), (case, chunk, b)


def test_topk_ragged_entry_counts(cskv):
    B, N, Di, k = 6, 9000, 128, 512
    q, kk = _bf16_case(5, B, N, Di, 8)
    nv = np.array([9000, 0, 100, 512, 8191, 4097], dtype=np.int32)
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, n_entries=to_dev(nv), chunk=1024).cpu().numpy()
    assert np.array_equal(ids, _oracle_ids(q, kk, k, nv))


@pytest.mark.parametrize("B,N,chunk", [(8, 3000, 256), (16, 5000, 0), (8, 20000, 1024), (9, 3000, 256)])
def test_topk_batches_of_whole_xcd_rounds(cskv, B, N, chunk):
    """A batch that is a multiple of 8 runs a one-dimensional grid whose ids put
    each sequence's chunks on one XCD (B = 9 keeps the two-dimensional grid):
    ids byte-exact against the oracle, with ragged counts (an empty sequence, a
    short one, a chunk boundary), twice on one workspace."""
    Di, k = 128, 512
    q, kk = _bf16_case(7000 + B * 10 + N // 1000, B, N, Di, 8)
    nv = np.array([N - 97 * b for b in range(B)], dtype=np.int32)
    nv[1], nv[2], nv[3] = 0, 300, min(N, 2 * max(chunk, 256))
    ref = _oracle_ids(q, kk, k, nv)
    for _ in range(2):
        ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, n_entries=to_dev(nv), chunk=chunk).cpu().numpy()
        assert np.array_equal(ids, ref)


def test_topk_short_sequences_leave_workspace_clear(cskv):
    """Calls on one workspace where some sequences hold no more than k entries,
    followed by calls where they hold more: every call must match the oracle
    (each call leaves the per-sequence histograms clear for the next)."""
    B, N, Di, k = 4, 6000, 128, 512
    q, kk = _bf16_case(11, B, N, Di, 8)
    for nv in ([512, 100, 6000, 0], [6000] * 4, [3000, 6000, 511, 513], [6000] * 4):
        nv = np.array(nv, dtype=np.int32)
        ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, n_entries=to_dev(nv), chunk=1024).cpu().numpy()
        assert np.array_equal(ids, _oracle_ids(q, kk, k, nv)), nv


def test_topk_no_entries(cskv):
    """n_max = 0: nothing is scored and every id is -1."""
    q, _ = _bf16_case(2, 2, 10, 128, 8)
    kk = np.zeros((2, 0, 128), dtype=np.uint16)
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), 16).cpu().numpy()
    assert ids.shape == (2, 16) and (ids == -1).all()


def test_topk_tie_groups(cskv):
    """Exact ties at the k-th score, spread over many chunks: a small group
    (ranked pairwise) and a group larger than 256 (radix select)."""
    B, N, Di = 2, 20000, 128
    rng = np.random.default_rng(17)
    q = np.zeros((B, Di), dtype=np.uint16)
    q[:, 0] = F.f32_to_bf16(np.float32(1.0))
    kk = np.zeros((B, N, Di), dtype=np.uint16)
    val = lambda x: F.f32_to_bf16(np.float32(x))
    kk[:, :, 0] = val(1.0)
    top = rng.choice(N, 130, replace=False)
    kk[0, top[:30], 0] = val(9.0)           # 30 above, then 100 tied at 5: take 20 of them
    kk[0, top[30:], 0] = val(5.0)
    many = rng.choice(N, 1000, replace=False)
    kk[1, many[:10], 0] = val(9.0)          # 10 above, then 990 tied at 5: take 290 of them
    kk[1, many[10:], 0] = val(5.0)
    for k in (50, 300):
        ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k, chunk=512).cpu().numpy()
        assert np.array_equal(ids, _oracle_ids(q, kk, k)), k


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


def test_topk_ties_beyond_lds_capacity(cskv):
    """Tens of thousands of entries share the threshold bin, more than the
    selection gathers into LDS: it runs from global memory instead and must
    still be exact."""
    B, N, Di, k = 2, 40000, 128, 512
    q = np.full((B, Di), F.f32_to_bf16(np.float32(1.0)), dtype=np.uint16)
    kk = np.zeros((B, N, Di), dtype=np.uint16)
    one = F.f32_to_bf16(np.float32(1.0))
    kk[0, 39000:39100, 0] = one                    # 100 entries score 1, the rest 0
    kk[1, 5:9, 0] = F.f32_to_bf16(np.float32(-1.0))
    ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k).cpu().numpy()
    assert np.array_equal(ids, _oracle_ids(q, kk, k))
    assert np.array_equal(ids[0], np.concatenate([np.arange(412), np.arange(39000, 39100)]).astype(np.int32))


def test_topk_workspace_reuse_across_shapes(cskv):
    """Calls with changing shapes and interleaved attend calls: every result
    must match the oracle (the workspace state is rebuilt when the shape changes)."""
    shapes = [(2, 5000, 128, 512), (3, 9000, 128, 512), (2, 5000, 128, 512), (1, 70000, 32, 64),
              (2, 5000, 128, 512)]
    for i, (B, N, Di, k) in enumerate(shapes):
        q, kk = _bf16_case(900 + i, B, N, Di, 8)
        ids = cskv.index_topk(to_dev_bf16(q), to_dev_bf16(kk), k).cpu().numpy()
        assert np.array_equal(ids, _oracle_ids(q, kk, k)), (i, B, N)
        Q = torch.zeros((B, 16, 128), dtype=torch.bfloat16, device="cuda")
        cache = torch.zeros((B, 700, 128), dtype=torch.bfloat16, device="cuda")
        cskv.attend(Q, cache, None, None, softmax_scale=0.1, splits=4)


def _device_int_keys(seed, B, N, Di, a):
    from synth import device as sd
    q = sd.new((B, Di), synth.KIND_INT_BF16, synth.stream_key(seed, synth.T_QIDX), a=a)
    kk = sd.new((B, N, Di), synth.KIND_INT_BF16, synth.stream_key(seed, synth.T_KIDX), a=a)
    return q, kk


@pytest.mark.slow
def test_topk_full_size_c4a_128k_bf16(cskv):
    """The 128K bf16 workload at full size (32 sequences x 32767 entries, Di 128,
    top-512), in the launch configuration the benchmark uses; every sequence
    is regenerated on the host for the oracle."""
    from synth.configs import C4A_128K as w
    B, N, Di = w.B, w.n_entries, w.Di
    q_d, kk_d = _device_int_keys(w.seed, B, N, Di, w.idx_range)
    ids = cskv.index_topk(q_d, kk_d, w.k).cpu().numpy()
    kq, kk_ = synth.stream_key(w.seed, synth.T_QIDX), synth.stream_key(w.seed, synth.T_KIDX)
    for b in range(B):
        q = F.bf16_to_f64(synth.int_bf16(kq, b * Di, Di, w.idx_range))
        keys = F.bf16_to_f64(synth.int_bf16(kk_, b * N * Di, N * Di, w.idx_range).reshape(N, Di))
        assert np.array_equal(ids[b], M.topk_ids(M.index_scores(q, keys), w.k)), b
    assert np.all(np.diff(ids, axis=1) > 0)


@pytest.mark.slow
def test_topk_full_size_c4a_1m_fp4(cskv):
    """The 1M-context fp4 workload at full size (8 sequences x 262143 entries),
    every sequence checked."""
    from synth import device as sd
    from synth.configs import C4A_1M_Q as w
    B, N, Di = w.B, w.n_entries, w.Di
    kq = synth.stream_key(w.seed, synth.T_QIDX)
    kc = synth.stream_key(w.seed, synth.T_KIDX)
    ks = synth.stream_key(w.seed, synth.T_KIDX_SCALE)
    q_d = sd.new((B, Di), synth.KIND_INT_BF16, kq, a=w.idx_range)
    codes_d = sd.new((B, N, Di // 2), synth.KIND_BYTES, kc)
    sc_d = sd.new((B, N, Di // 16), synth.KIND_POW2_E4M3, ks, emin=-2, emax=2)
    ids = cskv.index_topk(q_d, codes_d, w.k, k_scale=sc_d).cpu().numpy()
    for b in range(B):
        q = F.bf16_to_f64(synth.int_bf16(kq, b * Di, Di, w.idx_range))
        codes = synth.random_bytes(kc, b * N * Di // 2, N * Di // 2).reshape(N, Di // 2)
        sc = synth.pow2_e4m3(ks, b * N * Di // 16, N * Di // 16, -2, 2).reshape(N, Di // 16)
        assert np.array_equal(ids[b], M.topk_ids(M.index_scores(q, F.decode_fp4_g16(codes, sc)), w.k)), b
