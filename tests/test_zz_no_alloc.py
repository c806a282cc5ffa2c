"""cskv_attend_noalloc against cskv_attend: the same kernels with the split
partials in the library's per-device scratch array instead of a workspace.
Two calls in a row, the second with a smaller input, each compared with the
workspace entry point on the same inputs (bit for bit: same plan, same
kernels) and with the oracle (row-relative 2e-2)."""
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


def _case(cskv, seed, B, N, k, W, splits):
    H, D, R = 64, 512, 64
    Q = _bf16(seed, synth.T_Q, (B, H, D))
    cache = _bf16(seed, synth.T_CACHE, (B, N, D))
    win = _bf16(seed, synth.T_WIN, (B, W, D))
    rng = np.random.default_rng(seed)
    ids = None if k == 0 else np.stack([sorted_ids(rng, N, k, n_valid=k - (7 if b == 1 else 0)) for b in range(B)])
    pos = np.array([4000 + 131 * b for b in range(B)], dtype=np.int64)
    tau = 1 / np.sqrt(D)
    args = (to_dev_bf16(Q), to_dev_bf16(cache), None if ids is None else to_dev(ids), to_dev_bf16(win))
    kw = dict(softmax_scale=tau, rope_dims=R, q_pos=to_dev(pos), splits=splits)
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device="cuda")
    got = cskv.attend_noalloc(*args, out=out, **kw)
    want = cskv.attend(*args, **kw)
    torch.cuda.synchronize()
    got, want = got.cpu().numpy(), want.cpu().numpy()
    assert np.array_equal(got, want)
    ref = np.stack([M.attend(F.bf16_to_f64(Q[b]), F.bf16_to_f64(cache[b]), None if ids is None else ids[b],
                             F.bf16_to_f64(win[b]), tau, R, 10000.0, pos[b]) for b in range(B)])
    assert row_rel_err(got, ref) <= 2e-2


def test_attend_noalloc_two_calls_second_smaller(cskv):
    # dense over 3000 entries in 12 splits (partials in the scratch), then a
    # smaller sparse call whose partials overwrite the start of it
    _case(cskv, 801, B=4, N=3000, k=0, W=128, splits=12)
    _case(cskv, 802, B=2, N=900, k=256, W=40, splits=3)


def test_attend_noalloc_rejects_oversized_plan(cskv):
    B, H, D = 600, 64, 512
    Q = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((B, 64, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cskv.CskvError, match="scratch"):
        cskv.attend_noalloc(Q, cache, None, None, softmax_scale=0.1, splits=2)
