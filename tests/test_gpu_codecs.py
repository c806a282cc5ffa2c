"""Codec and generator parity on the GPU: the device routines must give the
oracle's codes bit for bit on identical inputs, and the device input filler
must reproduce the host generator exactly."""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from tests.helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cskv():
    import compressed_sparse_kv_compress_amd as m
    return m


def test_fp8_decode_all_codes(cskv):
    codes = np.tile(np.arange(256, dtype=np.uint8), (4, 2))          # [4, 512]
    scale = np.array([1.0, 0.5, 3.0e-3, 7.25], dtype=np.float32)
    got = cskv.decode_fp8_rows(to_dev(codes), to_dev(scale)).cpu().numpy().astype(np.float64)
    # the decoder writes fp32: the exact product rounded once
    ref = F.decode_fp8_rows(codes, scale).astype(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def test_fp4_decode_all_bytes(cskv):
    rng = np.random.default_rng(1)
    packed = np.tile(np.arange(256, dtype=np.uint8), (2, 1)).reshape(8, 64)   # every byte value
    scales = rng.integers(0, 0x7F, size=(8, 8), dtype=np.uint8)               # finite E4M3 scales
    scales[0] = 0x38                                                          # 1.0
    got = cskv.decode_fp4_g16(to_dev(packed), to_dev(scales)).cpu().numpy().astype(np.float64)
    ref = F.decode_fp4_g16(packed, scales)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("D", [64, 128, 512, 1024])
def test_fp8_encode_bit_exact_f32(cskv, D):
    rng = np.random.default_rng(D)
    rows = 300
    x = (rng.standard_normal((rows, D)) * 2.0 ** rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :5] = [448.0, -1e-30, 3.0, -0.0, 2.0 ** -12]
    # values on E4M3 rounding midpoints after scaling by a power of two
    mids = (F.E4M3_TABLE[1:0x7E] + F.E4M3_TABLE[2:0x7F]) / 2
    x[2, : min(D, mids.size)] = mids[: min(D, mids.size)].astype(np.float32)
    x[2, -1] = 448.0
    codes, scale = cskv.encode_fp8_rows(to_dev(x))
    rc, rs = F.encode_fp8_rows(x)
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_fp8_encode_bit_exact_bf16(cskv):
    k = synth.stream_key(7, synth.T_MISC)
    bits = synth.normal_bf16(k, 0, 257 * 512).reshape(257, 512)
    codes, scale = cskv.encode_fp8_rows(to_dev_bf16(bits))
    rc, rs = F.encode_fp8_rows(F.bf16_to_f32(bits))
    assert np.array_equal(scale.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


@pytest.mark.parametrize("Di", [16, 32, 128])
def test_fp4_encode_bit_exact(cskv, Di):
    rng = np.random.default_rng(Di)
    rows = 513
    x = (rng.standard_normal((rows, Di)) * 2.0 ** rng.integers(-14, 12, (rows, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :16] = np.array([6, 3, 1.5, -0.5, 0, 4, -6, 2, 1, -1, 0.5, -3, -4, 1.5, -2, 0.25], dtype=np.float32)
    x[2] = 1e-12                      # scale underflows to zero: raised to the smallest subnormal
    packed, scales = cskv.encode_fp4_g16(to_dev(x))
    rp, rsc = F.encode_fp4_g16(x)
    assert np.array_equal(scales.cpu().numpy(), rsc)
    assert np.array_equal(packed.cpu().numpy(), rp)


def test_device_filler_matches_host():
    from synth import device as sd
    key = synth.stream_key(0xABC, 3, 5)
    cases = [
        (synth.KIND_NORMAL_F32, {}, torch.float32, lambda o, n: synth.normal_f32(key, o, n)),
        (synth.KIND_NORMAL_BF16, {}, torch.bfloat16, lambda o, n: synth.normal_bf16(key, o, n)),
        (synth.KIND_INT_BF16, {"a": 8}, torch.bfloat16, lambda o, n: synth.int_bf16(key, o, n, 8)),
        (synth.KIND_BYTES, {}, torch.uint8, lambda o, n: synth.random_bytes(key, o, n)),
        (synth.KIND_POW2_E4M3, {"emin": -2, "emax": 2}, torch.uint8, lambda o, n: synth.pow2_e4m3(key, o, n, -2, 2)),
        (synth.KIND_FP8_CODES, {}, torch.uint8, lambda o, n: synth.fp8_codes(key, o, n)),
        (synth.KIND_POS_SCALE, {}, torch.float32, lambda o, n: synth.pos_scale(key, o, n)),
    ]
    for kind, kw, dt, host in cases:
        for off, n in [(0, 10000), (123456789, 4097)]:
            t = torch.empty(n, dtype=dt, device="cuda")
            sd.fill(t, kind, key, offset=off, **kw)
            got = t.view(torch.int16).cpu().numpy().view(np.uint16) if dt == torch.bfloat16 else t.cpu().numpy()
            assert np.array_equal(got, host(off, n)), (kind, off)
