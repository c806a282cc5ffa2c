"""The C ABI without a GPU: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments on the host
before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cskv.h")


@pytest.fixture(scope="module")
def lib():
    from compressed_sparse_kv_compress_amd import _lib
    return _lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cskv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib._lib, n), n
    assert sorted(lib.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert lib.version() == 100
    assert lib._lib_status_string(-1) == b"invalid argument"
    assert lib._lib_status_string(0) == b"ok"


def test_topk_workspace_sizes(lib):
    # 32 x 32767 entries, k = 512: a 4096-bin histogram per sequence and room
    # for every entry as a candidate (key + entry number), padded to whole
    # chunks, plus a candidate count per chunk and wave
    B, N = 32, 32767
    ws = lib._lib_topk_ws(B, N, 128, 512, lib.BF16, 0)
    need = B * (4096 * 4 + 2 * N * 4)
    assert need <= ws <= need + B * (2 * 16384 * 4 + 4096 * 4) + 64 * 1024
    # a single entry still needs the histogram and counter
    assert lib._lib_topk_ws(1, 1, 32, 64, lib.BF16, 0) >= 4096 * 4 + 4
    # the size grows with the batch
    assert lib._lib_topk_ws(64, N, 128, 512, lib.BF16, 0) > ws
    # rejected shapes report 0
    assert lib._lib_topk_ws(1, 100, 64, 8, lib.BF16, 0) == 0
    assert lib._lib_topk_ws(1, 100, 128, 4096, lib.BF16, 0) == 0
    # a sequence may span at most 2048 scoring chunks
    assert lib._lib_topk_ws(1, 2048 * 256, 128, 512, lib.BF16, 256) > 0
    assert lib._lib_topk_ws(1, 2048 * 256 + 1, 128, 512, lib.BF16, 256) == 0
    assert lib._lib_topk_ws(1, 2048 * 16384, 128, 512, lib.BF16, 0) > 0
    assert lib._lib_topk_ws(1, 2048 * 16384 + 1, 128, 512, lib.BF16, 0) == 0


def test_attend_workspace_sizes(lib):
    assert lib._lib_attend_ws(8, 64, 512, 640, 1) == 0
    # bf16 partials plus an fp32 (max, sum) pair per head and split
    assert lib._lib_attend_ws(8, 64, 512, 640, 4) == 8 * 4 * 64 * (512 * 2 + 8)
    assert lib._lib_attend_ws(8, 64, 384, 640, 4) == 0           # unsupported D


def test_compress_validation(lib):
    p = ctypes.c_void_p(16)           # never dereferenced: every call below is rejected first
    assert lib._lib_compress(7, p, p, 1, 64, 512, 0, lib.BF16, p, None, 100, None) == lib.EINVAL
    assert lib._lib_compress(0, p, p, 1, 64, 384, 0, lib.BF16, p, None, 100, None) == lib.EUNSUPPORTED
    assert lib._lib_compress(0, p, p, 1, 64, 512, 0, lib.BF16, p, None, 10, None) == lib.EINVAL   # 15 entries
    assert b"do not fit" in lib._lib_last_error()
    assert lib._lib_compress(0, None, p, 1, 64, 512, 0, lib.BF16, p, None, 100, None) == lib.EINVAL
    assert lib._lib_compress(0, p, p, 1, 64, 512, 0, lib.FP8_E4M3, p, None, 100, None) == lib.EINVAL
    assert lib._lib_compress(0, ctypes.c_void_p(18), p, 1, 64, 512, 0, lib.BF16, p, None, 100, None) == lib.EINVAL
    # nothing to do is not an error
    assert lib._lib_compress(0, None, None, 1, 7, 512, 0, lib.BF16, None, None, 0, None) == lib.OK
    assert lib._lib_compress(1, None, None, 0, 4096, 512, 0, lib.BF16, None, None, 32, None) == lib.OK


def test_append_validation(lib):
    p = ctypes.c_void_p(256)          # never dereferenced: every call below is rejected first
    f = lib._lib_append

    def call(**kw):
        a = dict(kind=0, s=p, g=p, pos=p, B=2, D=512, ring=p, rg=p, W=128, cdt=lib.BF16, cache=p, cs=None,
                 rows=64, ne=None, nw=None, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(kind=3) == lib.EINVAL
    assert call(D=384) == lib.EUNSUPPORTED
    assert call(cdt=9) == lib.EUNSUPPORTED
    assert call(cdt=lib.FP4_E2M1, D=128) == lib.EUNSUPPORTED      # fp4 rows: D = 512 only
    assert call(cdt=lib.FP8_ROPE64, D=128) == lib.EUNSUPPORTED    # mixed rows: D = 512 only
    assert call(W=7) == lib.EINVAL                          # a c4a entry needs 8 states
    assert call(kind=1, W=127) == lib.EINVAL                # a c128a entry needs 128
    assert b"W=127" in lib._lib_last_error()
    assert call(pos=None) == lib.EINVAL
    assert call(cdt=lib.FP8_E4M3) == lib.EINVAL             # fp8 cache without scales
    assert call(ring=ctypes.c_void_p(264)) == lib.EINVAL    # misaligned
    assert call(rows=-1) == lib.EINVAL
    assert call(B=0, s=None, g=None, pos=None, ring=None, rg=None, cache=None) == lib.OK


def test_topk_validation(lib):
    p = ctypes.c_void_p(256)
    f = lib._lib_topk
    assert f(p, lib.BF16, p, None, None, 1, 100, 128, 0, p, 0, None, 0, None) == lib.EINVAL          # k = 0
    assert f(p, lib.BF16, p, None, None, 1, 100, 128, 4096, p, 0, None, 0, None) == lib.EUNSUPPORTED
    assert f(p, lib.BF16, p, None, None, 1, 100, 96, 8, p, 0, None, 0, None) == lib.EUNSUPPORTED      # Di
    assert f(p, lib.FP4_E2M1, p, None, None, 1, 100, 128, 8, p, 0, None, 0, None) == lib.EINVAL       # no scales
    assert f(p, lib.BF16, p, None, None, 1, 100, 128, 8, p, 100, None, 0, None) == lib.EINVAL         # chunk
    assert f(None, lib.BF16, p, None, None, 1, 100, 128, 8, p, 0, None, 0, None) == lib.EINVAL
    # too small a workspace
    assert f(p, lib.BF16, p, None, None, 4, 100000, 128, 512, p, 0, p, 16, None) == lib.EINVAL
    assert b"workspace" in lib._lib_last_error()


def test_attend_validation(lib):
    p = ctypes.c_void_p(256)
    f = lib._lib_attend

    def call(**kw):
        a = dict(Q=p, B=1, H=64, D=512, cdt=lib.BF16, cache=p, cs=None, rows=10, ids=p, k=4, ne=None,
                 wdt=lib.BF16, win=p, ws_=None, W=4, wst=4, nw=None, R=64, base=10000.0, pos=p, tau=0.1, O=p,
                 splits=1, work=None, wsb=0, stream=None)
        a.update(kw)
        return f(*a.values())

    # only calls rejected on the host are made here (a valid one would launch)
    assert call(H=65) == lib.EUNSUPPORTED
    assert call(D=256) == lib.EUNSUPPORTED
    assert call(R=63) == lib.EINVAL
    assert call(R=1024) == lib.EINVAL
    assert call(wst=3) == lib.EINVAL
    assert call(cdt=lib.FP8_E4M3) == lib.EINVAL            # fp8 cache without scales
    assert call(cdt=lib.FP8_ROPE64) == lib.EINVAL          # mixed rows without scales
    assert call(cdt=lib.FP4_E2M1, D=128) == lib.EUNSUPPORTED
    assert call(wdt=lib.FP8_E4M3) == lib.EINVAL
    assert call(pos=None) == lib.EINVAL
    assert call(Q=ctypes.c_void_p(8)) == lib.EINVAL        # misaligned
    assert call(k=4000, splits=4, work=None, wsb=0) == lib.EINVAL  # needs a workspace
    assert call(B=0) == lib.OK


def test_codec_validation(lib):
    p = ctypes.c_void_p(256)
    assert lib._lib_enc8(lib.BF16, p, 4, 100, p, p, None) == lib.EUNSUPPORTED
    assert lib._lib_enc8(lib.FP8_E4M3, p, 4, 128, p, p, None) == lib.EUNSUPPORTED
    assert lib._lib_enc4(lib.F32, p, 4, 24, p, p, None) == lib.EINVAL
    assert lib._lib_dec4(p, p, 4, 24, p, None) == lib.EINVAL
    assert lib._lib_enc8(lib.F32, None, 0, 128, None, None, None) == lib.OK


def test_attend_noalloc_validation(lib):
    """The no-allocation attend validates like attend and rejects, on the host,
    a call whose split partials would not fit the library's scratch array."""
    p = ctypes.c_void_p(256)
    f = lib._lib_attend_noalloc

    def call(**kw):
        a = dict(Q=p, B=1, H=64, D=512, cdt=lib.BF16, cache=p, cs=None, rows=10, ids=p, k=4, ne=None,
                 wdt=lib.BF16, win=p, ws_=None, W=4, wst=4, nw=None, R=64, base=10000.0, pos=p, tau=0.1, O=p,
                 splits=1, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(H=65) == lib.EUNSUPPORTED
    assert call(R=63) == lib.EINVAL
    assert call(cdt=lib.FP8_E4M3) == lib.EINVAL            # fp8 cache without scales
    # 4096 sequences x 64 splits of partials: far beyond the 32 MiB scratch
    assert call(B=4096, k=4000, splits=64) == lib.EUNSUPPORTED
    assert b"scratch" in lib._lib_last_error()
    assert call(B=0) == lib.OK


def test_attend_partial_sizes_and_validation(lib):
    """The overlap entry points: partial sizes, and host-side argument checks
    (null or misaligned partial, unsupported shapes) before any launch."""
    assert lib._lib_partial_bytes(32, 64, 512) == 32 * 64 * (512 + 2) * 4
    assert lib._lib_partial_bytes(1, 8, 128) == 8 * 130 * 4
    assert lib._lib_partial_bytes(1, 65, 512) == 0 and lib._lib_partial_bytes(1, 8, 384) == 0
    p = ctypes.c_void_p(256)
    f = lib._lib_attend_part

    def call(**kw):
        a = dict(Q=p, B=1, H=64, D=512, cdt=lib.BF16, cache=p, cs=None, rows=10, ids=p, k=4, ne=None,
                 wdt=lib.BF16, win=None, ws_=None, W=0, wst=0, nw=None, R=64, base=10000.0, pos=p, tau=0.1,
                 part=p, O=p, splits=1, ws=None, wsb=0, stream=None)
        a.update(kw)
        return f(*a.values())

    assert call(part=None) == lib.EINVAL
    assert call(part=ctypes.c_void_p(264)) == lib.EINVAL         # not 16-byte aligned
    assert call(H=65) == lib.EUNSUPPORTED
    assert call(B=0, part=None) == lib.OK
    g = lib._lib_window_partial
    assert g(p, 1, 64, 384, lib.BF16, p, None, 4, 4, None, 0.1, p, None) == lib.EUNSUPPORTED
    assert g(p, 1, 64, 512, lib.FP8_E4M3, p, None, 4, 4, None, 0.1, p, None) == lib.EINVAL   # no window scales
    assert g(p, 1, 64, 512, lib.BF16, p, None, 4, 4, None, 0.1, None, None) == lib.EINVAL    # no partial
