"""Decode-step attention over compressed shared-K/V caches, for MI355X (gfx950).

The path (compress or the streaming append -> index_topk -> attend, with
fp8/fp4 cache codecs) runs in hand-written HIP kernels inside libcskv.so; this
package is a thin ctypes binding over its C ABI (include/cskv.h). PyTorch only provides device memory
and the current stream.
"""
from ._lib import (  # noqa: F401
    BF16, C128A, C4A, EHIP, EINVAL, EUNSUPPORTED, F32, FP4_E2M1, FP8_E4M3, FP8_ROPE64, LIB_PATH, MIX_ROPE, OK,
    CskvError, append, attend, attend_noalloc, attend_window_partial, compress, decode_fp4_g16, decode_fp8_rows,
    encode_fp4_g16, partial_bytes,
    encode_fp8_rows, index_topk, raw, version,
)
