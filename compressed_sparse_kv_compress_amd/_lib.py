"""ctypes binding of libcskv.so: argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
checks tensor devices, dtypes and layouts, passes raw device pointers and the
current HIP stream, and turns non-zero statuses into exceptions. There is no
fallback: if the library is missing or fails to load, importing raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSKV_LIBRARY names another build of the same library (the host-sanitized
# build that the CPU tests of the argument checks load); default: in-tree
LIB_PATH = os.environ.get("CSKV_LIBRARY") or os.path.join(_HERE, "libcskv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python compressed_sparse_kv_compress_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3
BF16, F32, FP8_E4M3, FP4_E2M1, FP8_ROPE64 = 0, 1, 2, 3, 4
MIX_ROPE = 64   # rotary channels a mixed (FP8_ROPE64) cache row keeps in bf16
C4A, C128A = 0, 1
KINDS = {"c4a": C4A, "c128a": C128A, C4A: C4A, C128A: C128A}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_lib_status_string = _sig("cskv_status_string", ctypes.c_char_p, _i32)
_lib_last_error = _sig("cskv_last_error", ctypes.c_char_p)
_lib_version = _sig("cskv_version", _i32)
_lib_compress = _sig("cskv_compress", _i32, _i32, _p, _p, _i64, _i64, _i32, _i64, _i32, _p, _p, _i64, _p)
_lib_topk_ws = _sig("cskv_index_topk_workspace", _sz, _i64, _i64, _i32, _i32, _i32, _i32)
_lib_topk = _sig("cskv_index_topk", _i32, _p, _i32, _p, _p, _p, _i64, _i64, _i32, _i32, _p, _i32, _p, _sz, _p)
_lib_attend_ws = _sig("cskv_attend_workspace", _sz, _i64, _i32, _i32, _i64, _i32)
_lib_attend = _sig("cskv_attend", _i32, _p, _i64, _i32, _i32, _i32, _p, _p, _i64, _p, _i32, _p,
                   _i32, _p, _p, _i32, _i64, _p, _i32, _f32, _p, _f32, _p, _i32, _p, _sz, _p)
_lib_attend_noalloc = _sig("cskv_attend_noalloc", _i32, _p, _i64, _i32, _i32, _i32, _p, _p, _i64, _p, _i32, _p,
                           _i32, _p, _p, _i32, _i64, _p, _i32, _f32, _p, _f32, _p, _i32, _p)
_lib_attend_part = _sig("cskv_attend_with_partial", _i32, _p, _i64, _i32, _i32, _i32, _p, _p, _i64, _p, _i32, _p,
                        _i32, _p, _p, _i32, _i64, _p, _i32, _f32, _p, _f32, _p, _p, _i32, _p, _sz, _p)
_lib_partial_bytes = _sig("cskv_attend_partial_bytes", _sz, _i64, _i32, _i32)
_lib_window_partial = _sig("cskv_attend_window_partial", _i32, _p, _i64, _i32, _i32, _i32, _p, _p, _i32, _i64, _p,
                           _f32, _p, _p)
_lib_append = _sig("cskv_append", _i32, _i32, _p, _p, _p, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _i64,
                   _p, _p, _p)
_lib_enc8 = _sig("cskv_encode_fp8_rows", _i32, _i32, _p, _i64, _i32, _p, _p, _p)
_lib_dec8 = _sig("cskv_decode_fp8_rows", _i32, _p, _p, _i64, _i32, _p, _p)
_lib_enc4 = _sig("cskv_encode_fp4_g16", _i32, _i32, _p, _i64, _i32, _p, _p, _p)
_lib_dec4 = _sig("cskv_decode_fp4_g16", _i32, _p, _p, _i64, _i32, _p, _p)

EXPORTS = ["cskv_status_string", "cskv_last_error", "cskv_version", "cskv_compress", "cskv_append",
           "cskv_index_topk_workspace", "cskv_index_topk", "cskv_attend_workspace", "cskv_attend",
           "cskv_attend_noalloc", "cskv_attend_partial_bytes", "cskv_attend_window_partial",
           "cskv_attend_with_partial",
           "cskv_encode_fp8_rows", "cskv_decode_fp8_rows", "cskv_encode_fp4_g16", "cskv_decode_fp4_g16"]


class CskvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib_status_string(status).decode()}: {message}")
        self.status = status


def _check(status: int):
    if status != OK:
        raise CskvError(status, _lib_last_error().decode())


def version() -> int:
    return int(_lib_version())


# Pointers and streams go to ctypes as plain integers (the c_void_p argtypes
# convert them): a per-argument c_void_p object costs more than the call's
# own conversion, and a decode step makes these calls once per layer.
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _bf16_like(t, name):
    if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError(f"{name} must hold bf16 bits (bfloat16/uint16/int16), got {t.dtype}")


def _dense(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_workspaces: dict = {}
_retired: list = []


def _workspace(purpose: str, nbytes: int, device, layout=None, stream=None) -> torch.Tensor | None:
    """A scratch buffer for one (purpose, device, current stream, layout).

    Calls on one stream are ordered, so they can share a buffer; calls on two
    streams never do. ``layout`` names the argument set of a workspace that
    carries state between calls (index_topk: histograms and counters that
    every call leaves zero): each layout gets a buffer of its own, zero-filled
    once when it is made, so a call with other arguments never sees or leaves
    another layout's state. A stateless buffer (layout None) grows on demand.
    No buffer is ever freed while the process runs (a grown one is retired,
    not dropped), so a HIP graph captured with a buffer's address can be
    replayed after later eager calls of any shape. ``stream`` is the
    device's current stream handle when the caller has it already."""
    if nbytes == 0:
        return None
    dev = device if isinstance(device, torch.device) else torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    key = (purpose, dev.index, stream, layout)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _retired.append(buf)
        # zeroed by a fill kernel (not a memset, which a captured graph
        # would hold as a node of its own)
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev).zero_()
        _workspaces[key] = buf
    return buf


_ws_sizes: dict = {}


def _ws_bytes(fn, *args) -> int:
    """A workspace-size query of the library, remembered per argument set
    (the sizes depend on the arguments alone)."""
    key = (id(fn), args)   # (ctypes functions are not hashable; these live as long as the module)
    n = _ws_sizes.get(key)
    if n is None:
        n = _ws_sizes[key] = int(fn(*args))
    return n


def _caller_workspace(ws: torch.Tensor, nbytes: int, name: str) -> torch.Tensor:
    if not ws.is_cuda or ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.numel() < nbytes:
        raise ValueError(f"{name} must be a contiguous uint8 GPU tensor of at least {nbytes} bytes")
    if ws.data_ptr() % 256:
        raise ValueError(f"{name} must be 256-byte aligned")
    return ws


# ------------------------------------------------------------------ compress

def _cache_format(cache: torch.Tensor, cache_scale: torch.Tensor | None, B: int, D: int) -> int:
    """The cache's row format from its dtype and width: bf16 [B, rows, D];
    fp8 codes uint8 [B, rows, D]; mixed rows uint8 [B, rows, D + 64] (the
    D - 64 fp8 codes, then the 64 rotary channels as bf16); or fp4 rows uint8
    [B, rows, D/2 + D/16] (E2M1 codes, then one E4M3 scale byte per 16
    channels). Both fp8 forms need cache_scale fp32 [B, rows]."""
    if cache.dim() != 3 or cache.shape[0] != B:
        raise ValueError("cache must be [B, rows, D] (or uint8 rows of a quantised format)")
    if cache.dtype == torch.uint8 and cache.shape[2] == D // 2 + D // 16:
        return FP4_E2M1
    if cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        if cache.shape[2] == D:
            fmt = FP8_E4M3
        elif cache.shape[2] == D + MIX_ROPE and cache.dtype == torch.uint8:
            fmt = FP8_ROPE64
        else:
            raise ValueError(f"an fp8 cache must be [B, rows, {D}] (codes) or [B, rows, {D + MIX_ROPE}] (mixed rows)")
        if cache_scale is None or cache_scale.dtype != torch.float32 or tuple(cache_scale.shape) != tuple(cache.shape[:2]):
            raise ValueError("an fp8 cache needs cache_scale fp32 [B, rows]")
        _dense(cache_scale, "cache_scale")
        return fmt
    if cache.shape[2] != D:
        raise ValueError("cache must be [B, rows, D]")
    _bf16_like(cache, "cache")
    return BF16


def compress(kind, S: torch.Tensor, gate: torch.Tensor, cache: torch.Tensor,
             cache_scale: torch.Tensor | None = None, first_entry: int = 0) -> int:
    """Writes the complete entries of the span S [B, T, D] (gate [B, T] fp32)
    into rows first_entry.. of cache [B, rows, D] (bf16, or uint8 fp8 codes
    with cache_scale [B, rows] fp32). Returns the number of entries written."""
    kind = KINDS[kind]
    _need_cuda(S, gate, cache, cache_scale)
    _bf16_like(S, "S")
    _dense(S, "S"); _dense(gate, "gate"); _dense(cache, "cache")
    B, T, D = S.shape
    if gate.dtype != torch.float32 or tuple(gate.shape) != (B, T):
        raise ValueError("gate must be fp32 [B, T]")
    dt = _cache_format(cache, cache_scale, B, D)
    _check(_lib_compress(kind, _ptr(S), _ptr(gate), B, T, D, first_entry, dt, _ptr(cache),
                         _ptr(cache_scale), cache.shape[1], _stream(S.device)))
    w, s = (8, 4) if kind == C4A else (128, 128)
    return 0 if T < w else (T - w) // s + 1


def append(kind, s_new: torch.Tensor, g_new: torch.Tensor, pos: torch.Tensor, ring: torch.Tensor,
           ring_gate: torch.Tensor, cache: torch.Tensor, cache_scale: torch.Tensor | None = None,
           n_entries: torch.Tensor | None = None, n_window: torch.Tensor | None = None) -> None:
    """Streaming decode: sequence b appends s_new[b] ([B, D] bf16, gate logit
    g_new[b] fp32) as token pos[b] (int64 [B]; negative skips it) into its ring
    ([B, W, D] bf16, ring_gate [B, W] fp32; token p in slot p mod W) and, when
    the token completes an entry, writes that entry into cache (as compress()).
    Optionally sets n_entries / n_window (int32 [B]) for index_topk / attend."""
    kind = KINDS[kind]
    _need_cuda(s_new, g_new, pos, ring, ring_gate, cache, cache_scale, n_entries, n_window)
    _bf16_like(s_new, "s_new"); _bf16_like(ring, "ring")
    for t, n in ((s_new, "s_new"), (g_new, "g_new"), (pos, "pos"), (ring, "ring"), (ring_gate, "ring_gate"),
                 (cache, "cache")):
        _dense(t, n)
    B, D = s_new.shape
    if g_new.dtype != torch.float32 or g_new.numel() != B:
        raise ValueError("g_new must be fp32 [B]")
    if pos.dtype != torch.int64 or pos.numel() != B:
        raise ValueError("pos must be int64 [B]")
    if ring.dim() != 3 or ring.shape[0] != B or ring.shape[2] != D:
        raise ValueError("ring must be [B, W, D]")
    W = ring.shape[1]
    if ring_gate.dtype != torch.float32 or tuple(ring_gate.shape) != (B, W):
        raise ValueError("ring_gate must be fp32 [B, W]")
    dt = _cache_format(cache, cache_scale, B, D)
    for t, n in ((n_entries, "n_entries"), (n_window, "n_window")):
        if t is not None and (t.dtype != torch.int32 or t.numel() != B or not t.is_contiguous()):
            raise ValueError(f"{n} must be contiguous int32 [B]")
    _check(_lib_append(kind, _ptr(s_new), _ptr(g_new), _ptr(pos), B, D, _ptr(ring), _ptr(ring_gate), W, dt,
                       _ptr(cache), _ptr(cache_scale), cache.shape[1], _ptr(n_entries), _ptr(n_window),
                       _stream(s_new.device)))


# ------------------------------------------------------------------ index / top-k

def index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, k: int, k_scale: torch.Tensor | None = None,
               n_entries: torch.Tensor | None = None, ids: torch.Tensor | None = None,
               chunk: int = 0, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """ids [B, k] int32 of the best k entries per sequence (ascending, -1 padded).
    Keys are bf16 [B, N, Di], or fp4 packed uint8 [B, N, Di/2] with k_scale
    uint8 [B, N, Di/16]. ``workspace`` (uint8, at least
    index_topk_workspace_bytes() bytes, zero-filled before its first use) is
    the caller's own; otherwise the binding keeps one per stream and argument
    set."""
    _need_cuda(q_idx, k_idx, k_scale, n_entries, ids)
    _bf16_like(q_idx, "q_idx")
    _dense(q_idx, "q_idx"); _dense(k_idx, "k_idx")
    B, Di = q_idx.shape
    if k_scale is None:
        _bf16_like(k_idx, "k_idx")
        key_dtype = BF16
        if k_idx.shape[0] != B or k_idx.shape[2] != Di:
            raise ValueError("k_idx must be [B, N, Di]")
    else:
        key_dtype = FP4_E2M1
        _dense(k_scale, "k_scale")
        if k_idx.dtype != torch.uint8 or tuple(k_idx.shape) != (B, k_idx.shape[1], Di // 2):
            raise ValueError("fp4 k_idx must be uint8 [B, N, Di/2]")
        if k_scale.dtype != torch.uint8 or tuple(k_scale.shape) != (B, k_idx.shape[1], Di // 16):
            raise ValueError("k_scale must be uint8 [B, N, Di/16]")
    N = k_idx.shape[1]
    if n_entries is not None:
        _dense(n_entries, "n_entries")
        if n_entries.dtype != torch.int32 or n_entries.numel() != B:
            raise ValueError("n_entries must be int32 [B]")
    if ids is None:
        ids = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    elif ids.dtype != torch.int32 or tuple(ids.shape) != (B, k) or not ids.is_contiguous():
        raise ValueError("ids must be contiguous int32 [B, k]")
    nbytes = _ws_bytes(_lib_topk_ws, B, N, Di, k, key_dtype, chunk)   # 0 also when the call will reject
    stream = _stream(q_idx.device)
    if workspace is not None:
        ws = _caller_workspace(workspace, nbytes, "workspace")
    else:
        ws = _workspace("index_topk", nbytes, q_idx.device, layout=(B, N, Di, k, key_dtype, chunk), stream=stream)
    _check(_lib_topk(_ptr(q_idx), key_dtype, _ptr(k_idx), _ptr(k_scale), _ptr(n_entries), B, N, Di, k,
                     _ptr(ids), chunk, _ptr(ws), 0 if ws is None else ws.numel(), stream))
    return ids


# ------------------------------------------------------------------ attend

def _window_args(window, window_scale, B, D):
    """(window or None, W, batch stride in rows, fp8?) of an attend window [B, W, D]."""
    if window is None:
        return None, 0, 0, False
    shape = window.shape
    if len(shape) != 3 or shape[0] != B or shape[2] != D:
        if len(shape) >= 2 and shape[1] == 0:
            return None, 0, 0, False
        raise ValueError("window must be [B, W, D]")
    W = shape[1]
    if W == 0:
        return None, 0, 0, False
    st = window.stride()
    if st[2] != 1 or st[1] != D or st[0] % D != 0:
        raise ValueError("window rows must be dense with a whole-row batch stride")
    wstride = st[0] // D
    win_fp8 = window.dtype in (torch.uint8, torch.float8_e4m3fn)
    if win_fp8:
        if window_scale is None or window_scale.dtype != torch.float32:
            raise ValueError("an fp8 window needs window_scale fp32 [B, W]")
        if window_scale.stride(1) != 1 or window_scale.stride(0) != wstride:
            raise ValueError("window_scale must share the window's batch stride (in rows)")
    else:
        _bf16_like(window, "window")
    return window, W, wstride, win_fp8


def attend(Q: torch.Tensor, cache: torch.Tensor, ids: torch.Tensor | None, window: torch.Tensor | None, *,
           softmax_scale: float, rope_dims: int = 0, rope_base: float = 10000.0,
           q_pos: torch.Tensor | None = None, cache_scale: torch.Tensor | None = None,
           window_scale: torch.Tensor | None = None, n_entries: torch.Tensor | None = None,
           n_window: torch.Tensor | None = None, out: torch.Tensor | None = None,
           splits: int = 0, workspace: torch.Tensor | None = None, noalloc: bool = False,
           partial: torch.Tensor | None = None) -> torch.Tensor:
    """O [B, H, D] fp32: softmax attention of Q [B, H, D] (bf16) over the cache
    rows named by ids [B, k] (or all of the first n_entries rows when ids is
    None) followed by the window rows [B, W, D], then inverse RoPE on the last
    rope_dims channels at positions q_pos [B] int64. The window may be a view
    whose last two dimensions are dense (e.g. the tail of a state span).
    n_window [B] int32 keeps only the first n_window[b] window rows (a ring
    from append() that has not wrapped yet). With ``partial`` (from
    attend_window_partial, complete on this stream), O also covers that
    partial's keys, in the same softmax (cskv_attend_with_partial)."""
    _need_cuda(Q, cache, ids, window, q_pos, cache_scale, window_scale, n_entries, n_window, out, partial)
    _bf16_like(Q, "Q")
    _dense(Q, "Q"); _dense(cache, "cache")
    B, H, D = Q.shape
    cache_dt = _cache_format(cache, cache_scale, B, D)
    k = 0
    if ids is not None:
        if ids.dtype != torch.int32 or ids.dim() != 2 or ids.shape[0] != B or not ids.is_contiguous():
            raise ValueError("ids must be contiguous int32 [B, k]")
        k = ids.shape[1]
    if n_entries is not None and (n_entries.dtype != torch.int32 or n_entries.numel() != B):
        raise ValueError("n_entries must be int32 [B]")
    if n_window is not None and (n_window.dtype != torch.int32 or n_window.numel() != B
                                 or not n_window.is_contiguous()):
        raise ValueError("n_window must be contiguous int32 [B]")
    window, W, wstride, win_fp8 = _window_args(window, window_scale, B, D)
    if rope_dims and (q_pos is None or q_pos.dtype != torch.int64 or q_pos.numel() != B):
        raise ValueError("rope_dims > 0 needs q_pos int64 [B]")
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float32, device=Q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, H, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [B, H, D]")
    if partial is not None:
        if noalloc:
            raise ValueError("attend_noalloc takes no partial")
        _check_partial(partial, B, H, D)
    if noalloc:
        _check(_lib_attend_noalloc(_ptr(Q), B, H, D, cache_dt, _ptr(cache), _ptr(cache_scale),
                                   cache.shape[1], _ptr(ids), k, _ptr(n_entries), FP8_E4M3 if win_fp8 else BF16,
                                   _ptr(window), _ptr(window_scale), W, wstride, _ptr(n_window), rope_dims,
                                   rope_base, _ptr(q_pos), softmax_scale, _ptr(out), splits, _stream(Q.device)))
        return out
    max_keys = (k if ids is not None else cache.shape[1]) + W
    nbytes = _ws_bytes(_lib_attend_ws, B, H, D, max_keys, splits)
    stream = _stream(Q.device)
    if workspace is not None:
        ws = _caller_workspace(workspace, nbytes, "workspace")
    else:
        ws = _workspace("attend", nbytes, Q.device, stream=stream)
    if partial is not None:
        _check(_lib_attend_part(_ptr(Q), B, H, D, cache_dt, _ptr(cache), _ptr(cache_scale),
                                cache.shape[1], _ptr(ids), k, _ptr(n_entries), FP8_E4M3 if win_fp8 else BF16,
                                _ptr(window), _ptr(window_scale), W, wstride, _ptr(n_window), rope_dims, rope_base,
                                _ptr(q_pos), softmax_scale, _ptr(partial), _ptr(out), splits, _ptr(ws),
                                0 if ws is None else ws.numel(), stream))
        return out
    _check(_lib_attend(_ptr(Q), B, H, D, cache_dt, _ptr(cache), _ptr(cache_scale),
                       cache.shape[1], _ptr(ids), k, _ptr(n_entries), FP8_E4M3 if win_fp8 else BF16,
                       _ptr(window), _ptr(window_scale), W, wstride, _ptr(n_window), rope_dims, rope_base,
                       _ptr(q_pos),
                       softmax_scale, _ptr(out), splits, _ptr(ws), 0 if ws is None else ws.numel(),
                       stream))
    return out


def partial_bytes(B: int, H: int, D: int) -> int:
    """Bytes of an attend partial of B sequences and H heads (0 if unsupported)."""
    return _lib_partial_bytes(B, H, D)


def _check_partial(partial: torch.Tensor, B: int, H: int, D: int) -> None:
    need = _lib_partial_bytes(B, H, D)
    if (partial.dtype != torch.float32 or not partial.is_contiguous()
            or partial.numel() * 4 < need or partial.data_ptr() % 16):
        raise ValueError(f"partial must be a contiguous, 16-byte aligned fp32 buffer of {need} bytes")


def attend_window_partial(Q: torch.Tensor, window: torch.Tensor | None, *, softmax_scale: float,
                          window_scale: torch.Tensor | None = None, n_window: torch.Tensor | None = None,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """The attend partial of Q [B, H, D] over the window rows alone
    (cskv_attend_window_partial): a flat fp32 buffer holding values
    [B, H, D] (normalised by their own softmax sum, not rotated) and then
    (reference maximum in log2 units, sum) pairs [B, H]. Pass it to
    attend(..., partial=) with the selected entries; it needs no indexer
    result, so it can run on another stream while the indexer runs."""
    _need_cuda(Q, window, window_scale, n_window, out)
    _bf16_like(Q, "Q")
    _dense(Q, "Q")
    B, H, D = Q.shape
    window, W, wstride, win_fp8 = _window_args(window, window_scale, B, D)
    if n_window is not None and (n_window.dtype != torch.int32 or n_window.numel() != B
                                 or not n_window.is_contiguous()):
        raise ValueError("n_window must be contiguous int32 [B]")
    need = _lib_partial_bytes(B, H, D)
    if out is None:
        out = torch.empty(max(need // 4, 1), dtype=torch.float32, device=Q.device)
    else:
        _check_partial(out, B, H, D)
    _check(_lib_window_partial(_ptr(Q), B, H, D, FP8_E4M3 if win_fp8 else BF16, _ptr(window),
                               _ptr(window_scale), W, wstride, _ptr(n_window), softmax_scale, _ptr(out),
                               _stream(Q.device)))
    return out


def attend_noalloc(Q: torch.Tensor, cache: torch.Tensor, ids: torch.Tensor | None, window: torch.Tensor | None,
                   **kw) -> torch.Tensor:
    """attend() through cskv_attend_noalloc: the split partials live in the
    library's per-device scratch array instead of a workspace, and the call
    allocates nothing (pass ``out`` too, for a caller that cannot allocate).
    Calls that overlap in time on one GPU share that scratch and race."""
    if "workspace" in kw:
        raise TypeError("attend_noalloc takes no workspace")
    return attend(Q, cache, ids, window, noalloc=True, **kw)


# ------------------------------------------------------------------ codecs

def encode_fp8_rows(x: torch.Tensor):
    """[rows, D] bf16 or fp32 -> (codes uint8 [rows, D], scale fp32 [rows])."""
    _need_cuda(x)
    _dense(x, "x")
    in_dt = F32 if x.dtype == torch.float32 else BF16
    if in_dt == BF16:
        _bf16_like(x, "x")
    rows, D = x.reshape(-1, x.shape[-1]).shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(_lib_enc8(in_dt, _ptr(x), rows, D, _ptr(codes), _ptr(scale), _stream(x.device)))
    return codes, scale


def decode_fp8_rows(codes: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    _need_cuda(codes, scale)
    _dense(codes, "codes"); _dense(scale, "scale")
    rows, D = codes.reshape(-1, codes.shape[-1]).shape
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(_lib_dec8(_ptr(codes), _ptr(scale), rows, D, _ptr(out), _stream(codes.device)))
    return out


def encode_fp4_g16(x: torch.Tensor):
    """[rows, Di] bf16 or fp32 -> (packed uint8 [rows, Di/2], scales uint8 [rows, Di/16])."""
    _need_cuda(x)
    _dense(x, "x")
    in_dt = F32 if x.dtype == torch.float32 else BF16
    if in_dt == BF16:
        _bf16_like(x, "x")
    Di = x.shape[-1]
    rows = x.numel() // Di
    packed = torch.empty(x.shape[:-1] + (Di // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (Di // 16,), dtype=torch.uint8, device=x.device)
    _check(_lib_enc4(in_dt, _ptr(x), rows, Di, _ptr(packed), _ptr(scales), _stream(x.device)))
    return packed, scales


def decode_fp4_g16(packed: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    _need_cuda(packed, scales)
    _dense(packed, "packed"); _dense(scales, "scales")
    Di = packed.shape[-1] * 2
    rows = packed.numel() // (Di // 2)
    out = torch.empty(packed.shape[:-1] + (Di,), dtype=torch.float32, device=packed.device)
    _check(_lib_dec4(_ptr(packed), _ptr(scales), rows, Di, _ptr(out), _stream(packed.device)))
    return out


# ------------------------------------------------------------------ raw access (tests, bench)

def raw():
    """The ctypes handle of libcskv.so, for tests of the C ABI itself."""
    return _lib
