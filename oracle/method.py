"""The decode step of compressed shared-K/V attention, as plain definitions.

Everything here is float64 (numpy), one sequence at a time, no blocking or
fusion. Sources:

[P2] Step 3 ("DeepSeek V4 makes one vector do both jobs"): every token leaves
one shared state S_j, used both as the key (score = Q . S_j) and as the value.
[P1] paragraph "Shared key and value": same fact; V4 applies an inverse RoPE to
the attention output.
[P1] paragraphs "c4a (the milder scheme)" / "c128a (the aggressive scheme)" and
[P2] Step 4 ("Older shared states are compressed"): a c4a entry is a learned
weighted sum of 8 states with stride 4 (the walkthrough's example: states
S0..S7 and S4..S11 give the first two entries); a c128a entry is a weighted sum
of 128 states with stride 128 (S0..S127, S128..S255).
[P2] Step 5 ("The query now reads a mixed memory map"): a learned indexer
scores the c4a entries and the query reads only the selected ones (top-k, k =
512 by default per [P1]); all c128a entries are read.
[P2] Step 6 ("The newest tokens stay uncompressed") and [P1] paragraph "The
sliding window": every layer also reads the last 128 uncompressed states.
[P2] Step 1 ("One token becomes three views"): softmax attention, output =
weighted sum of the values.

Readings where the pages are silent or loose (each is listed with its reason
in the design notes):
* gate: every token carries one scalar gate logit; an entry's weights are the
  softmax of the logits of its own window (so one token weighs differently in
  its two c4a windows).
* counts: an entry exists once its window is complete: floor((T-8)/4)+1 c4a
  entries and floor(T/128) c128a entries for T states; entries are numbered
  from 0 (entry c covers states s*c .. s*c+w-1).
* indexer: one score per entry, the dot product of the query's indexer vector
  with the entry's indexer key.
* top-k order: score descending, then entry number ascending (ties go to the
  lowest entry); NaN scores rank below every number; the ids are returned in
  ascending order, padded with -1 when fewer than k entries exist.
* attention: one softmax jointly over the selected entries and the window
  rows, logits scaled by tau; an empty key set gives a zero output.
* inverse RoPE: the last R channels form interleaved pairs (2i, 2i+1) rotated
  by -pos * base^(-2i/R), pos being the query's position.
"""
from __future__ import annotations

import numpy as np

C4A = "c4a"
C128A = "c128a"
WINDOW = {C4A: (8, 4), C128A: (128, 128)}   # (states per entry, stride)


# ------------------------------------------------------------------ compress

def entry_count(kind: str, T: int) -> int:
    w, s = WINDOW[kind]
    return 0 if T < w else (T - w) // s + 1


def entry_span(kind: str, c: int) -> range:
    """States folded into entry c."""
    w, s = WINDOW[kind]
    return range(s * c, s * c + w)


def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def compress_entry(kind: str, S: np.ndarray, g: np.ndarray, c: int) -> np.ndarray:
    """One entry: sum over its window of softmax(gate logits)_j * S_j."""
    span = list(entry_span(kind, c))
    wts = softmax(np.asarray(g, dtype=np.float64)[span])
    return wts @ np.asarray(S, dtype=np.float64)[span]


def compress(kind: str, S: np.ndarray, g: np.ndarray, first: int = 0, count: int | None = None) -> np.ndarray:
    """Entries ``first .. first+count-1`` of the states S [T, D] with gate
    logits g [T] (all complete entries by default). Returns [count, D] float64."""
    T = np.asarray(S).shape[0]
    n = entry_count(kind, T)
    if count is None:
        count = n - first
    assert 0 <= first and first + count <= n
    D = np.asarray(S).shape[1]
    out = np.zeros((count, D), dtype=np.float64)
    for i in range(count):
        out[i] = compress_entry(kind, S, g, first + i)
    return out


# ------------------------------------------------------------------- indexer

def index_scores(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """score[c] = q_idx . k_idx[c] for keys [N, Di] (float64)."""
    return np.asarray(k_idx, dtype=np.float64) @ np.asarray(q_idx, dtype=np.float64)


def topk_ids(scores: np.ndarray, k: int, n_valid: int | None = None) -> np.ndarray:
    """The k best of the first n_valid entries (score descending, entry
    ascending on ties, NaN lowest), as int32 ids in ascending order, padded
    with -1 to length k."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0] if n_valid is None else int(min(max(n_valid, 0), s.shape[0]))
    s = s[:n]
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s)
    order = np.lexsort((np.arange(n), neg, nan))   # last key is the primary key
    take = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: take.shape[0]] = take
    return out


# ----------------------------------------------------------------- attention

def gather_keys(cache: np.ndarray, ids: np.ndarray | None, window: np.ndarray | None,
                n_entries: int | None = None) -> np.ndarray:
    """The key (= value) rows a query reads: the selected cache entries in the
    order of ``ids`` (ids < 0 skipped; ``ids=None`` means every one of the
    first n_entries entries), then the window rows."""
    cache = np.asarray(cache, dtype=np.float64)
    if ids is None:
        n = cache.shape[0] if n_entries is None else n_entries
        rows = cache[:n]
    else:
        ids = np.asarray(ids)
        rows = cache[ids[ids >= 0]]
    parts = [rows]
    if window is not None and np.asarray(window).shape[0] > 0:
        parts.append(np.asarray(window, dtype=np.float64))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, cache.shape[1]))


def attention(Q: np.ndarray, K: np.ndarray, tau: float) -> np.ndarray:
    """Shared-K/V softmax attention: O[h] = sum_j softmax_j(tau * Q[h].K_j) K_j."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros_like(Q)
    logits = tau * (Q @ K.T)
    return softmax(logits, axis=1) @ K


def rope_angles(R: int, base: float, pos: float) -> np.ndarray:
    """Angle pos * base^(-2i/R) of each rotary pair i < R/2."""
    i = np.arange(R // 2, dtype=np.float64)
    return float(pos) * np.power(float(base), -2.0 * i / R)


def inverse_rope(O: np.ndarray, R: int, base: float, pos: float) -> np.ndarray:
    """Rotate each pair (2i, 2i+1) of the last R channels by -pos*theta_i."""
    O = np.array(O, dtype=np.float64, copy=True)
    if R == 0:
        return O
    D = O.shape[-1]
    a = -rope_angles(R, base, pos)
    c, s = np.cos(a), np.sin(a)
    x = O[..., D - R + 0::2].copy()
    y = O[..., D - R + 1::2].copy()
    O[..., D - R + 0::2] = x * c - y * s
    O[..., D - R + 1::2] = x * s + y * c
    return O


def attend(Q: np.ndarray, cache: np.ndarray, ids: np.ndarray | None, window: np.ndarray | None,
           tau: float, R: int, base: float, q_pos: float, n_entries: int | None = None) -> np.ndarray:
    """One sequence: attention over the gathered keys, then inverse RoPE."""
    K = gather_keys(cache, ids, window, n_entries)
    return inverse_rope(attention(Q, K, tau), R, base, q_pos)


# ------------------------------------------------------- split attention
#
# [P1] "How DeepSeek V4 Uses Less Memory: KV Cache Explained", the passage on
# the decode-path kernels: the indexer runs on a stream of its own beside the
# main attention path. Reading: the window rows need no indexer result, so
# their share of the softmax can be computed while the indexer runs and be
# combined with the selected entries' share afterwards. A softmax over the
# union of disjoint key sets follows exactly from each set's normalised output
# and its log-sum-exp: O = sum_s 2^(lse_s - LSE) O_s, LSE = log2 sum_s 2^lse_s.

def attention_partial(Q: np.ndarray, K: np.ndarray, tau: float):
    """(O, lse) of Q [H, D] over keys K [N, D]: O = attention(Q, K, tau) and
    lse[h] = log2 sum_j 2^x_hj with x = tau log2(e) Q[h].K_j (log2 units).
    No key: O = 0 and lse = -inf."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros_like(Q), np.full(Q.shape[0], -np.inf)
    x = tau * np.log2(np.e) * (Q @ K.T)
    m = x.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log2(np.exp2(x - m).sum(axis=1))
    return attention(Q, K, tau), lse


def merge_partials(parts):
    """Combines partials (O_s, lse_s) over disjoint key sets into the output
    over their union; sets without keys (lse = -inf) take no part."""
    lses = np.stack([lse for _, lse in parts])            # [S, H]
    top = lses.max(axis=0)
    w = np.exp2(lses - np.where(np.isfinite(top), top, 0.0))   # 0 for a set without keys
    total = w.sum(axis=0)
    w = w / np.where(total > 0, total, 1.0)
    return sum(w[s][:, None] * np.asarray(parts[s][0], dtype=np.float64) for s in range(len(parts)))


# ------------------------------------------------------------ decode layers

def c4a_decode(Q, q_idx, k_idx, cache, window, k, tau, R, base, q_pos, n_entries=None):
    """A c4a layer for one sequence: indexer scores, top-k, gather attention."""
    scores = index_scores(q_idx, k_idx)
    ids = topk_ids(scores, k, n_entries)
    return ids, attend(Q, cache, ids, window, tau, R, base, q_pos)


def c128a_decode(Q, cache, window, tau, R, base, q_pos, n_entries=None):
    """A c128a layer for one sequence: dense attention over every entry."""
    return attend(Q, cache, None, window, tau, R, base, q_pos, n_entries)


# ------------------------------------------------------- streaming decode
#
# [P1] cache-block paragraph: besides the compressed entries, each layer keeps
# a constant-size compressor state and the sliding window; [P1] "c4a" / "c128a"
# and [P2] Step 4: an entry exists once the last state of its window exists,
# so a decoder appending one state per step completes a c4a entry every 4
# steps and a c128a entry every 128. [P2] Step 6: the window is the newest W
# states. Reading: one ring of the last W states and their gate logits per
# sequence (token p in slot p mod W) is both the window and the compressor's
# carry; it needs W >= 8 (c4a) or W >= 128 (c128a).

def append(kind: str, ring: np.ndarray, ring_gate: np.ndarray, s_new: np.ndarray, g_new: float,
           pos: int):
    """Appends state s_new with gate logit g_new as token ``pos`` of one
    sequence: stores it in ring slot pos mod W (ring [W, D], ring_gate [W],
    both modified in place) and, when the token completes an entry, returns
    (c, entry row) computed from the ring as the definition does from the
    states; otherwise (None, None)."""
    w, s = WINDOW[kind]
    W = ring.shape[0]
    assert W >= w and pos >= 0
    ring[pos % W] = np.asarray(s_new, dtype=np.float64)
    ring_gate[pos % W] = float(g_new)
    first = pos + 1 - w                    # first state of the window ending at pos
    if first < 0 or first % s != 0:
        return None, None
    slots = [(first + j) % W for j in range(w)]
    wts = softmax(np.asarray(ring_gate, dtype=np.float64)[slots])
    return first // s, wts @ np.asarray(ring, dtype=np.float64)[slots]


def stream_counts(kind: str, pos: int, W: int) -> tuple[int, int]:
    """(complete entries, window rows) of a sequence whose newest token is pos."""
    return entry_count(kind, pos + 1), min(pos + 1, W)
