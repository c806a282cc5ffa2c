"""The five decode workloads, as shapes, value distributions and seeds.

Each workload is one decode step of a compressed-KV attention layer (or of a
61-layer stack). The figures come from the pages' own workloads: top-512
selection, a 128-token window, 30 c4a + 31 c128a layers, 128K and 1M contexts,
fp8 attention caches and fp4 indexer keys. Values are synthetic.
"""
from __future__ import annotations

import math
from dataclasses import dataclass


def c4a_entries(L: int) -> int:
    """Complete c4a windows (8 tokens, stride 4) in a context of L tokens."""
    return 0 if L < 8 else (L - 8) // 4 + 1


def c128a_entries(L: int) -> int:
    """Complete c128a windows (128 tokens, stride 128) in a context of L tokens."""
    return L // 128


@dataclass(frozen=True)
class Workload:
    name: str
    number: int
    kind: str              # "c4a", "c128a", "mixed" or "stream" (c4a, one token appended per step)
    B: int                 # sequences in the batch
    L: int                 # context length in tokens (the query is token L-1)
    D: int                 # shared-state width (keys and values are the same S rows)
    R: int                 # rotary channels, the last R of D
    H: int                 # query heads
    W: int                 # uncompressed window rows
    Di: int = 0            # indexer key width (c4a)
    k: int = 0             # top-k (c4a)
    idx_range: int = 0     # indexer values are integers in [-idx_range, idx_range]
    cache_dtype: str = "bf16"   # "bf16", "fp8", "mixed" (fp8 codes + bf16 rotary channels) or "fp4"
    key_dtype: str = "bf16"     # indexer keys: "bf16" or "fp4"
    rope_base: float = 10000.0
    layers: int = 1
    reuse_ids: bool = False     # mixed stack: every second c4a layer reuses the ids of the one before
    only_layers: tuple = ()     # mixed stack: build just these layers of the stack (checks of late layers)
    description: str = ""

    @property
    def seed(self) -> int:
        return 0xC5C0DE00 + self.number

    @property
    def tau(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def q_pos(self) -> int:
        return self.L - 1

    @property
    def n_entries(self) -> int:
        if self.kind in ("c4a", "stream"):
            return c4a_entries(self.L)
        if self.kind == "c128a":
            return c128a_entries(self.L)
        raise ValueError("mixed workloads have per-layer entry counts")

    def layer_kind(self, layer: int) -> str:
        """Mixed stack: c128a on even layers (31 of 61), c4a on odd layers (30)."""
        if self.kind == "stream":
            return "c4a"
        if self.kind != "mixed":
            return self.kind
        return "c128a" if layer % 2 == 0 else "c4a"

    def reuses(self, layer: int):
        """Mixed stack with id reuse: the c4a layer whose ids this layer takes
        (c4a layers 3, 7, 11, ... take those of layers 1, 5, 9, ...), or None."""
        if not self.reuse_ids or self.layer_kind(layer) != "c4a" or layer % 4 != 3:
            return None
        return layer - 2

    def stream_lag(self, b: int) -> int:
        """Streaming workload: sequence b's context is L - stream_lag(b) tokens
        when the timed steps start (a ragged batch: lags 0 .. 127)."""
        return (37 * b) % 128


TINY = Workload(
    name="tiny_c4a_2k", number=1, kind="c4a", B=1, L=2048, D=128, R=32, H=8, W=32,
    Di=32, k=64, idx_range=4,
    description="one c4a layer, 1 sequence, 2048 tokens, D=128 (32 rotary), 8 heads, "
                "indexer dim 32 ints in [-4,4], top-64 + 32-row window",
)

C4A_128K = Workload(
    name="c4a_128k_bf16", number=2, kind="c4a", B=32, L=131072, D=512, R=64, H=64, W=128,
    Di=128, k=512, idx_range=8,
    description="one c4a layer, 32 sequences x 131072 tokens, D=512 (64 rotary), 64 heads, "
                "indexer dim 128 ints in [-8,8] (bf16), top-512 + 128-row window",
)

C128A_1M = Workload(
    name="c128a_1m_bf16", number=3, kind="c128a", B=16, L=1 << 20, D=512, R=64, H=64, W=128,
    description="one c128a layer, 16 sequences x 1048576 tokens, dense over 8192 entries "
                "+ 128-row window, 64 heads",
)

C4A_1M_Q = Workload(
    name="c4a_1m_fp8_fp4", number=4, kind="c4a", B=8, L=1 << 20, D=512, R=64, H=64, W=128,
    Di=128, k=512, idx_range=8, cache_dtype="fp8", key_dtype="fp4",
    description="one c4a layer, 8 sequences x 1048576 tokens, fp8 E4M3 attention cache "
                "(row fp32 scale), fp4 E2M1 indexer keys (E4M3 scale per 16), top-512 + 128-row window",
)

MIXED_61 = Workload(
    name="mixed61_256k_bf16", number=5, kind="mixed", B=64, L=262144, D=512, R=64, H=64, W=128,
    Di=128, k=512, idx_range=8, layers=61,
    description="61-layer decode step (31 c128a on even layers, 30 c4a on odd), 64 sequences "
                "x 262144 tokens; each layer compresses 128 new tokens, then attends",
)

MIXED_61_REUSE = Workload(
    name="mixed61_256k_reuse", number=9, kind="mixed", B=64, L=262144, D=512, R=64, H=64, W=128,
    Di=128, k=512, idx_range=8, layers=61, reuse_ids=True,
    description="the 61-layer step with top-k ids reused across c4a layers: 15 of the 30 c4a layers "
                "skip their indexer and attend over the previous c4a layer's selection",
)

STREAM_C4A_128K = Workload(
    name="stream_c4a_128k_bf16", number=6, kind="stream", B=32, L=131072, D=512, R=64, H=64, W=128,
    Di=128, k=512, idx_range=8,
    description="streaming c4a decode: 32 sequences at ragged contexts 131072 - (0..127) tokens; each step "
                "appends one state per sequence to its 128-row ring (an entry every 4 steps), then "
                "index_topk over the ragged entry counts and attend over the ring as window",
)

C128A_1M_MIXED = Workload(
    name="c128a_1m_mixed", number=7, kind="c128a", B=16, L=1 << 20, D=512, R=64, H=64, W=128,
    cache_dtype="mixed",
    description="one c128a layer as c128a_1m_bf16, with the mixed-precision attention cache: 448 fp8 "
                "channels (per-token scale) + the 64 rotary channels in bf16, 580 B per entry; bf16 window",
)

C128A_1M_FP4 = Workload(
    name="c128a_1m_fp4", number=8, kind="c128a", B=16, L=1 << 20, D=512, R=64, H=64, W=128,
    cache_dtype="fp4",
    description="one c128a layer as c128a_1m_bf16, with an fp4 attention cache: E2M1 codes and one E4M3 "
                "scale per 16 channels, 288 B per entry; bf16 window",
)

ALL = [TINY, C4A_128K, C128A_1M, C4A_1M_Q, MIXED_61, STREAM_C4A_128K, C128A_1M_MIXED, C128A_1M_FP4, MIXED_61_REUSE]
BY_NAME = {w.name: w for w in ALL}
