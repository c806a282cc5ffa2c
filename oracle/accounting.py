"""Cache bytes per token and per sequence for the layouts the pages size.

[P1] paragraph on the V3.2 starting point: a V3.2-style layer stores a 576-value
MLA entry plus a 128-value indexer entry per token, in bf16, over 61 layers.
[P1] paragraph on the V4 hybrid: 30 c4a layers and 31 c128a layers.
[P1] paragraph on block types: about 320 MiB per c4a layer and about 8 MiB per
c128a layer at 1M tokens. [P1] summary and key points: about 9.62 GiB per
1M-token sequence in bf16 (about 8.7x below 83.9 GiB); fp8 attention + fp4
indexer caches roughly halve that again. [P1] paragraph "c128a": at most about
8,000 entries at 1M context.

Layouts (widths D = 512 shared-state channels, Di = 128 indexer channels):
* bf16: c4a entry = (D + Di) * 2 bytes; c128a entry = D * 2 bytes.
* quantised: c4a entry = D fp8 codes + 4-byte row scale + Di/2 fp4 bytes +
  Di/16 E4M3 group scales; c128a entry = D fp8 codes + 4-byte row scale.
* mixed ([P1] mixed-precision bullet): the R rotary channels in bf16, the other
  D - R in fp8 with a 4-byte row scale.
* fp4 main rows ([P3] "Three mechanisms", third): D/2 E2M1 code bytes plus one
  E4M3 scale byte per 16 channels.
"""
from __future__ import annotations

from .method import C128A, C4A, entry_count

GiB = float(1 << 30)
MiB = float(1 << 20)


def v32_bytes_per_token_layer(mla: int = 576, indexer: int = 128, elem_bytes: int = 2) -> int:
    return (mla + indexer) * elem_bytes


def v32_sequence_bytes(tokens: int, layers: int = 61) -> int:
    return v32_bytes_per_token_layer() * tokens * layers


def entry_bytes(kind: str, D: int = 512, Di: int = 128, quantised: bool = False) -> int:
    if not quantised:
        return (D + Di) * 2 if kind == C4A else D * 2
    attn = D + 4
    return attn + Di // 2 + Di // 16 if kind == C4A else attn


def layer_bytes(kind: str, tokens: int, D: int = 512, Di: int = 128, quantised: bool = False) -> int:
    return entry_count(kind, tokens) * entry_bytes(kind, D, Di, quantised)


def v4_sequence_bytes(tokens: int, n_c4a: int = 30, n_c128a: int = 31, D: int = 512, Di: int = 128,
                      quantised: bool = False, window: int = 0) -> int:
    """Compressed caches of one sequence over the hybrid stack, plus (optionally)
    each layer's uncompressed window of ``window`` rows."""
    total = n_c4a * layer_bytes(C4A, tokens, D, Di, quantised) + n_c128a * layer_bytes(C128A, tokens, D, Di, quantised)
    row = (D + 4) if quantised else 2 * D
    return total + (n_c4a + n_c128a) * window * row


def mixed_attention_row_bytes(D: int = 512, R: int = 64) -> int:
    """An attention row: the rotary channels in bf16, every other channel an fp8 code."""
    return (D - R) + 2 * R + 4


def fp4_attention_row_bytes(D: int = 512) -> int:
    """An attention row of E2M1 codes with one E4M3 scale byte per 16 channels."""
    return D // 2 + D // 16
