"""Byte accounting of the global cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[FP4] section "Le coût d'une entrée": an entry of C channels with 4-bit
values and one scale byte per block of b channels costs C*4/8 + (C/b)*1
bytes. [FP4] section "Le compte par couche": a layer of ratio m costs
entry/m bytes per token; the four source layers (three at ratio 2, one at
ratio 1) give the per-token total. [FP4] section "Ce que cela donne aux
échelles réelles" multiplies by the context length. [FP4] sections "Le
facteur 437 contre DeepSeek-V1" and "La contrepartie : la fenêtre glissante"
give a BF16 GQA cache and an FP8 sliding-window cache in the same units.
"""
from fractions import Fraction


def entry_bytes(channels, block, scale_bytes=1, value_bits=4):
    """Bytes of one cache entry: packed values plus one scale per block (0 = no scales)."""
    data = Fraction(channels * value_bits, 8)
    scales = Fraction(channels, block) * scale_bytes if block else 0
    return data + scales


def layer_bytes_per_token(ratio, lat=(512, 16, 1), idx=(128, 32, 1)):
    """Amortised bytes per token of one source layer of the given ratio."""
    return (entry_bytes(*lat) + entry_bytes(*idx)) / ratio


def bytes_per_token(ratios, lat=(512, 16, 1), idx=(128, 32, 1)):
    """Global-cache bytes per token for source layers with the given ratios."""
    return sum(layer_bytes_per_token(r, lat, idx) for r in ratios)


def cache_bytes(context_tokens, per_token):
    return context_tokens * per_token


def gqa_bf16_bytes_per_token(layers, kv_heads, head_dim, elem_bytes=2):
    """Keys and values of a plain GQA cache."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def sliding_window_bytes(layers, window, channels, block, elem_bytes=1, scale_bytes=1):
    """Per-sequence sliding-window cache: window tokens per layer, values plus block scales."""
    return layers * window * (channels * elem_bytes + (channels // block) * scale_bytes)
