"""Cache-size arithmetic of «The KV Cache and PagedAttention».

› "800 KB a Token": every token keeps one key and one value per layer, each
of `hidden` numbers; OPT-13B has 40 layers, hidden 5,120, 2 bytes a number.
› "800 KB a Token" also gives the 12 GB cache of a 40 GB card and the
resulting number of tokens and 2,048-token texts. › "What Came After": with
fewer key/value sets than heads, only the sets are stored.

Readings: KB, GB on the pages are binary (KiB, GiB). 819,200 B is exactly
800 KiB, and 12 GiB / 819,200 B is 15,728 tokens ("about 15,700"); with
decimal 12e9 B it would be 14,648.
"""
from __future__ import annotations

KIB = 1024
GIB = 1024 ** 3


def kv_bytes_per_token(layers: int, kv_numbers_per_layer: int, bytes_per_number: int) -> int:
    """One key and one value of `kv_numbers_per_layer` numbers, in every layer."""
    return 2 * kv_numbers_per_layer * layers * bytes_per_number


def kv_bytes_per_token_heads(layers: int, kv_heads: int, head_dim: int, bytes_per_number: int) -> int:
    """Same with the per-layer size given as key/value heads x head size."""
    return kv_bytes_per_token(layers, kv_heads * head_dim, bytes_per_number)


def tokens_that_fit(cache_bytes: int, bytes_per_token: int) -> int:
    return cache_bytes // bytes_per_token


def texts_that_fit(cache_bytes: int, bytes_per_token: int, text_tokens: int) -> int:
    """Texts of `text_tokens` each when every text reserves its full length."""
    return tokens_that_fit(cache_bytes, bytes_per_token) // text_tokens


def blocks_per_layer(cache_bytes: int, layers: int, kv_heads: int, head_dim: int,
                     block_size: int, bytes_per_number: int) -> int:
    """Physical blocks of one layer's key and value pools within `cache_bytes`."""
    block_bytes = 2 * kv_heads * head_dim * block_size * bytes_per_number
    return (cache_bytes // layers) // block_bytes
