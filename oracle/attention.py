"""Generation-phase attention over a paged KV cache, in float64.

What is computed («KV cache» › "How it works"; «The KV Cache and
PagedAttention» › "One Token at a Time"): in one generation step the new
position's query is compared with the key of every cached position of its
text, its own key included, and the resulting softmax weights mix the
values. Paging changes only where those keys and values are stored
(› "Like Pages of Memory", › "The Block Table"): a text's logical block j
lives in whatever physical block its block table names, and the attention
reads each block through that table. So the result is exactly the textbook
softmax(q K^T * scale) V over the text's tokens in logical order.

Readings where the pages are silent:
  * scale = 1/sqrt(head_dim) unless given (the pages defer the attention
    formula to a plate that is not included);
  * heads are independent; with fewer key/value heads than query heads
    (heads sharing one set of keys and values, › "What Came After"), query
    head h reads key/value head h // (num_heads // num_kv_heads);
  * a text with no cached token yields zeros;
  * pools stored in 8-bit floating point (uint8 codes, see oracle/fp8.py) hold
    decode(code) * scale, with one scale for the key pool and one for the value
    pool; attention runs on those values.
"""
from __future__ import annotations

import math

import numpy as np


def to_f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or torch CPU tensor (fp16/bf16/fp32)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def gather_tokens(pool: np.ndarray, table_row, ctx_len: int, block_size: int,
                  kv_head: int) -> np.ndarray:
    """Keys (or values) of one text and head, in logical token order.

    pool: [num_blocks, num_kv_heads, block_size, head_dim]. Token t of the
    text sits in logical block t // block_size at place t % block_size; the
    table maps the logical block to its physical block (› "The Block Table").
    """
    t = np.arange(ctx_len)
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return pool[phys, kv_head, t % block_size, :]


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Textbook attention of one query over L keys/values (all float64).

    z_t = scale * <q, K_t>;  p = softmax(z);  out = sum_t p_t V_t.
    The maximum is subtracted before exponentiating; this changes nothing in
    exact arithmetic and keeps exp in range.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    p = w / w.sum()
    return p @ V


def pool_values(pool, pool_scale: float = 1.0) -> np.ndarray:
    """float64 values of a key or value pool; uint8 pools are E4M3 codes times pool_scale."""
    try:
        import torch
        if isinstance(pool, torch.Tensor) and pool.dtype == torch.uint8:
            pool = pool.numpy()
    except ImportError:  # pragma: no cover
        pass
    if isinstance(pool, np.ndarray) and pool.dtype == np.uint8:
        from . import fp8
        return fp8.dequantize(pool, pool_scale)
    return to_f64(pool)


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, block_size: int,
                     scale: float | None = None, pairs=None, k_scale: float = 1.0,
                     v_scale: float = 1.0) -> np.ndarray:
    """Paged decode attention for a batch: out[s, h, :] as float64.

    q: [S, H, D]; k_cache, v_cache: [N, H_kv, B, D]; block_tables: [S, max_blocks]
    (entries past a text's last block are never read); context_lens: [S], the
    number of tokens each text attends, counting the step's new token.
    k_scale, v_scale: pool scales, used when the pools hold uint8 E4M3 codes.
    `pairs`: optional list of (s, h) to compute; other outputs stay NaN.
    """
    qd = to_f64(q)
    kd = pool_values(k_cache, k_scale)
    vd = pool_values(v_cache, v_scale)
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens, dtype=np.int64)
    S, H, D = qd.shape
    Hkv = kd.shape[1]
    assert H % Hkv == 0, "query heads must be a multiple of key/value heads"
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.full((S, H, D), np.nan)
    todo = pairs if pairs is not None else [(s, h) for s in range(S) for h in range(H)]
    for s, h in todo:
        L = int(lens[s])
        K = gather_tokens(kd, tables[s], L, block_size, h // group)
        V = gather_tokens(vd, tables[s], L, block_size, h // group)
        out[s, h] = softmax_attention(qd[s, h], K, V, scale)
    return out


def contiguous_attention(q, K, V, scale: float | None = None) -> np.ndarray:
    """Attention of one text held contiguously (no paging): q [H, D], K/V [L, H_kv, D]."""
    qd, Kd, Vd = to_f64(q), to_f64(K), to_f64(V)
    H, D = qd.shape
    group = H // Kd.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return np.stack([softmax_attention(qd[h], Kd[:, h // group], Vd[:, h // group], scale)
                     for h in range(H)])


def max_abs_error(got, want: np.ndarray) -> float:
    """max |got - want| over all elements, got converted exactly to float64."""
    g = to_f64(got)
    return float(np.max(np.abs(g - want))) if want.size else 0.0
