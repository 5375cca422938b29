"""Prompt-phase (causal) attention over a paged KV cache, in float64.

What is computed («The KV Cache and PagedAttention» › "One Token at a Time"):
the prompt phase takes a text's whole prompt in one go, which yields every
prompt token's key and value; each token's attention needs the keys and values
of every token before it (› "What It Does") and, as in generation, its own
(«KV cache» › "How it works"). So the query at position p of a text attends
positions 0..p of that text: causal attention. The same call covers
  * a fresh prompt (the queries are all of the text's positions),
  * a prompt whose first blocks are already cached — a reused prefix
    (› "What Came After") or a text whose prompt and written tokens are
    recomputed as one new prompt (› "When Memory Runs Out"): the queries are the
    text's last n positions, and they also attend the cached positions before them.
The new tokens' keys and values are written into the cache first (as in the
generation phase), so every key and value is read through the block table.

Readings where the pages are silent:
  * the queries of text s are its last n_s positions: query i of the text sits
    at position context_len_s - n_s + i (with n_s = 1 this is generation-phase
    decode attention, oracle/attention.py);
  * queries of all texts are packed row after row; q_start[s] .. q_start[s+1]-1
    are text s's rows;
  * scale, shared key/value heads and 8-bit pools as in oracle/attention.py.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import gather_tokens, pool_values, softmax_attention, to_f64


def query_positions(context_lens, q_start):
    """(text, position) of every packed query row."""
    lens = np.asarray(context_lens, dtype=np.int64)
    qs = np.asarray(q_start, dtype=np.int64)
    rows = []
    for s in range(len(lens)):
        n = int(qs[s + 1] - qs[s])
        rows.extend((s, int(lens[s]) - n + i) for i in range(n))
    return rows


def prefill_attention(q, k_cache, v_cache, block_tables, context_lens, q_start,
                      block_size: int, scale: float | None = None, k_scale: float = 1.0,
                      v_scale: float = 1.0, rows=None) -> np.ndarray:
    """Causal paged attention of packed prompt queries: out[row, h, :] as float64.

    q: [T, H, D] with T = q_start[-1]; k_cache, v_cache: [N, H_kv, B, D];
    block_tables: [S, max_blocks]; context_lens: [S] tokens cached per text,
    the queries' own included; q_start: [S+1] row offsets, non-decreasing, with
    q_start[s+1] - q_start[s] <= context_lens[s].
    `rows`: optional list of (row, h) to compute; other outputs stay NaN.
    """
    qd = to_f64(q)
    kd = pool_values(k_cache, k_scale)
    vd = pool_values(v_cache, v_scale)
    tables = np.asarray(block_tables)
    T, H, D = qd.shape
    Hkv = kd.shape[1]
    assert H % Hkv == 0
    group = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    where = query_positions(context_lens, q_start)
    assert len(where) == T
    out = np.full((T, H, D), np.nan)
    todo = rows if rows is not None else [(r, h) for r in range(T) for h in range(H)]
    cache = {}
    for r, h in todo:
        s, p = where[r]
        key = (s, h // group)
        if key not in cache:
            L = int(np.asarray(context_lens)[s])
            cache[key] = (gather_tokens(kd, tables[s], L, block_size, h // group),
                          gather_tokens(vd, tables[s], L, block_size, h // group))
        K, V = cache[key]
        out[r, h] = softmax_attention(qd[r, h], K[:p + 1], V[:p + 1], scale)
    return out
