"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

A pin set that lets a dropped term, a wrong index, a wrong scale or a swapped
operand through would not pin anything; every mutant below must fail at
least one of the attention checks.
"""
import math

import numpy as np
import pytest

import pins
from oracle import attention


def _fails_some_check(monkeypatch, name, fake):
    monkeypatch.setattr(attention, name, fake)
    caught = []
    for check in pins.ATTENTION_CHECKS:
        try:
            check(attention.decode_attention)
        except (AssertionError, IndexError, ValueError):
            caught.append(check.__name__)
    return caught


def _gather_swapped(pool, table_row, L, B, kvh):          # block and place swapped
    t = np.arange(L)
    phys = np.asarray(table_row, dtype=np.int64)[np.minimum(t % B, len(table_row) - 1)]
    return pool[phys, kvh, np.minimum(t // B, pool.shape[2] - 1), :]


def _gather_drop_last(pool, table_row, L, B, kvh):        # new token not attended
    t = np.arange(max(L - 1, 0) if L > 1 else L)
    phys = np.asarray(table_row, dtype=np.int64)[t // B]
    return pool[phys, kvh, t % B, :]


def _gather_first_block_only(pool, table_row, L, B, kvh):  # ignores the table past entry 0
    t = np.arange(L)
    phys = np.full(L, int(table_row[0]), dtype=np.int64)
    return pool[phys, kvh, t % B, :]


def _softmax_wrong_scale(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = (K @ q) / q.shape[0]
    w = np.exp(z - z.max())
    return (w / w.sum()) @ V


def _softmax_unnormalised(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ q)
    return np.exp(z - z.max()) @ V


def _softmax_mixes_keys(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w / w.sum()) @ K


def _softmax_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = -scale * (K @ q)
    w = np.exp(z - z.max())
    return (w / w.sum()) @ V


MUTANTS = [
    ("gather_tokens", _gather_swapped),
    ("gather_tokens", _gather_drop_last),
    ("gather_tokens", _gather_first_block_only),
    ("softmax_attention", _softmax_wrong_scale),
    ("softmax_attention", _softmax_unnormalised),
    ("softmax_attention", _softmax_mixes_keys),
    ("softmax_attention", _softmax_sign),
]


@pytest.mark.parametrize("name,fake", MUTANTS, ids=lambda x: getattr(x, "__name__", str(x)))
def test_mutant_is_caught(monkeypatch, name, fake):
    caught = _fails_some_check(monkeypatch, name, fake)
    assert caught, f"no pin caught mutant {fake.__name__}"


def test_gqa_mapping_mutant_is_caught(monkeypatch):
    """Query head h must read key/value head h // group, not h % H_kv."""
    real = attention.decode_attention

    def wrong(q, k_cache, v_cache, block_tables, context_lens, block_size, scale=None, pairs=None):
        qd, kd, vd = attention.to_f64(q), attention.to_f64(k_cache), attention.to_f64(v_cache)
        S, H, D = qd.shape
        Hkv = kd.shape[1]
        out = np.full((S, H, D), np.nan)
        for s in range(S):
            for h in range(H):
                L = int(context_lens[s])
                K = attention.gather_tokens(kd, block_tables[s], L, block_size, h % Hkv)
                V = attention.gather_tokens(vd, block_tables[s], L, block_size, h % Hkv)
                out[s, h] = attention.softmax_attention(qd[s, h], K, V, 1 / math.sqrt(D))
        return out

    with pytest.raises(AssertionError):
        pins.check_brute_force(wrong)
    pins.check_brute_force(real)
