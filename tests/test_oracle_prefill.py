"""The oracle's prompt-phase attention against its pins, and planted mistakes caught."""
import math

import numpy as np
import pytest

import prefill_pins as pp
from oracle import attention
from oracle.prefill import prefill_attention, query_positions


@pytest.mark.parametrize("check", pp.CHECKS, ids=lambda c: c.__name__)
def test_oracle_passes(check):
    check(prefill_attention)


def test_query_positions_are_the_last_positions():
    assert query_positions([5, 3, 4], [0, 2, 2, 6]) == [(0, 3), (0, 4), (2, 0), (2, 1), (2, 2), (2, 3)]


def test_unused_places_are_never_read():
    ctx, new = [7, 5], [3, 5]
    a = pp.make_case(2, ctx, new, fill=np.nan)
    b = pp.make_case(2, ctx, new, fill=0.0)
    oa = prefill_attention(a[0], a[3], a[4], a[5], ctx, a[6], 4)
    ob = prefill_attention(b[0], b[3], b[4], b[5], ctx, b[6], 4)
    assert np.isfinite(oa).all() and np.array_equal(oa, ob)


def _variant(limit=lambda p: p + 1, pos=None, head=lambda h, G, Hkv: h // G):
    """prefill written again with one step replaceable (for planted mistakes)."""
    def fn(q, kc, vc, tables, ctx, q_start, B, scale=None):
        qd = attention.to_f64(q)
        T, H, D = qd.shape
        Hkv = kc.shape[1]
        G = H // Hkv
        out = np.full((T, H, D), np.nan)
        for s in range(len(ctx)):
            n = int(q_start[s + 1] - q_start[s])
            for i in range(n):
                p = pos(ctx[s], n, i) if pos else ctx[s] - n + i
                for h in range(H):
                    K = attention.gather_tokens(kc, tables[s], ctx[s], B, head(h, G, Hkv))
                    V = attention.gather_tokens(vc, tables[s], ctx[s], B, head(h, G, Hkv))
                    m = max(0, min(limit(p), ctx[s]))
                    out[q_start[s] + i, h] = attention.softmax_attention(
                        qd[q_start[s] + i, h], K[:m], V[:m], 1 / math.sqrt(D))
        return out
    return fn


MUTANTS = {
    "excludes_own_key": _variant(limit=lambda p: p),
    "sees_next_key": _variant(limit=lambda p: p + 2),
    "no_causal_mask": _variant(limit=lambda p: 10 ** 9),
    "queries_at_first_positions": _variant(pos=lambda L, n, i: i),
    "shared_head_modulo": _variant(head=lambda h, G, Hkv: h % Hkv),
}


def test_variant_without_mistake_passes():
    for check in pp.CHECKS:
        check(_variant())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    caught = []
    for check in pp.CHECKS:
        try:
            check(MUTANTS[name])
        except (AssertionError, IndexError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin caught {name}"
