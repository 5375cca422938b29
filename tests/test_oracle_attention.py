"""The oracle's attention against brute force, a library routine and exact facts."""
import numpy as np
import pytest

import pins
from oracle import attention


@pytest.mark.parametrize("check", pins.ATTENTION_CHECKS, ids=lambda c: c.__name__)
def test_oracle_attention_pin(check):
    check(attention.decode_attention)


def test_contiguous_matches_paged():
    """contiguous_attention is the same definition on an unpaged text."""
    rng = np.random.default_rng(0)
    L, H, D, B = 19, 4, 8, 4
    K = rng.standard_normal((L, 2, D))
    V = rng.standard_normal((L, 2, D))
    q = rng.standard_normal((H, D))
    kc, vc, tables = pins._scatter([K], [V], [L], B, 8, rng)
    paged = attention.decode_attention(q[None], kc, vc, tables, [L], B)[0]
    np.testing.assert_allclose(attention.contiguous_attention(q, K, V), paged, rtol=0, atol=1e-13)


def test_pairs_subset_is_same_values():
    rng = np.random.default_rng(1)
    q, lk, lv, kc, vc, tables = pins._random_case(21, [5, 9], H=2, Hkv=2)
    full = attention.decode_attention(q, kc, vc, tables, [5, 9], 4)
    part = attention.decode_attention(q, kc, vc, tables, [5, 9], 4, pairs=[(1, 0)])
    assert np.array_equal(part[1, 0], full[1, 0])
    assert np.isnan(part[0, 0]).all()
