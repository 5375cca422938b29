"""Facts that pin the oracle's prompt-phase (causal) attention to something else.

Each check takes a prefill attention function with the signature of
oracle.prefill.prefill_attention (the oracle's, or a deliberately broken
variant) and raises AssertionError when it disagrees with:
  * torch's scaled_dot_product_attention in float64 with is_causal=True on
    fresh prompts held contiguously (a library routine);
  * the generation-phase oracle, itself pinned separately: a query at position
    p equals decode attention over the text's first p + 1 tokens;
  * brute force with Python loops on tiny inputs;
  * causality: keys and values after a query's position do not move it, and
    the first position of a fresh prompt returns its own value exactly;
  * block placement («The KV Cache and PagedAttention» › "The Block Table").
"""
from __future__ import annotations

import math

import numpy as np
import torch

from pins import _scatter, brute_force


def make_case(seed, ctx, new, H=2, Hkv=2, D=8, B=4, extra_blocks=5, fill=np.nan):
    """Texts with ctx[s] cached tokens, the last new[s] of which are the prompt's queries."""
    rng = np.random.default_rng(seed)
    lk = [rng.standard_normal((L, Hkv, D)) for L in ctx]
    lv = [rng.standard_normal((L, Hkv, D)) for L in ctx]
    q_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int64)
    q = rng.standard_normal((int(q_start[-1]), H, D))
    nb = sum((L + B - 1) // B for L in ctx) + extra_blocks
    kc, vc, tables = _scatter(lk, lv, ctx, B, nb, rng, fill=fill)
    return q, lk, lv, kc, vc, tables, q_start


def check_sdpa_causal(fn):
    """Fresh prompts (every position a query) against SDPA with is_causal=True."""
    ctx = [1, 7, 16, 21]
    H, Hkv, D, B = 4, 2, 16, 4
    q, lk, lv, kc, vc, tables, q_start = make_case(3, ctx, ctx, H=H, Hkv=Hkv, D=D, B=B)
    out = fn(q, kc, vc, tables, ctx, q_start, B)
    G = H // Hkv
    for s, L in enumerate(ctx):
        K = torch.from_numpy(lk[s]).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        V = torch.from_numpy(lv[s]).repeat_interleave(G, dim=1).permute(1, 0, 2).contiguous()
        Q = torch.from_numpy(q[q_start[s]:q_start[s + 1]]).permute(1, 0, 2).contiguous()
        want = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
        np.testing.assert_allclose(out[q_start[s]:q_start[s + 1]], want.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def check_decode_consistency(fn):
    """Query at position p == generation-phase attention over the first p + 1 tokens."""
    from oracle.attention import decode_attention
    ctx = [9, 14, 5, 30]
    new = [3, 14, 0, 7]      # cached prefixes 6, 0, 5, 23
    H, Hkv, D, B = 4, 1, 8, 4
    q, lk, lv, kc, vc, tables, q_start = make_case(8, ctx, new, H=H, Hkv=Hkv, D=D, B=B)
    out = fn(q, kc, vc, tables, ctx, q_start, B)
    for s, L in enumerate(ctx):
        for i in range(new[s]):
            r = q_start[s] + i
            p = L - new[s] + i
            want = decode_attention(q[r:r + 1], kc, vc, tables[s:s + 1], [p + 1], B)
            np.testing.assert_allclose(out[r], want[0], rtol=0, atol=1e-12)


def check_brute_force(fn):
    ctx, new = [5, 9], [5, 4]
    q, lk, lv, kc, vc, tables, q_start = make_case(17, ctx, new, H=3, Hkv=3, D=4, B=4)
    out = fn(q, kc, vc, tables, ctx, q_start, 4)
    scale = 1 / math.sqrt(4)
    for s, L in enumerate(ctx):
        for i in range(new[s]):
            p = L - new[s] + i
            for h in range(3):
                want = brute_force(q[q_start[s] + i, h], lk[s][:p + 1, h], lv[s][:p + 1, h], scale)
                np.testing.assert_allclose(out[q_start[s] + i, h], want, rtol=0, atol=1e-12)


def check_later_tokens_do_not_matter(fn):
    """Changing keys and values after position p leaves the query at p bit-identical."""
    ctx, new = [12, 8], [12, 5]
    q, lk, lv, kc, vc, tables, q_start = make_case(21, ctx, new)
    base = fn(q, kc, vc, tables, ctx, q_start, 4)
    k2, v2 = kc.copy(), vc.copy()
    for s, L in enumerate(ctx):
        cut = L - 2            # positions cut+1 .. L-1 change
        for t in range(cut + 1, L):
            b = tables[s, t // 4]
            k2[b, :, t % 4] += 3.0
            v2[b, :, t % 4] -= 5.0
    moved = fn(q, k2, v2, tables, ctx, q_start, 4)
    for s, L in enumerate(ctx):
        for i in range(new[s]):
            r, p = q_start[s] + i, L - new[s] + i
            if p <= L - 2:
                assert np.array_equal(base[r], moved[r]), (s, i)
            else:
                assert not np.allclose(base[r], moved[r]), (s, i)


def check_first_position_is_its_value(fn):
    ctx = [6, 3]
    q, lk, lv, kc, vc, tables, q_start = make_case(4, ctx, ctx)
    out = fn(q, kc, vc, tables, ctx, q_start, 4)
    for s in range(len(ctx)):
        assert np.array_equal(out[q_start[s]], lv[s][0])


def check_placement_permutation(fn):
    ctx, new = [10, 7], [4, 7]
    q, lk, lv, kc, vc, tables, q_start = make_case(6, ctx, new, extra_blocks=6)
    base = fn(q, kc, vc, tables, ctx, q_start, 4)
    perm = np.random.default_rng(0).permutation(kc.shape[0])
    k2, v2 = np.empty_like(kc), np.empty_like(vc)
    k2[perm], v2[perm] = kc, vc
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = fn(q, k2, v2, t2, ctx, q_start, 4)
    assert np.array_equal(base, moved)


CHECKS = [check_sdpa_causal, check_decode_consistency, check_brute_force,
          check_later_tokens_do_not_matter, check_first_position_is_its_value,
          check_placement_permutation]
