"""Facts that pin the oracle's attention to something other than itself.

Each check takes the attention function under test (the oracle's
`decode_attention`, or a deliberately broken copy of it) and raises
AssertionError when the function disagrees with:
  * brute force: pure-Python loops over the text held contiguously, never
    paged (the paging must not change the result);
  * a library routine: torch's scaled_dot_product_attention in float64 on the
    contiguous text (the textbook definition, independent of this code);
  * closed forms and exact invariants of softmax attention;
  * the pages' statement that blocks need not sit next to each other
    («The KV Cache and PagedAttention» › "The Block Table").
"""
from __future__ import annotations

import math

import numpy as np
import torch


def _scatter(logical_k, logical_v, lens, block_size, num_blocks, rng, fill=np.nan):
    """Place each text's tokens into randomly chosen physical blocks.

    Returns (k_cache, v_cache, tables) in float64. logical_*: list per text of
    [L, H_kv, D]. Uses its own layout arithmetic so a gather bug in the code
    under test cannot cancel against it.
    """
    Hkv, D = logical_k[0].shape[1], logical_k[0].shape[2]
    kc = np.full((num_blocks, Hkv, block_size, D), fill)
    vc = np.full((num_blocks, Hkv, block_size, D), fill)
    perm = list(rng.permutation(num_blocks))
    maxb = max(1, max((L + block_size - 1) // block_size for L in lens))
    tables = np.full((len(lens), maxb), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        for j in range((L + block_size - 1) // block_size):
            tables[s, j] = perm.pop()
        for t in range(L):
            b = tables[s, t // block_size]
            for hk in range(Hkv):
                kc[b, hk, t % block_size, :] = logical_k[s][t, hk]
                vc[b, hk, t % block_size, :] = logical_v[s][t, hk]
    return kc, vc, tables


def _random_case(seed, lens, H=2, Hkv=2, D=8, B=4, extra_blocks=5):
    rng = np.random.default_rng(seed)
    lk = [rng.standard_normal((L, Hkv, D)) for L in lens]
    lv = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((len(lens), H, D))
    nb = sum((L + B - 1) // B for L in lens) + extra_blocks
    kc, vc, tables = _scatter(lk, lv, lens, B, nb, rng)
    return q, lk, lv, kc, vc, tables


def brute_force(q_vec, K, V, scale):
    """softmax(scale * q.K) . V with Python loops and math.exp."""
    L, D = len(K), len(q_vec)
    scores = []
    for t in range(L):
        acc = 0.0
        for d in range(D):
            acc += float(q_vec[d]) * float(K[t][d])
        scores.append(scale * acc)
    m = max(scores)
    w = [math.exp(z - m) for z in scores]
    tot = sum(w)
    return [sum(w[t] / tot * float(V[t][d]) for t in range(L)) for d in range(D)]


def check_brute_force(fn):
    for lens, H, Hkv, B in (([1, 5, 9], 2, 2, 4), ([7, 16, 3], 4, 2, 4), ([11, 2], 3, 1, 8)):
        q, lk, lv, kc, vc, tables = _random_case(11 + len(lens) + H, lens, H=H, Hkv=Hkv, B=B)
        out = fn(q, kc, vc, tables, lens, B)
        G = H // Hkv
        scale = 1.0 / math.sqrt(q.shape[-1])
        for s, L in enumerate(lens):
            for h in range(H):
                want = brute_force(q[s, h], lk[s][:, h // G], lv[s][:, h // G], scale)
                np.testing.assert_allclose(out[s, h], want, rtol=0, atol=1e-12)


def check_sdpa(fn):
    """Agreement with torch.nn.functional.scaled_dot_product_attention (fp64, CPU)."""
    lens = [3, 17, 32, 1]
    H, Hkv, D, B = 4, 2, 16, 4
    q, lk, lv, kc, vc, tables = _random_case(5, lens, H=H, Hkv=Hkv, D=D, B=B)
    out = fn(q, kc, vc, tables, lens, B)
    G = H // Hkv
    for s, L in enumerate(lens):
        K = torch.from_numpy(lk[s]).repeat_interleave(G, dim=1).permute(1, 0, 2)  # [H, L, D]
        V = torch.from_numpy(lv[s]).repeat_interleave(G, dim=1).permute(1, 0, 2)
        Q = torch.from_numpy(q[s]).unsqueeze(1)                                     # [H, 1, D]
        want = torch.nn.functional.scaled_dot_product_attention(Q, K.contiguous(), V.contiguous())
        np.testing.assert_allclose(out[s], want[:, 0].numpy(), rtol=0, atol=1e-12)


def check_placement_permutation(fn):
    """Moving blocks to other physical places (and the tables with them) changes no bit."""
    lens = [6, 13, 4]
    B = 4
    q, lk, lv, kc, vc, tables = _random_case(7, lens, B=B, extra_blocks=7)
    base = fn(q, kc, vc, tables, lens, B)
    rng = np.random.default_rng(99)
    pi = rng.permutation(kc.shape[0])           # old block b moves to pi[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = fn(q, kc2, vc2, t2, lens, B)
    assert np.array_equal(base, moved), "placement changed the result"


def check_equal_keys_mean(fn):
    """Identical keys give equal weights: the output is the mean of the values."""
    rng = np.random.default_rng(3)
    lens = [9, 22]
    B, H, D = 4, 2, 8
    lk = []
    for L in lens:
        k = np.broadcast_to(rng.standard_normal((1, H, D)), (L, H, D)).copy()
        lk.append(k)
    lv = [rng.standard_normal((L, H, D)) for L in lens]
    q = rng.standard_normal((len(lens), H, D))
    kc, vc, tables = _scatter(lk, lv, lens, B, 20, rng)
    out = fn(q, kc, vc, tables, lens, B)
    for s in range(len(lens)):
        want = lv[s].mean(axis=0)
        np.testing.assert_allclose(out[s], want, rtol=1e-14, atol=1e-15)


def check_single_token(fn):
    """With one cached token the weight is exactly 1: out == v_0 bit for bit."""
    rng = np.random.default_rng(4)
    lk = [rng.standard_normal((1, 2, 8))]
    lv = [rng.standard_normal((1, 2, 8))]
    q = rng.standard_normal((1, 2, 8)) * 50.0
    kc, vc, tables = _scatter(lk, lv, [1], 4, 3, rng)
    out = fn(q, kc, vc, tables, [1], 4)
    assert np.array_equal(out[0], lv[0][0]), "single token must return its value exactly"


def check_dominant_new_token(fn):
    """A last-token key far along q takes all the weight: out ~= v of the new token."""
    rng = np.random.default_rng(6)
    lens = [13, 5]
    B, H, D = 4, 2, 8
    q = rng.standard_normal((len(lens), H, D))
    lk = [rng.standard_normal((L, H, D)) * 0.1 for L in lens]
    lv = [rng.standard_normal((L, H, D)) for L in lens]
    for s, L in enumerate(lens):
        lk[s][L - 1] = 40.0 * q[s] / np.linalg.norm(q[s], axis=-1, keepdims=True)
    kc, vc, tables = _scatter(lk, lv, lens, B, 12, rng)
    out = fn(q, kc, vc, tables, lens, B)
    for s, L in enumerate(lens):
        np.testing.assert_allclose(out[s], lv[s][L - 1], rtol=0, atol=1e-6)


def check_key_shift(fn):
    """Adding one vector c to every key shifts all scores equally: no change."""
    lens = [10, 3]
    B = 4
    q, lk, lv, kc, vc, tables = _random_case(8, lens, B=B)
    base = fn(q, kc, vc, tables, lens, B)
    c = np.random.default_rng(1).standard_normal((kc.shape[1], kc.shape[3]))
    shifted = fn(q, kc + c[None, :, None, :], vc, tables, lens, B)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-12)


def check_value_affine(fn):
    """out(a V + b) = a out(V) + b (the weights sum to one)."""
    lens = [10, 7]
    B = 4
    q, lk, lv, kc, vc, tables = _random_case(9, lens, B=B)
    base = fn(q, kc, vc, tables, lens, B)
    b = np.random.default_rng(2).standard_normal((vc.shape[1], vc.shape[3]))
    got = fn(q, kc, -2.5 * vc + b[None, :, None, :], tables, lens, B)
    want = -2.5 * base + np.repeat(b, q.shape[1] // b.shape[0], axis=0)[None]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def check_block_size_invariance(fn):
    """The same logical text stored in blocks of 4 or of 16 gives the same output."""
    lens = [37, 5, 16]
    rng = np.random.default_rng(12)
    H, D = 2, 8
    lk = [rng.standard_normal((L, H, D)) for L in lens]
    lv = [rng.standard_normal((L, H, D)) for L in lens]
    q = rng.standard_normal((len(lens), H, D))
    k4, v4, t4 = _scatter(lk, lv, lens, 4, 40, rng)
    k16, v16, t16 = _scatter(lk, lv, lens, 16, 10, rng)
    np.testing.assert_allclose(fn(q, k4, v4, t4, lens, 4), fn(q, k16, v16, t16, lens, 16),
                               rtol=0, atol=1e-13)


def check_unused_places_never_read(fn):
    """NaN in every unfilled place and unused block leaves the output finite."""
    lens = [6, 9]
    B = 4
    q, lk, lv, kc, vc, tables = _random_case(13, lens, B=B)
    out = fn(q, kc, vc, tables, lens, B)   # _scatter fills unused places with NaN
    assert np.isfinite(out).all()


def check_empty_text(fn):
    rng = np.random.default_rng(14)
    lens = [0, 3]
    lk = [rng.standard_normal((L, 2, 8)) for L in lens]
    lv = [rng.standard_normal((L, 2, 8)) for L in lens]
    q = rng.standard_normal((2, 2, 8))
    kc, vc, tables = _scatter(lk, lv, lens, 4, 4, rng)
    out = fn(q, kc, vc, tables, lens, 4)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


ATTENTION_CHECKS = [
    check_brute_force, check_sdpa, check_placement_permutation, check_equal_keys_mean,
    check_single_token, check_dominant_new_token, check_key_shift, check_value_affine,
    check_block_size_invariance, check_unused_places_never_read, check_empty_text,
]
