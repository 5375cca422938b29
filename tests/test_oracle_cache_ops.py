"""The oracle's cache writes against flat-memory brute force and exact facts.

The brute force addresses the pool as one flat array with the row-major
offset ((block * H_kv + head) * B + place) * D + d, a different formulation
of the layout than the models' tensor indexing, so a swapped index in a
model shows up here.
"""
import numpy as np
import torch

from oracle import cache_ops
from oracle.allocator import BlockAllocator
from oracle.attention import gather_tokens


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _pool(N, H, B, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((N, H, B, D), generator=g).to(dtype)


def test_kv_write_flat_brute_force():
    for dtype in (torch.float32, torch.float16, torch.bfloat16):
        N, H, B, D = 7, 3, 4, 8
        kc, vc = _pool(N, H, B, D, dtype, 1), _pool(N, H, B, D, dtype, 2)
        k_flat = kc.clone().reshape(-1)
        v_flat = vc.clone().reshape(-1)
        g = torch.Generator().manual_seed(3)
        T = 9
        kn = torch.randn((T, H, D), generator=g).to(dtype)
        vn = torch.randn((T, H, D), generator=g).to(dtype)
        slots = list(np.random.default_rng(4).choice(N * B, size=T, replace=False))
        cache_ops.kv_write(kc, vc, kn, vn, slots, B)
        for i, slot in enumerate(slots):
            blk, place = int(slot) // B, int(slot) % B
            for h in range(H):
                for d in range(D):
                    off = ((blk * H + h) * B + place) * D + d
                    k_flat[off] = kn[i, h, d]
                    v_flat[off] = vn[i, h, d]
        assert torch.equal(_bits(kc.reshape(-1)), _bits(k_flat))
        assert torch.equal(_bits(vc.reshape(-1)), _bits(v_flat))


def test_kv_write_keeps_bit_patterns():
    """A write moves bits: NaN payloads, -0.0 and subnormals arrive unchanged."""
    N, H, B, D = 2, 1, 4, 4
    kc = torch.zeros((N, H, B, D), dtype=torch.float16)
    vc = torch.zeros((N, H, B, D), dtype=torch.float16)
    pattern = torch.tensor([0x7E01, 0x8000, 0x0001, 0xFC00], dtype=torch.int32).to(torch.int16)
    kn = pattern.view(torch.float16).reshape(1, 1, D)
    cache_ops.kv_write(kc, vc, kn, kn.clone(), [5], B)
    assert torch.equal(_bits(kc[1, 0, 1]), pattern)
    assert torch.equal(_bits(vc[1, 0, 1]), pattern)


def test_write_then_gather_is_identity():
    """Tokens written to the slots the allocator hands out read back in order."""
    rng = np.random.default_rng(5)
    B, H, D, N = 4, 2, 8, 32
    a = BlockAllocator(N, B, rng.permutation(N))
    kc = torch.full((N, H, B, D), float("nan"), dtype=torch.float64)
    vc = kc.clone()
    logical = {}
    for L in (1, 4, 9, 14):
        sid = a.add()
        k = torch.randn(L, H, D, dtype=torch.float64)
        v = torch.randn(L, H, D, dtype=torch.float64)
        slots, pair = a.append(sid, L)
        assert pair == (-1, -1)
        cache_ops.kv_write(kc, vc, k, v, slots, B)
        logical[sid] = (k, v)
    for sid, (k, v) in logical.items():
        tables, lens = a.export([sid], 8)
        for h in range(H):
            got_k = gather_tokens(kc.numpy(), tables[0], lens[0], B, h)
            got_v = gather_tokens(vc.numpy(), tables[0], lens[0], B, h)
            assert np.array_equal(got_k, k[:, h].numpy())
            assert np.array_equal(got_v, v[:, h].numpy())


def test_copy_blocks_whole_block_and_order():
    N, H, B, D = 6, 2, 4, 4
    kc, vc = _pool(N, H, B, D, torch.bfloat16, 7), _pool(N, H, B, D, torch.bfloat16, 8)
    k0, v0 = kc.clone(), vc.clone()
    cache_ops.copy_blocks(kc, vc, [(1, 4), (4, 5), (2, 0)])
    assert torch.equal(_bits(kc[4]), _bits(k0[1])) and torch.equal(_bits(vc[4]), _bits(v0[1]))
    assert torch.equal(_bits(kc[5]), _bits(k0[1])), "pairs apply in order"
    assert torch.equal(_bits(kc[0]), _bits(k0[2])) and torch.equal(_bits(vc[0]), _bits(v0[2]))
    for b in (1, 2, 3):
        assert torch.equal(_bits(kc[b]), _bits(k0[b])) and torch.equal(_bits(vc[b]), _bits(v0[b]))
