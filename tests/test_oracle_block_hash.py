"""The oracle's chained block hash: FNV-1a's published test values and the chain's
defining properties (a block's hash depends on its tokens and everything before)."""
import numpy as np

from oracle.block_hash import block_hashes, fnv1a64


def test_fnv1a64_published_values():
    # test values published with the FNV-1a algorithm (64-bit)
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_one_block_is_fnv_of_parent_and_tokens():
    toks = [1, 2, 0x01020304, -1]
    want = fnv1a64(bytes(8) + bytes([1, 0, 0, 0, 2, 0, 0, 0, 4, 3, 2, 1, 255, 255, 255, 255]))
    assert block_hashes(toks, 4) == [want]


def test_only_full_blocks_are_hashed():
    assert len(block_hashes(list(range(11)), 4)) == 2
    assert block_hashes([], 4) == [] and block_hashes([5, 6, 7], 4) == []


def test_chain_depends_on_everything_before():
    rng = np.random.default_rng(0)
    a = [int(x) for x in rng.integers(0, 50000, 64)]
    b = list(a)
    b[21] += 1                       # block 5 of 16 (block size 4) differs
    ha, hb = block_hashes(a, 4), block_hashes(b, 4)
    assert ha[:5] == hb[:5]
    assert all(x != y for x, y in zip(ha[5:], hb[5:]))
    # the same block content after a different history hashes differently
    c = [7, 7, 7, 7] + a[4:8]
    d = [8, 8, 8, 8] + a[4:8]
    assert block_hashes(c, 4)[1] != block_hashes(d, 4)[1]


def test_parent_continues_the_chain():
    toks = list(range(40))
    full = block_hashes(toks, 8)
    assert block_hashes(toks[16:], 8, parent=full[1]) == full[2:]
