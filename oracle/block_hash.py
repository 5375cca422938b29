"""Chained block hashes for reusing cached prompt prefixes (oracle side).

«The KV Cache and PagedAttention» › "What Came After": with automatic prefix
caching every full block gets a hash of its tokens and of everything before
them, and a new request that begins with the same tokens reuses those blocks.

The pages name no hash function. Reading taken: 64-bit FNV-1a (Fowler, Noll
and Vo; offset basis 0xcbf29ce484222325, prime 0x100000001b3, each byte xored
in, then a multiplication modulo 2^64), chained block by block:

    h_j = FNV-1a( le64(h_{j-1}) || le32(t_{jB}) || ... || le32(t_{jB+B-1}) ),  h_{-1} = parent

with token ids as 32-bit little-endian integers and parent = 0 at a text's start.
Only full blocks are hashed. Written from that definition, byte by byte.
"""
from __future__ import annotations

from typing import List, Sequence

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    h = FNV64_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & MASK64
    return h


def block_hashes(tokens: Sequence[int], block_size: int, parent: int = 0) -> List[int]:
    """Chained hashes of the full blocks of `tokens` (len(tokens) // block_size of them)."""
    out = []
    h = parent & MASK64
    for j in range(len(tokens) // block_size):
        data = h.to_bytes(8, "little")
        for t in tokens[j * block_size:(j + 1) * block_size]:
            data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
        h = fnv1a64(data)
        out.append(h)
    return out
