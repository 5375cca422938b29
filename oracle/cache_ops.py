"""Byte-level models of the two cache writes, on torch CPU tensors.

kv_write — «The KV Cache and PagedAttention» › "One Token at a Time": each
generation step computes only the new token's key and value and adds them
to the cache; «KV cache» › "How it works": the new key and value are
written into the cache. With paging the token's place is its slot:
physical block * block_size + place in block (› "The Block Table").

copy_blocks — › "Shared, Copied on Write": before a text writes into a block
it shares, the block is copied and the write goes to the copy. The copy
takes the whole block, keys and values, so the copy holds the same filled
places as the original.

Both are pure moves of stored numbers: the models copy element bit
patterns and never convert them.
"""
from __future__ import annotations


def kv_write(k_cache, v_cache, k_new, v_new, slots, block_size: int) -> None:
    """In place: for token i, k_cache[slot_i // B, :, slot_i % B, :] = k_new[i] (same for v).

    k_cache, v_cache: [N, H_kv, B, D]; k_new, v_new: [T, H_kv, D]; slots: T ints.
    Slots must be distinct (each place holds one token).
    """
    slots = [int(s) for s in slots]
    assert len(set(slots)) == len(slots), "slots must be distinct"
    for i, slot in enumerate(slots):
        blk, place = divmod(slot, block_size)
        k_cache[blk, :, place, :] = k_new[i]
        v_cache[blk, :, place, :] = v_new[i]


def copy_blocks(k_cache, v_cache, pairs) -> None:
    """In place, pairs applied in order: pool[dst] = pool[src] for K and V."""
    for src, dst in pairs:
        k_cache[int(dst)] = k_cache[int(src)].clone()
        v_cache[int(dst)] = v_cache[int(src)].clone()
