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

swap_blocks — › "When Memory Runs Out": a text that gives way can have its
blocks moved to the CPU's memory and back; whole blocks move between two
pools.

All three are pure moves of stored numbers: the models copy element bit
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


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs) -> None:
    """Whole blocks from one pool pair to another («The KV Cache and PagedAttention» ›
    "When Memory Runs Out": a text's blocks moved to the CPU's memory and back): pairs
    applied in order, dst[d] = src[s] for K and V; a pair naming a block outside its
    pool moves nothing."""
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not (0 <= src < src_k.shape[0] and 0 <= dst < dst_k.shape[0]):
            continue
        dst_k[dst] = src_k[src].clone()
        dst_v[dst] = src_v[src].clone()


def quantize_rows(x, scale: float):
    """E4M3 codes of values x stored with `scale`, rounding decided in float32.

    The code of x is encode(float32(x) * float32(1 / scale)): one float32
    multiply by the float32 reciprocal of the scale (each rounded to nearest
    even), then the E4M3 rounding of that float32 value (oracle/fp8.py).
    """
    import numpy as np
    import torch

    from . import fp8
    x32 = x.detach().to("cpu", torch.float32).numpy()
    inv = np.float32(1.0) / np.float32(scale)
    y = (x32 * inv).astype(np.float32)
    return torch.from_numpy(fp8.encode(y.astype(np.float64)))


def kv_write_fp8(k_cache, v_cache, k_new, v_new, slots, block_size: int, k_scale: float,
                 v_scale: float) -> None:
    """kv_write into uint8 E4M3 pools: each new value is quantized with its pool's scale
    («The KV Cache and PagedAttention» › "What Came After": one byte a number)."""
    kv_write(k_cache, v_cache, quantize_rows(k_new, k_scale), quantize_rows(v_new, v_scale),
             slots, block_size)
