"""A paged KV cache on one GPU: device pools plus the native block allocator.

Thin layer over the C ABI (every step runs in libpagedkv.so): the allocator
hands out slots and copy-on-write pairs on the host, the pairs and slots go to
the device, and the device entry points copy blocks, write the new keys and
values, and run decode attention. One decode step, in order («The KV Cache and
PagedAttention» › "One Token at a Time", › "Shared, Copied on Write"):
  1. pa_step_append     one slot per text; a copy pair when its last block is shared
  2. pa_copy_blocks     copies before any new token is written
  3. pa_kv_write        the new tokens' keys and values into their slots
  4. pa_decode_attention over the whole cache, new token included
Several layers may share one allocator (the same block tables address every
layer's pools), as a model with several attention layers would.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from . import _lib as L

_TORCH_DTYPES = None


def torch_dtype(name: str):
    """torch dtype of a format name; "fp8" pools hold E4M3 codes as uint8."""
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.uint8}[name]


class BlockAllocator:
    """Owner of a native pa_alloc handle (host memory only)."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.h = L.pa_alloc_create(num_blocks, block_size, free_order)

    def close(self):
        if self.h is not None:
            L.pa_alloc_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self) -> int:
        return L.pa_seq_add(self.h)

    def fork(self, parent: int) -> int:
        return L.pa_seq_fork(self.h, parent)

    def append(self, seq: int, n: int):
        return L.pa_seq_append(self.h, seq, n)

    def step_append(self, seqs: Sequence[int]):
        return L.pa_step_append(self.h, seqs)

    def free(self, seq: int) -> None:
        L.pa_seq_free(self.h, seq)

    def info(self, seq: int):
        return L.pa_seq_info(self.h, seq)

    def table(self, seq: int):
        return L.pa_seq_block_table(self.h, seq)

    def export(self, seqs: Sequence[int], max_blocks: int):
        return L.pa_export_tables(self.h, seqs, max_blocks)

    def ref(self, block: int) -> int:
        return L.pa_block_ref(self.h, block)

    def num_free(self) -> int:
        return L.pa_num_free(self.h)

    def stats(self):
        return L.pa_alloc_stats(self.h)

    def share_groups(self, seqs: Sequence[int], max_members: int, inner_members: int = 0):
        """Share groups of the batch for the shared-block decodes, read off the tables:
        (first, count, prefix) arrays, and with inner_members >= 2 the inner level too."""
        outer = L.pa_share_groups(self.h, seqs, max_members)
        if inner_members < 2:
            return outer
        return outer, L.pa_share_groups_inner(self.h, seqs, outer, inner_members)

    # prefix caching
    def add_cached(self, hashes: Sequence[int]):
        """New text on the registered blocks matching its leading hashes: (id, blocks reused)."""
        return L.pa_seq_add_cached(self.h, hashes)

    def cache_blocks(self, seq: int, hashes: Sequence[int]) -> None:
        L.pa_seq_cache_blocks(self.h, seq, hashes)

    def cache_stats(self):
        return L.pa_cache_stats(self.h)

    # swapping to host memory
    def host_pool(self, num_host_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        L.pa_alloc_host_pool(self.h, num_host_blocks, free_order)

    def swap_out(self, seqs: Sequence[int]):
        """(device block, host block) pairs to move."""
        return L.pa_swap_out(self.h, seqs)

    def swap_in(self, seqs: Sequence[int]):
        """(host block, device block) pairs to move."""
        return L.pa_swap_in(self.h, seqs)

    def swapped(self, seq: int) -> bool:
        return L.pa_seq_swapped(self.h, seq)

    def host_ref(self, block: int) -> int:
        return L.pa_host_block_ref(self.h, block)

    def host_num_free(self) -> int:
        return L.pa_host_num_free(self.h)


class PagedKVCache:
    """K/V pools [num_blocks, num_kv_heads, block_size, head_dim] per layer on one device.

    dtype "fp8" keeps E4M3 codes (one byte a number) with one scale per pool; new keys
    and values (any 16/32-bit format) are quantized as they are written.
    """

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype: str = "f16", layers: int = 1, device: str = "cuda",
                 free_order: Optional[Sequence[int]] = None, fill: Optional[float] = None,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        import torch
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        self.dtype, self.device = dtype, device
        self.fp8 = dtype == "fp8"
        self.k_scale, self.v_scale = k_scale, v_scale
        self.alloc = BlockAllocator(num_blocks, block_size, free_order)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        tdt = torch_dtype(dtype)
        if self.fp8 and fill is not None:
            fill = 0x7F  # the E4M3 NaN code marks places never written
        if fill is None:
            self.k = [torch.empty(shape, dtype=tdt, device=device) for _ in range(layers)]
            self.v = [torch.empty(shape, dtype=tdt, device=device) for _ in range(layers)]
        else:
            self.k = [torch.full(shape, fill, dtype=tdt, device=device) for _ in range(layers)]
            self.v = [torch.full(shape, fill, dtype=tdt, device=device) for _ in range(layers)]
        self._ws = None
        self._ws_key = None

    # ---- cache management (host allocator + device copies/writes) ----------
    def add(self) -> int:
        return self.alloc.add()

    def fork(self, parent: int) -> int:
        return self.alloc.fork(parent)

    def free(self, seq: int) -> None:
        self.alloc.free(seq)

    def append(self, seq: int, k, v, layer: int = 0):
        """Append n tokens' keys/values ([n, Hkv, D] device tensors) to one text."""
        import torch
        n = int(k.shape[0])
        slots, pair = self.alloc.append(seq, n)
        if pair[0] >= 0:
            p = torch.tensor([pair], dtype=torch.int32, device=self.device)
            for li in range(len(self.k)):
                L.pa_copy_blocks(self.k[li], self.v[li], p)
        if n:
            self.write(slots, k, v, layer)
        return slots, pair

    # ---- swapping to host memory ("When Memory Runs Out") -------------------
    def host_pool(self, num_host_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        """Pinned host pools of num_host_blocks blocks per layer, for texts that give way."""
        import torch
        self.alloc.host_pool(num_host_blocks, free_order)
        shape = (num_host_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        tdt = torch_dtype(self.dtype)
        self.hk = [torch.empty(shape, dtype=tdt, pin_memory=True) for _ in self.k]
        self.hv = [torch.empty(shape, dtype=tdt, pin_memory=True) for _ in self.k]

    def swap_out(self, seqs: Sequence[int]):
        """Move the texts' blocks (every layer) to the host pools; returns the pairs. The
        freed device blocks may be handed out at once: the copies are stream-ordered before
        any later write on this stream."""
        pairs = self.alloc.swap_out(seqs)
        self._move(pairs, to_host=True)
        return pairs

    def swap_in(self, seqs: Sequence[int]):
        pairs = self.alloc.swap_in(seqs)
        self._move(pairs, to_host=False)
        return pairs

    def _move(self, pairs, to_host: bool) -> None:
        import torch
        if not pairs:
            return
        p = torch.as_tensor(np.asarray(pairs, dtype=np.int32).reshape(-1, 2)).to(self.device)
        for li in range(len(self.k)):
            if to_host:
                L.pa_swap_blocks(self.hk[li], self.hv[li], self.k[li], self.v[li], p)
            else:
                L.pa_swap_blocks(self.k[li], self.v[li], self.hk[li], self.hv[li], p)

    def write(self, slots, k, v, layer: int = 0) -> None:
        import torch
        s = slots if isinstance(slots, torch.Tensor) else \
            torch.as_tensor(np.asarray(slots, dtype=np.int64)).to(self.device)
        if self.fp8:
            L.pa_kv_write_fp8(self.k[layer], self.v[layer], k, v, s, self.k_scale, self.v_scale)
        else:
            L.pa_kv_write(self.k[layer], self.v[layer], k, v, s)

    def copy(self, pairs, layer: Optional[int] = None) -> None:
        import torch
        if not pairs:
            return
        p = torch.as_tensor(np.asarray(pairs, dtype=np.int32).reshape(-1, 2)).to(self.device)
        for li in (range(len(self.k)) if layer is None else [layer]):
            L.pa_copy_blocks(self.k[li], self.v[li], p)

    def tables(self, seqs: Sequence[int], max_blocks: Optional[int] = None):
        """Device block tables [S, max_blocks] and context lengths [S], plus the host copies."""
        import torch
        if max_blocks is None:
            max_blocks = max(1, max(self.alloc.info(s)[1] for s in seqs))
        t, lens = self.alloc.export(seqs, max_blocks)
        return (torch.from_numpy(t).to(self.device), torch.from_numpy(lens).to(self.device), t, lens)

    # ---- attention ---------------------------------------------------------
    def workspace(self, num_seqs: int, num_heads: int, max_context_len: int,
                  partition_tokens: int = 0):
        import torch
        key = (num_seqs, num_heads, max_context_len, partition_tokens)
        if self._ws_key != key:
            nbytes = L.pa_decode_workspace_bytes(num_seqs, num_heads, self.head_dim,
                                                 max_context_len, partition_tokens)
            if self._ws is None or self._ws.numel() < nbytes:
                self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws_key = key
        return self._ws

    def attend(self, q, block_tables, context_lens, max_context_len: int, out=None,
               layer: int = 0, partition_tokens: int = 0, scale: Optional[float] = None):
        import torch
        S, H, D = q.shape
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(S, H, max_context_len, partition_tokens)
        if self.fp8:
            L.pa_decode_attention_fp8(out, q, self.k[layer], self.v[layer], block_tables,
                                      context_lens, max_context_len, ws, self.k_scale,
                                      self.v_scale, partition_tokens=partition_tokens, scale=scale)
        else:
            L.pa_decode_attention(out, q, self.k[layer], self.v[layer], block_tables,
                                  context_lens, max_context_len, ws,
                                  partition_tokens=partition_tokens, scale=scale)
        return out

    def step(self, seqs: Sequence[int], k_new, v_new, q, max_blocks: Optional[int] = None,
             partition_tokens: int = 0, scale: Optional[float] = None, fused: bool = True):
        """One decode step for `seqs` (single layer). Returns (out, slots, pairs, host tables, lens).

        With 16/32-bit pools the new rows are written inside the decode launch
        (pa_decode_attention_write) unless fused=False; E4M3 pools write first."""
        import torch
        slots, pairs, done = self.alloc.step_append(seqs)
        self.copy(pairs)
        bt, cl, t_host, lens = self.tables(seqs, max_blocks)
        if fused and not self.fp8:
            S, H, D = q.shape
            mctx = int(lens.max())
            out = torch.empty_like(q)
            s = torch.as_tensor(np.asarray(slots, dtype=np.int64)).to(self.device)
            L.pa_decode_attention_write(out, q, self.k[0], self.v[0], k_new, v_new, s, bt, cl,
                                        mctx, self.workspace(S, H, mctx, partition_tokens),
                                        partition_tokens=partition_tokens, scale=scale)
            return out, slots, pairs, t_host, lens
        self.write(slots, k_new, v_new)
        out = self.attend(q, bt, cl, int(lens.max()), partition_tokens=partition_tokens,
                          scale=scale)
        return out, slots, pairs, t_host, lens
