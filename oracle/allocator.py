"""Pure-Python model of the paged KV cache's block allocator.

Policy, from «The KV Cache and PagedAttention»:
  * › "Like Pages of Memory": memory is cut into equal physical blocks of
    `block_size` token places; a text sees its logical blocks in order.
  * › "The Block Table": one table per text; each entry names the physical
    block holding a logical block and how many of its places are filled. A
    new physical block is taken only when every earlier block of the text
    is full, so only the last block can be partly empty.
  * › "The Block Table": a finished text's blocks return for reuse.
  * › "Shared, Copied on Write": sharers of a prompt (parallel sampling,
    beam search) point at the same physical blocks and every physical block
    counts the texts using it. Before a text writes into a block that is
    shared, the block is copied, the write goes to the copy, and the
    original's count drops by one.
  * › "When Memory Runs Out": a text holds all of its blocks or none; an
    append that cannot get every block it needs changes nothing.

Readings where the pages are silent (the native allocator implements the
same ones, so block tables can be compared bit for bit):
  * The free list is a stack. `free_order[0]` is handed out first; blocks
    released by `free` are pushed in logical order, so the text's last
    block is the next one handed out.
  * Sequence ids count up from 0 and are never reused.
  * The copy-on-write copy goes to whichever sharer writes first; once the
    count is back to 1 the remaining holder writes in place. A shared block
    that is already full is never copied: the append opens a new block.
  * One append of n tokens can copy at most one block (the last one).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class NoBlocks(Exception):
    """Not enough free blocks; the allocator is unchanged."""


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if free_order is None:
            free_order = range(num_blocks)
        order = [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free_order must permute the blocks"
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(reversed(order))  # top of stack = end of list
        self.ref: List[int] = [0] * num_blocks
        self.blocks: Dict[int, List[int]] = {}
        self.filled: Dict[int, List[int]] = {}
        self.next_id = 0

    # -- texts --------------------------------------------------------------
    def add(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.blocks[sid] = []
        self.filled[sid] = []
        return sid

    def fork(self, parent: int) -> int:
        """A new text sharing every block of `parent`; each block's count + 1."""
        child = self.add()
        self.blocks[child] = list(self.blocks[parent])
        self.filled[child] = list(self.filled[parent])
        for b in self.blocks[child]:
            self.ref[b] += 1
        return child

    def append(self, sid: int, n: int) -> Tuple[List[int], Tuple[int, int]]:
        """Give `n` new tokens their slots; returns (slots, (cow_src, cow_dst)).

        (cow_src, cow_dst) is (-1, -1) when no block was copied.
        """
        B = self.block_size
        blocks, filled = self.blocks[sid], self.filled[sid]
        if n == 0:
            return [], (-1, -1)
        room = 0
        copy = False
        if blocks and filled[-1] < B:
            room = B - filled[-1]
            copy = self.ref[blocks[-1]] > 1
        beyond = max(0, n - room)
        need = (1 if copy else 0) + (beyond + B - 1) // B
        if need > len(self.free):
            raise NoBlocks(f"need {need} blocks, {len(self.free)} free")
        pair = (-1, -1)
        if copy:
            src = blocks[-1]
            dst = self.free.pop()
            self.ref[dst] = 1
            self.ref[src] -= 1
            blocks[-1] = dst
            pair = (src, dst)
        slots = []
        for _ in range(n):
            if not blocks or filled[-1] == B:
                b = self.free.pop()
                self.ref[b] = 1
                blocks.append(b)
                filled.append(0)
            slots.append(blocks[-1] * B + filled[-1])
            filled[-1] += 1
        return slots, pair

    def free_seq(self, sid: int) -> None:
        for b in self.blocks[sid]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.blocks[sid]
        del self.filled[sid]

    # -- views --------------------------------------------------------------
    def context_len(self, sid: int) -> int:
        return sum(self.filled[sid])

    def table(self, sid: int) -> List[Tuple[int, int]]:
        """Block-table entries (physical block, places filled) in logical order."""
        return list(zip(self.blocks[sid], self.filled[sid]))

    def export(self, sids: Sequence[int], max_blocks: int):
        """Dense tables [len(sids), max_blocks] padded with -1, and context lengths."""
        tables = [[-1] * max_blocks for _ in sids]
        lens = []
        for i, sid in enumerate(sids):
            bl = self.blocks[sid]
            assert len(bl) <= max_blocks
            tables[i][:len(bl)] = bl
            lens.append(self.context_len(sid))
        return tables, lens

    def num_free(self) -> int:
        return len(self.free)

    def used_and_filled(self) -> Tuple[int, int]:
        """(physical blocks in use, filled places over those blocks)."""
        seen = {}
        for sid, bl in self.blocks.items():
            for b, f in zip(bl, self.filled[sid]):
                seen[b] = f
        return self.num_blocks - len(self.free), sum(seen.values())
