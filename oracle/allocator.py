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

Prefix caching (› "What Came After": a full block gets a hash of its tokens
and everything before them; a request that begins the same way reuses the
blocks). Readings where the page is silent:
  * blocks are registered explicitly (`cache_blocks`) once their keys and
    values are written; a hash already registered, or a block already
    carrying a hash, is left as it is;
  * `add_cached` starts a text on the longest run of registered blocks
    matching its leading block hashes, each block's count + 1; a registered
    block whose count had dropped to 0 is taken back out of the free list;
  * a registered block whose count drops to 0 stays registered and goes to
    the bottom of the free stack, after every unregistered free block, so
    cached blocks are handed out last: least recently freed first, and of one
    text's blocks the later ones first. Handing a registered block out again
    drops its registration (eviction).
Without registered blocks every behaviour above is unchanged.

Swapping (› "When Memory Runs Out": a text that gives way hands back all of
its blocks; one of the paper's answers moves them to the CPU's memory and
back when the text's turn comes). Readings where the page is silent:
  * a second stack of host blocks, `free_order` as for the device pool;
  * `swap_out(texts)` moves every block the listed texts hold, each distinct
    block once (texts in list order, logical blocks in order, first
    occurrence), so blocks they share stay shared on the host with the count
    of listed holders; a block also held by a text not listed is copied and
    stays on the device for it; device blocks nobody holds any more are
    released as `free` releases them, in that order; `swap_in` is the mirror
    image (device blocks from the top of the free stack, host blocks no text
    holds any more back onto the host stack, in that order);
  * both are all-or-nothing: too few free blocks on the receiving side
    changes nothing;
  * a swapped-out text cannot be appended to, forked, exported or
    registered; freeing it releases its host blocks.
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
        self.hash_of: Dict[int, int] = {}    # registered block -> its hash
        self.block_of: Dict[int, int] = {}   # hash -> registered block
        self.num_host_blocks = 0
        self.host_free: List[int] = []       # top of stack = end of list
        self.host_ref: List[int] = []
        self.swapped: set = set()            # texts whose blocks are host blocks

    # -- texts --------------------------------------------------------------
    def add(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.blocks[sid] = []
        self.filled[sid] = []
        return sid

    def _resident(self, sid: int) -> None:
        if sid in self.swapped:
            raise ValueError(f"text {sid} is swapped out")

    def fork(self, parent: int) -> int:
        """A new text sharing every block of `parent`; each block's count + 1."""
        self._resident(parent)
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
        self._resident(sid)
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
            dst = self._take()
            self.ref[src] -= 1
            blocks[-1] = dst
            pair = (src, dst)
        slots = []
        for _ in range(n):
            if not blocks or filled[-1] == B:
                b = self._take()
                blocks.append(b)
                filled.append(0)
            slots.append(blocks[-1] * B + filled[-1])
            filled[-1] += 1
        return slots, pair

    def _take(self) -> int:
        """Top of the free stack, with count 1; a registered block loses its registration."""
        b = self.free.pop()
        if b in self.hash_of:
            del self.block_of[self.hash_of.pop(b)]
        self.ref[b] = 1
        return b

    def _release(self, blocks: Sequence[int]) -> None:
        """Device blocks whose count dropped to 0, in order, back onto the free stack."""
        cached = []
        for b in blocks:
            if b in self.hash_of:
                cached.append(b)
            else:
                self.free.append(b)
        for b in reversed(cached):
            self.free.insert(0, b)  # bottom of the stack: handed out after all others

    def free_seq(self, sid: int) -> None:
        if sid in self.swapped:
            for h in self.blocks[sid]:
                self.host_ref[h] -= 1
                if self.host_ref[h] == 0:
                    self.host_free.append(h)
            self.swapped.discard(sid)
        else:
            zero = []
            for b in self.blocks[sid]:
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    zero.append(b)
            self._release(zero)
        del self.blocks[sid]
        del self.filled[sid]

    # -- swapping -----------------------------------------------------------
    def host_pool(self, num_host_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        assert self.num_host_blocks == 0, "the host pool is set up once"
        order = list(range(num_host_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_host_blocks))
        self.num_host_blocks = num_host_blocks
        self.host_free = list(reversed(order))
        self.host_ref = [0] * num_host_blocks

    def _holders(self, sids: Sequence[int], swapped: bool):
        """Distinct blocks of the listed texts in first-seen order, and how many of the
        listed texts hold each."""
        assert self.num_host_blocks > 0, "no host pool"
        assert len(set(sids)) == len(sids), "a text listed twice"
        for sid in sids:
            if (sid in self.swapped) != swapped:
                raise ValueError(f"text {sid} is on the wrong side")
        order, count = [], {}
        for sid in sids:
            for b in self.blocks[sid]:
                if b not in count:
                    count[b] = 0
                    order.append(b)
                count[b] += 1
        return order, count

    def swap_out(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Move the texts to host blocks; returns (device block, host block) pairs."""
        order, count = self._holders(sids, False)
        if len(order) > len(self.host_free):
            raise NoBlocks(f"need {len(order)} host blocks, {len(self.host_free)} free")
        host_of, pairs, zero = {}, [], []
        for b in order:
            h = self.host_free.pop()
            self.host_ref[h] = count[b]
            host_of[b] = h
            pairs.append((b, h))
            self.ref[b] -= count[b]
            if self.ref[b] == 0:
                zero.append(b)
        for sid in sids:
            self.blocks[sid] = [host_of[b] for b in self.blocks[sid]]
            self.swapped.add(sid)
        self._release(zero)
        return pairs

    def swap_in(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Bring the texts back to device blocks; returns (host block, device block) pairs."""
        order, count = self._holders(sids, True)
        if len(order) > len(self.free):
            raise NoBlocks(f"need {len(order)} blocks, {len(self.free)} free")
        dev_of, pairs = {}, []
        for h in order:
            b = self._take()
            self.ref[b] = count[h]
            dev_of[h] = b
            pairs.append((h, b))
        for sid in sids:
            self.blocks[sid] = [dev_of[h] for h in self.blocks[sid]]
            self.swapped.discard(sid)
        for h in order:
            self.host_ref[h] -= count[h]
            if self.host_ref[h] == 0:
                self.host_free.append(h)
        return pairs

    # -- prefix caching -----------------------------------------------------
    def add_cached(self, hashes: Sequence[int]) -> Tuple[int, int]:
        """A new text starting on the registered blocks that match its leading block
        hashes; returns (text id, blocks reused)."""
        sid = self.add()
        n = 0
        for h in hashes:
            b = self.block_of.get(int(h))
            if b is None:
                break
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            self.blocks[sid].append(b)
            self.filled[sid].append(self.block_size)
            n += 1
        return sid, n

    def cache_blocks(self, sid: int, hashes: Sequence[int]) -> None:
        """Register the text's first len(hashes) blocks, which must be full."""
        self._resident(sid)
        bl, fl = self.blocks[sid], self.filled[sid]
        if len(hashes) > len(bl) or any(f != self.block_size for f in fl[:len(hashes)]):
            raise ValueError("only full blocks of the text can be registered")
        for b, h in zip(bl, hashes):
            h = int(h)
            if h in self.block_of or b in self.hash_of:
                continue
            self.block_of[h] = b
            self.hash_of[b] = h

    def cached_blocks(self) -> Tuple[int, int]:
        """(registered blocks, registered blocks that are free)."""
        return len(self.hash_of), sum(1 for b in self.hash_of if self.ref[b] == 0)

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
            self._resident(sid)
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
            if sid in self.swapped:
                continue
            for b, f in zip(bl, self.filled[sid]):
                seen[b] = f
        return self.num_blocks - len(self.free), sum(seen.values())
