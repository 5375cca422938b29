"""The oracle's block allocator against the pages' worked example and invariants."""
import json
import os

import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import BlockAllocator, NoBlocks

STAND = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "stand_cow.json")))


def test_stand_copy_on_write():
    """Two answers share a prompt of two blocks, the last half full; the first writer copies."""
    B = STAND["block_size"]
    a = BlockAllocator(8, B)
    prompt = a.add()
    n = (STAND["prompt_blocks"] - 1) * B + STAND["last_block_filled"]
    a.append(prompt, n)
    first_block, shared_last = a.blocks[prompt]
    ans1, ans2 = a.fork(prompt), a.fork(prompt)
    a.free_seq(prompt)
    assert a.ref[shared_last] == STAND["expect"]["copied_block_ref_before"]
    slots1, pair1 = a.append(ans1, 1)
    assert pair1[0] == shared_last and pair1[1] != shared_last
    assert a.ref[shared_last] == STAND["expect"]["copied_block_ref_after"]
    assert slots1 == [pair1[1] * B + STAND["last_block_filled"]]
    slots2, pair2 = a.append(ans2, 1)
    assert pair2 == (-1, -1), "the last holder writes in place"
    assert slots2 == [shared_last * B + STAND["last_block_filled"]]
    assert a.ref[first_block] == STAND["expect"]["first_block_stays_shared_ref"]
    assert a.blocks[ans1][0] == a.blocks[ans2][0] == first_block


def test_full_shared_block_is_not_copied():
    a = BlockAllocator(8, 4)
    p = a.add()
    a.append(p, 8)
    c = a.fork(p)
    slots, pair = a.append(c, 1)
    assert pair == (-1, -1)
    assert len(a.blocks[c]) == 3 and a.ref[a.blocks[c][2]] == 1


def test_free_list_order_and_reuse():
    a = BlockAllocator(6, 2, free_order=[3, 0, 5, 1, 4, 2])
    s = a.add()
    slots, _ = a.append(s, 5)
    assert a.blocks[s] == [3, 0, 5]
    assert slots == [6, 7, 0, 1, 10]
    a.free_seq(s)
    t = a.add()
    a.append(t, 2)
    assert a.blocks[t] == [5], "the freed text's last block is handed out next"
    assert a.num_free() == 5


def test_no_blocks_changes_nothing():
    a = BlockAllocator(4, 4)
    s = a.add()
    a.append(s, 10)
    c = a.fork(s)
    before = (list(a.free), list(a.ref), {k: list(v) for k, v in a.blocks.items()},
              {k: list(v) for k, v in a.filled.items()})
    with pytest.raises(NoBlocks):
        a.append(c, 8)   # copy of the shared last block + 2 new blocks > 1 free
    after = (list(a.free), list(a.ref), {k: list(v) for k, v in a.blocks.items()},
             {k: list(v) for k, v in a.filled.items()})
    assert before == after


def check_invariants(a: BlockAllocator):
    B = a.block_size
    refs = [0] * a.num_blocks
    for sid, bl in a.blocks.items():
        f = a.filled[sid]
        assert len(bl) == len(f)
        assert all(x == B for x in f[:-1]), "only the last block may be partly filled"
        if f:
            assert 1 <= f[-1] <= B
            assert len(bl) == -(-a.context_len(sid) // B), "a new block only when the last is full"
        assert len(set(bl)) == len(bl)
        for b in bl:
            refs[b] += 1
    assert refs == a.ref, "each block counts exactly the texts using it"
    assert sorted(a.free) == [b for b in range(a.num_blocks) if refs[b] == 0]
    used, filled = a.used_and_filled()
    assert used + a.num_free() == a.num_blocks
    assert filled <= used * B


ops = st.lists(st.tuples(st.sampled_from(["add", "append", "fork", "free"]),
                         st.integers(0, 50), st.integers(0, 9)), max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops, st.sampled_from([1, 2, 4]), st.integers(4, 24))
def test_random_ops_keep_invariants(seq, B, N):
    a = BlockAllocator(N, B)
    live = []
    for kind, pick, n in seq:
        if kind == "add" or not live:
            live.append(a.add())
        elif kind == "append":
            sid = live[pick % len(live)]
            others = {b for o in live if o != sid for b in a.blocks[o]}
            try:
                slots, pair = a.append(sid, n)
            except NoBlocks:
                continue
            for slot in slots:
                assert slot // B not in others, "a write never lands in a block another text holds"
                assert a.ref[slot // B] == 1
            if pair[0] >= 0:
                assert a.ref[pair[1]] == 1 and a.ref[pair[0]] >= 1
        elif kind == "fork":
            live.append(a.fork(live[pick % len(live)]))
        else:
            a.free_seq(live.pop(pick % len(live)))
        check_invariants(a)
    for sid in live:
        a.free_seq(sid)
    assert a.num_free() == N and a.ref == [0] * N
