"""Replaying workload scripts through the oracle: pool mode equals logical mode."""
import numpy as np

import workloads as wl
from oracle.replay import Replay


def small_sharing():
    return wl.SHARING_32x8.scaled(groups=2, samples=4, num_seqs=8, num_heads=2, num_kv_heads=2,
                                  head_dim=8, block_size=4, num_blocks=64, prompt_len=6,
                                  suffix_lo=0, suffix_hi=5, steps=3)


def test_tiny_lengths_and_fresh_blocks():
    w = wl.TINY
    d = wl.draw(w)
    assert d.prefill_lens == [4, 12, 21, 36]
    r = Replay(w, d)
    steps = r.run(wl.script(w, d))
    assert steps[0].lens == [5, 13, 22, 37]
    # texts 0, 1 and 3 had full last blocks and open a new one at the write
    nblocks = [int((t >= 0).sum()) for t in steps[0].tables]
    assert nblocks == [2, 4, 6, 10]
    assert steps[0].pairs == []
    assert np.isfinite(steps[0].out).all()


def test_pool_and_logical_modes_agree():
    fp8_sharing = small_sharing().scaled(dtype="f16", cache_dtype="fp8", kv_std=0.3,
                                         k_scale=1 / 64, v_scale=1 / 16)
    for w in (wl.TINY, small_sharing(), fp8_sharing):
        d = wl.draw(w)
        a = Replay(w, d, pool=True).run(wl.script(w, d))
        b = Replay(w, d, pool=False).run(wl.script(w, d))
        assert len(a) == len(b) == w.steps
        for x, y in zip(a, b):
            assert x.slots == y.slots and x.pairs == y.pairs and x.lens == y.lens
            assert np.array_equal(x.tables, y.tables)
            np.testing.assert_allclose(x.out, y.out, rtol=0, atol=1e-12)


def test_sharing_steps_copy_on_write():
    w = small_sharing()
    d = wl.draw(w)
    steps = Replay(w, d, pool=True).run(wl.script(w, d))
    for st in steps:
        # an even/odd pair shares a partly filled last block unless its length is a multiple of B
        for (src, dst) in st.pairs:
            assert src != dst
        assert len(st.pairs) <= w.groups * (w.samples // 2)
    assert sum(len(st.pairs) for st in steps) > 0
