"""Prefix caching end to end through the C ABI against the oracle.

Requests that begin with shared system prompts are admitted batch by batch: each
looks up its full blocks' chained hashes (pa_hash_blocks, pa_seq_add_cached), gets
slots for the tokens not cached (pa_seq_append), writes their keys and values
(pa_kv_write), runs the prompt phase over them (pa_prefill_attention) and registers
its full blocks (pa_seq_cache_blocks); finished requests are freed and their cached
blocks evicted as the small pool runs short. The oracle replays the same schedule
with its allocator model, block hash, cache writes and prompt-phase attention: reuse
counts, slots, tables and whole pools bit-exact, outputs within the tolerance.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_common import assert_close, say
from oracle import cache_ops
from oracle.allocator import BlockAllocator as Model
from oracle.block_hash import block_hashes
from oracle.prefill import prefill_attention
from paged_kv_cache_320_amd import PagedKVCache

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def request_data(d, r):
    i = d.req_sys[r]
    toks = np.concatenate([d.sys_tokens[i], d.user_tokens[r]])
    k = torch.cat([d.sys_k[i], d.user_k[r]])
    v = torch.cat([d.sys_v[i], d.user_v[r]])
    return toks, k, v


def run_native(w, d, native):
    B = w.block_size
    cache = PagedKVCache(w.num_blocks, B, w.num_kv_heads, w.head_dim, w.dtype,
                         free_order=d.free_order, fill=float("nan"))
    a = cache.alloc
    log = []
    sid_of = {}
    for op, reqs in wl.prefix_schedule(w):
        if op == "finish":
            for r in reqs:
                a.free(sid_of.pop(r))
            continue
        rec = {"cached": [], "slots": [], "q": [], "lens": []}
        seqs = []
        for r in reqs:
            toks, k, v = request_data(d, r)
            L = len(toks)
            hashes = native.pa_hash_blocks(toks, B)
            sid, nc = a.add_cached(hashes[:(L - 1) // B])
            slots, pair = a.append(sid, L - nc * B)
            assert pair == (-1, -1)
            cache.write(slots, k[nc * B:].cuda(), v[nc * B:].cuda())
            sid_of[r] = sid
            seqs.append(sid)
            rec["cached"].append(nc)
            rec["slots"] += slots
            rec["q"].append(d.q[r][nc * B:])
        maxb = max(a.info(s)[1] for s in seqs)
        t, lens = a.export(seqs, maxb)
        q = torch.cat(rec["q"]).contiguous()
        q_start = np.concatenate([[0], np.cumsum([x.shape[0] for x in rec["q"]])]).astype(np.int32)
        out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
        native.pa_prefill_attention(out, q.cuda(), cache.k[0], cache.v[0], torch.from_numpy(t).cuda(),
                                    torch.from_numpy(lens).cuda(), torch.from_numpy(q_start).cuda(),
                                    int(np.diff(q_start).max()))
        for r, sid in zip(reqs, seqs):
            toks, _, _ = request_data(d, r)
            a.cache_blocks(sid, native.pa_hash_blocks(toks, B))
        rec.update(tables=t, lens=list(lens), q_start=q_start, out=out.cpu(), q=q,
                   stats=a.cache_stats())
        log.append(rec)
    torch.cuda.synchronize()
    return log, cache


def run_oracle(w, d):
    B = w.block_size
    m = Model(w.num_blocks, B, d.free_order)
    shape = (w.num_blocks, w.num_kv_heads, B, w.head_dim)
    kp = torch.full(shape, float("nan"), dtype=TD[w.dtype])
    vp = torch.full(shape, float("nan"), dtype=TD[w.dtype])
    log = []
    sid_of = {}
    for op, reqs in wl.prefix_schedule(w):
        if op == "finish":
            for r in reqs:
                m.free_seq(sid_of.pop(r))
            continue
        rec = {"cached": [], "slots": []}
        seqs = []
        for r in reqs:
            toks, k, v = request_data(d, r)
            L = len(toks)
            sid, nc = m.add_cached(block_hashes(toks, B)[:(L - 1) // B])
            slots, pair = m.append(sid, L - nc * B)
            assert pair == (-1, -1)
            cache_ops.kv_write(kp, vp, k[nc * B:], v[nc * B:], slots, B)
            sid_of[r] = sid
            seqs.append(sid)
            rec["cached"].append(nc)
            rec["slots"] += slots
        maxb = max(len(m.blocks[s]) for s in seqs)
        t, lens = m.export(seqs, maxb)
        for r, sid in zip(reqs, seqs):
            toks, _, _ = request_data(d, r)
            m.cache_blocks(sid, block_hashes(toks, B))
        rec.update(tables=np.asarray(t, dtype=np.int32), lens=lens, stats=m.cached_blocks(),
                   pools=(kp.clone(), vp.clone()))
        log.append(rec)
    return log, kp, vp


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefix_caching_end_to_end(native, dtype):
    w = wl.PREFIX_CHAT.scaled(dtype=dtype)
    say(f"prefix caching {w.name} dtype={dtype}")
    d = wl.draw_prefix(w)
    nat, cache = run_native(w, d, native)
    ora, kp, vp = run_oracle(w, d)
    reused = 0
    for b, (n, o) in enumerate(zip(nat, ora)):
        assert n["cached"] == o["cached"], f"batch {b}: blocks reused differ"
        assert n["slots"] == o["slots"], f"batch {b}: slots differ"
        assert np.array_equal(n["tables"], o["tables"]) and n["lens"] == o["lens"]
        assert n["stats"] == o["stats"]
        reused += sum(n["cached"])
        k_b, v_b = o["pools"]
        want = prefill_attention(n["q"], k_b, v_b, o["tables"], o["lens"], n["q_start"],
                                 w.block_size)
        assert_close(n["out"], want, dtype, f"batch {b}")
    assert reused > 0, "the schedule must reuse cached blocks"
    assert nat[-1]["stats"][0] > 0
    torch.cuda.synchronize()
    assert torch.equal(cache.k[0].cpu().view(torch.int16), kp.view(torch.int16))
    assert torch.equal(cache.v[0].cpu().view(torch.int16), vp.view(torch.int16))
