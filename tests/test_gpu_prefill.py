"""pa_prefill_attention (prompt phase, causal) on the GPU against the fp64 oracle.

Seeded cases spanning several 128-query tiles and 32-key tiles with ragged ends,
fresh prompts and prompts after a cached prefix, every dtype / head_dim /
block_size the call supports, shared key/value heads, and the degenerate cases.
"""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle.attention import decode_attention
from oracle.prefill import prefill_attention

pytestmark = pytest.mark.gpu

TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def make_case(seed, ctx, new, H, Hkv, D, B, dtype, kv_std=0.5, q_std=1.0, extra=7,
              fill=float("nan")):
    """Texts with ctx[s] cached tokens in randomly placed blocks (unused places = fill);
    the last new[s] positions are the prompt's queries, packed row after row."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nblk = [(L + B - 1) // B for L in ctx]
    N = sum(nblk) + extra
    kc = torch.full((N, Hkv, B, D), fill, dtype=TD[dtype])
    vc = torch.full((N, Hkv, B, D), fill, dtype=TD[dtype])
    perm = list(rng.permutation(N))
    tables = np.full((len(ctx), max(1, max(nblk))), -1, dtype=np.int32)
    for s, L in enumerate(ctx):
        k = (torch.randn((L, Hkv, D), generator=g) * kv_std).to(TD[dtype])
        v = (torch.randn((L, Hkv, D), generator=g) * kv_std).to(TD[dtype])
        for j in range(nblk[s]):
            tables[s, j] = perm.pop()
        for t in range(L):
            kc[tables[s, t // B], :, t % B] = k[t]
            vc[tables[s, t // B], :, t % B] = v[t]
    q_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = (torch.randn((int(q_start[-1]), H, D), generator=g) * q_std).to(TD[dtype])
    return q, kc, vc, tables, np.asarray(ctx, dtype=np.int32), q_start


def run_gpu(native, q, kc, vc, tables, ctx, q_start, max_q=None, out_rows=None, scale=None):
    T, H, D = q.shape
    if max_q is None:
        max_q = int(np.diff(q_start).max()) if len(ctx) else 0
    out = torch.full((out_rows or T, H, D), 7.0, dtype=q.dtype, device="cuda")
    native.pa_prefill_attention(out, q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(tables).cuda(),
                                torch.from_numpy(ctx).cuda(), torch.from_numpy(q_start).cuda(),
                                max_q, scale=scale)
    torch.cuda.synchronize()
    return out.cpu()


SHAPES = [(dt, D, B) for dt in ("f16", "bf16") for D in (64, 128) for B in (4, 8, 16, 32)]


@pytest.mark.parametrize("dtype,D,B", SHAPES)
def test_fresh_prompts_match_oracle(native, dtype, D, B):
    ctx = [1, 5, 33, 128, 129, 300]
    H = Hkv = 2
    say(f"prefill fresh dtype={dtype} D={D} B={B} ctx={ctx}")
    q, kc, vc, tables, L, qs = make_case(D * 100 + B, ctx, ctx, H, Hkv, D, B, dtype)
    want = prefill_attention(q, kc, vc, tables, L, qs, B)
    assert_close(run_gpu(native, q, kc, vc, tables, L, qs), want, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2), (8, 1), (6, 3)])
def test_prompt_after_cached_prefix(native, dtype, H, Hkv):
    ctx = [40, 300, 17, 9, 260]
    new = [7, 130, 17, 1, 0]
    say(f"prefill prefix dtype={dtype} H={H} Hkv={Hkv}")
    q, kc, vc, tables, L, qs = make_case(H * 10 + Hkv, ctx, new, H, Hkv, 128, 16, dtype)
    want = prefill_attention(q, kc, vc, tables, L, qs, 16)
    assert_close(run_gpu(native, q, kc, vc, tables, L, qs), want, dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_sharp_scores(native, dtype):
    """Peaked softmax (q x 8): a misplaced key or a wrong causal limit cannot hide."""
    ctx, new = [200, 77], [200, 50]
    q, kc, vc, tables, L, qs = make_case(5, ctx, new, 4, 4, 128, 16, dtype, kv_std=0.5, q_std=8.0)
    want = prefill_attention(q, kc, vc, tables, L, qs, 16)
    assert_close(run_gpu(native, q, kc, vc, tables, L, qs), want, dtype)


def test_last_row_equals_decode(native):
    """A prompt's last row attends the whole cache: the decode kernel's result."""
    ctx = [150, 64, 1]
    new = [100, 64, 1]
    q, kc, vc, tables, L, qs = make_case(11, ctx, new, 4, 2, 128, 16, "f16")
    got = run_gpu(native, q, kc, vc, tables, L, qs)
    last = torch.stack([q[qs[s + 1] - 1] for s in range(len(ctx))])
    ws = native.decode_workspace(len(ctx), 4, 128, int(L.max()), 0)
    dec = torch.empty(last.shape, dtype=last.dtype, device="cuda")
    native.pa_decode_attention(dec, last.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(tables).cuda(),
                               torch.from_numpy(L).cuda(), int(L.max()), ws)
    want = decode_attention(last, kc, vc, tables, L, 16)
    rows = torch.stack([got[qs[s + 1] - 1] for s in range(len(ctx))])
    assert_close(rows, want, "f16", "prefill last rows")
    assert_close(dec.cpu(), want, "f16", "decode")


def test_first_position_is_its_value(native):
    """A fresh prompt's first query attends one key: out = v_0 exactly."""
    ctx = [3, 130]
    q, kc, vc, tables, L, qs = make_case(2, ctx, ctx, 2, 2, 64, 8, "bf16")
    got = run_gpu(native, q, kc, vc, tables, L, qs)
    for s in range(len(ctx)):
        v0 = vc[tables[s, 0], :, 0]
        assert torch.equal(got[qs[s]], v0)


def test_placement_does_not_change_a_bit(native):
    ctx, new = [97, 260], [60, 260]
    a = make_case(3, ctx, new, 4, 4, 128, 16, "f16")
    q, kc, vc, tables, L, qs = a
    base = run_gpu(native, *a)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(kc.shape[0]))
    k2, v2 = torch.empty_like(kc), torch.empty_like(vc)
    k2[perm], v2[perm] = kc, vc
    t2 = np.where(tables >= 0, perm.numpy()[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = run_gpu(native, q, k2, v2, t2, L, qs)
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_unused_places_are_never_read(native):
    ctx, new = [45, 19], [45, 3]
    a = make_case(4, ctx, new, 2, 2, 128, 16, "f16", fill=float("nan"))
    b = make_case(4, ctx, new, 2, 2, 128, 16, "f16", fill=0.0)
    ga, gb = run_gpu(native, *a), run_gpu(native, *b)
    assert torch.isfinite(ga.float()).all()
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


def test_bad_entries_poison_only_their_text(native):
    ctx, new = [40, 40, 40], [10, 10, 50]   # text 2 asks for more queries than it has tokens
    q, kc, vc, tables, L, qs = make_case(6, ctx, new, 2, 2, 64, 8, "f16")
    tables = tables.copy()
    tables[0, 2] = kc.shape[0] + 5            # outside the pool, read by text 0
    got = run_gpu(native, q, kc, vc, tables, L, qs).float()
    assert torch.isnan(got[qs[0]:qs[1]]).all()
    assert torch.isnan(got[qs[2]:qs[3]]).all()
    want = prefill_attention(q[qs[1]:qs[2]], kc, vc, tables[1:2], L[1:2], np.array([0, 10]), 8)
    assert_close(got[qs[1]:qs[2]], want, "f16")


def test_rows_outside_the_output_are_not_written(native):
    """q_start past num_rows: that text is skipped, the others are computed."""
    ctx, new = [20, 30], [20, 30]
    q, kc, vc, tables, L, qs = make_case(8, ctx, new, 2, 2, 64, 16, "f16")
    q = q[:25]
    got = run_gpu(native, q, kc, vc, tables, L, qs, max_q=30)
    assert (got[20:25].float() == 7.0).all()
    want = prefill_attention(q[:20], kc, vc, tables[:1], L[:1], np.array([0, 20]), 16)
    assert_close(got[:20], want, "f16")


def test_small_max_q_len_still_covers_every_row(native):
    ctx, new = [300, 10], [300, 10]
    q, kc, vc, tables, L, qs = make_case(9, ctx, new, 2, 2, 64, 16, "bf16")
    want = prefill_attention(q, kc, vc, tables, L, qs, 16)
    assert_close(run_gpu(native, q, kc, vc, tables, L, qs, max_q=1), want, "bf16")


def test_rejects_unsupported(native):
    q = torch.zeros((4, 2, 128), dtype=torch.float32, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.float32, device="cuda")
    t = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    L = torch.full((1,), 4, dtype=torch.int32, device="cuda")
    qs = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    with pytest.raises(native.PagedKVError):
        native.pa_prefill_attention(q.clone(), q, kc, kc, t, L, qs, 4)


def test_scale_argument(native):
    """Any scale > 0 (the score order is kept); 0 and negative scales are rejected."""
    ctx = [50]
    q, kc, vc, tables, L, qs = make_case(12, ctx, ctx, 2, 2, 128, 16, "f16")
    want = prefill_attention(q, kc, vc, tables, L, qs, 16, scale=0.3)
    assert_close(run_gpu(native, q, kc, vc, tables, L, qs, scale=0.3), want, "f16")
    with pytest.raises(native.PagedKVError):
        run_gpu(native, q, kc, vc, tables, L, qs, scale=-0.3)


@pytest.mark.parametrize("w", __import__("workloads").PROMPT, ids=lambda w: w.name)
def test_full_size_prompt_workload(native, w):
    """The prompt-phase workloads at full size, in the launch configuration the bench times:
    the prompts' keys and values (after the shared cached prefix, if any) in randomly placed
    blocks, one pa_prefill_attention launch, and seeded sampled (row, head) outputs (every
    text's first and last rows included) against the oracle computed row by row."""
    import workloads as wl
    say(f"prompt workload {w.name} (full size)")
    d = wl.draw_prompt(w)
    lens = list(d.prompt_lens)
    S, H, Hkv, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    ctx = [w.prefix_len + n for n in lens]
    nblk = [(L + B - 1) // B for L in ctx]
    N = sum(nblk) + 3
    rng = np.random.default_rng(w.seed)
    perm = rng.permutation(N)
    tables = np.full((S, max(nblk)), -1, dtype=np.int32)
    kc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[w.dtype])
    vc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[w.dtype])
    off = 0
    for s in range(S):
        tables[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += nblk[s]
        ks = torch.cat([d.prefix_k, d.prompt_k[s]])
        vs = torch.cat([d.prefix_v, d.prompt_v[s]])
        t = torch.arange(ks.shape[0])
        blk = torch.from_numpy(tables[s].astype(np.int64))[t // B]
        kc[blk, :, t % B] = ks
        vc[blk, :, t % B] = vs
    L = np.asarray(ctx, dtype=np.int32)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    got = run_gpu(native, d.q, kc, vc, tables, L, qs, max_q=max(lens))
    say("  GPU done")
    sample = np.random.default_rng(w.seed + 1)
    rows = [(int(sample.integers(qs[-1])), int(sample.integers(H))) for _ in range(48)]
    rows += [(int(qs[s]), s % H) for s in range(S)] + [(int(qs[s + 1] - 1), (s + 1) % H)
                                                        for s in range(S)]
    want = prefill_attention(d.q, kc, vc, tables, L, qs, B, rows=rows)
    g = got.to(torch.float64).numpy()
    for r, h in rows:
        assert_close(g[r, h], want[r, h], w.dtype, f"{w.name} row {r} head {h}")
