"""pa_decode_attention on the GPU against the fp64 oracle, through the C ABI.

Small seeded cases that still span several segments and a ragged last chunk,
every dtype / head_dim / block_size the library supports, shared key/value
heads, and the method's degenerate cases.
"""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def make_case(seed, lens, H, Hkv, D, B, dtype, kv_std=1.0, q_std=1.0, extra=7, fill=float("nan")):
    """Pools with every text's tokens in randomly placed blocks; unused places = fill."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nblk = [(L + B - 1) // B for L in lens]
    N = sum(nblk) + extra
    kc = torch.full((N, Hkv, B, D), fill, dtype=TD[dtype])
    vc = torch.full((N, Hkv, B, D), fill, dtype=TD[dtype])
    perm = list(rng.permutation(N))
    maxb = max(1, max(nblk))
    tables = np.full((len(lens), maxb), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        k = (torch.randn((L, Hkv, D), generator=g) * kv_std).to(TD[dtype])
        v = (torch.randn((L, Hkv, D), generator=g) * kv_std).to(TD[dtype])
        for j in range(nblk[s]):
            tables[s, j] = perm.pop()
        for t in range(L):
            kc[tables[s, t // B], :, t % B] = k[t]
            vc[tables[s, t // B], :, t % B] = v[t]
    q = (torch.randn((len(lens), H, D), generator=g) * q_std).to(TD[dtype])
    return q, kc, vc, tables, np.asarray(lens, dtype=np.int32)


def run_gpu(native, q, kc, vc, tables, lens, partition_tokens=0, max_ctx=None, scale=None):
    S, H, D = q.shape
    if max_ctx is None:
        max_ctx = int(lens.max()) if len(lens) else 0
    ws = native.decode_workspace(S, H, D, max_ctx, partition_tokens)
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention(out, q.cuda(), kc.cuda(), vc.cuda(),
                               torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                               max_ctx, ws, partition_tokens=partition_tokens, scale=scale)
    torch.cuda.synchronize()
    return out.cpu()


SHAPES = [(dt, D, B) for dt in ("f32", "f16", "bf16") for D in (64, 128) for B in (4, 8, 16, 32)]


@pytest.mark.parametrize("dtype,D,B", SHAPES)
def test_matches_oracle(native, dtype, D, B):
    lens = [1, 5, 16, 17, 40, 129, 300, 2]
    H = Hkv = 4
    say(f"decode dtype={dtype} D={D} B={B} lens={lens}")
    kv_std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(D)
    q, kc, vc, tables, L = make_case(D * 100 + B, lens, H, Hkv, D, B, dtype, kv_std=kv_std)
    want = decode_attention(q, kc, vc, tables, L, B)
    for T in (0, 16, 64):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T)
        assert_close(got, want, dtype, f"partition_tokens={T}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_sharp_scores(native, dtype):
    """Peaked softmax (q x 32, V ~ N(0,1)): a dropped or misplaced block cannot hide."""
    lens = [33, 250, 777]
    q, kc, vc, tables, L = make_case(7, lens, 8, 8, 128, 16, dtype, kv_std=1.0 / math.sqrt(128),
                                     q_std=32.0)
    vc = torch.where(torch.isnan(vc), vc, vc * math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=32)
    assert_close(got, want, dtype, "sharp")


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (40, 8), (32, 2), (64, 8), (12, 4), (6, 3)])
def test_shared_kv_heads(native, H, Hkv):
    """Query heads sharing key/value heads: one stream of a K/V head serves 1, 2, 4 or 8 of
    them (G = 5 and 3 fall back to one head per wave; G = 16 uses two groups of 8)."""
    lens = [3, 70, 31, 400]
    say(f"gqa H={H} Hkv={Hkv}")
    q, kc, vc, tables, L = make_case(H + Hkv, lens, H, Hkv, 128, 16, "f16",
                                     kv_std=1.0 / math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    for T in (0, 32):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T)
        assert_close(got, want, "f16", f"gqa T={T}")


@pytest.mark.parametrize("dtype,D,B", [("f32", 64, 4), ("bf16", 128, 32), ("f16", 64, 8),
                                       ("bf16", 64, 16), ("f32", 128, 16)])
@pytest.mark.parametrize("G", [2, 4, 8])
def test_shared_kv_heads_all_formats(native, dtype, D, B, G):
    lens = [1, 17, 129, 300]
    Hkv = 2
    kv_std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(D)
    say(f"gqa dtype={dtype} D={D} B={B} G={G}")
    q, kc, vc, tables, L = make_case(G * 10 + D + B, lens, G * Hkv, Hkv, D, B, dtype, kv_std=kv_std)
    want = decode_attention(q, kc, vc, tables, L, B)
    for T in (0, 16):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T)
        assert_close(got, want, dtype, f"T={T}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,B", [(64, 4), (64, 16), (128, 8), (128, 16), (128, 32)])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_eight_heads_per_kv_head_on_matrix_cores(native, dtype, D, B, G):
    """4 or 8 query heads per wave on MFMA (16-bit formats): every block size, ragged
    chunks, runs split over segments and whole runs in one segment."""
    lens = [1, 15, 16, 17, 129, 300, 1025]
    Hkv = 2
    say(f"gqa mfma dtype={dtype} D={D} B={B} G={G}")
    q, kc, vc, tables, L = make_case(G + D + B, lens, G * Hkv, Hkv, D, B, dtype,
                                     kv_std=1.0 / math.sqrt(D))
    want = decode_attention(q, kc, vc, tables, L, B)
    for T in (0, 16, 48, 2048):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T)
        assert_close(got, want, dtype, f"T={T}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_eight_heads_sharp_and_degenerate(native, dtype):
    """MFMA path: peaked softmax, one-token texts (exact), empty texts (zeros) and a bad
    table entry (only its text is NaN)."""
    lens = [33, 1, 0, 250, 777]
    q, kc, vc, tables, L = make_case(77, lens, 16, 2, 128, 16, dtype,
                                     kv_std=1.0 / math.sqrt(128), q_std=32.0)
    vc = torch.where(torch.isnan(vc), vc, vc * math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=32)
    assert_close(got, want, dtype, "sharp")
    for h in range(16):
        assert torch.equal(got[1, h], vc[tables[1, 0], h // 8, 0])
    assert (got[2].float() == 0).all()
    bad = tables.copy()
    bad[3, 5] = kc.shape[0] + 3
    got = run_gpu(native, q, kc, vc, bad, L, partition_tokens=32).float()
    assert torch.isnan(got[3]).all()
    keep = [0, 1, 2, 4]
    assert_close(got[keep], want[keep], dtype, "others")


def test_single_token_is_exact(native):
    for dtype in ("f32", "f16", "bf16"):
        q, kc, vc, tables, L = make_case(3, [1, 1, 1], 4, 4, 128, 16, dtype)
        got = run_gpu(native, q, kc, vc, tables, L)
        for s in range(3):
            v0 = vc[tables[s, 0], :, 0]
            assert torch.equal(got[s], v0), f"{dtype}: out != v_0"


def test_empty_context_gives_zeros(native):
    q, kc, vc, tables, L = make_case(4, [0, 9, 0], 4, 4, 64, 4, "f16")
    got = run_gpu(native, q, kc, vc, tables, L)
    assert torch.count_nonzero(got[0]) == 0 and torch.count_nonzero(got[2]) == 0
    want = decode_attention(q, kc, vc, tables, L, 4)
    assert_close(got, want, "f16", "ragged with empty texts")


def test_placement_does_not_change_a_bit(native):
    """The same logical cache under another block placement: identical output bits."""
    lens = [100, 513, 47, 1000]
    q, kc, vc, tables, L = make_case(9, lens, 8, 8, 128, 16, "f16", kv_std=1 / math.sqrt(128))
    base = run_gpu(native, q, kc, vc, tables, L)
    pi = torch.from_numpy(np.random.default_rng(5).permutation(kc.shape[0]))
    kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    t2 = np.where(tables >= 0, pi.numpy()[np.maximum(tables, 0)], -1).astype(np.int32)
    moved = run_gpu(native, q, kc2, vc2, t2, L)
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_unused_places_are_never_read(native):
    """NaN in unfilled places and unused blocks vs zeros there: same output bits."""
    lens = [5, 18, 33]
    a = make_case(11, lens, 4, 4, 128, 16, "bf16", fill=float("nan"))
    b = make_case(11, lens, 4, 4, 128, 16, "bf16", fill=0.0)
    ga, gb = run_gpu(native, *a), run_gpu(native, *b)
    assert torch.isfinite(ga.float()).all()
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


def test_bad_table_entry_poisons_only_its_text(native):
    lens = [20, 20, 20]
    q, kc, vc, tables, L = make_case(12, lens, 4, 4, 64, 16, "f32")
    tables = tables.copy()
    tables[1, 1] = kc.shape[0] + 100       # outside the pool
    got = run_gpu(native, q, kc, vc, tables, L)
    assert torch.isnan(got[1]).all()
    want = decode_attention(q, kc, vc, tables, L, 16, pairs=[(s, h) for s in (0, 2) for h in range(4)])
    assert_close(got, want, "f32", "other texts")


def test_context_longer_than_table_poisons(native):
    q, kc, vc, tables, L = make_case(13, [10, 10], 4, 4, 64, 4, "f32")
    L = L.copy()
    L[0] = tables.shape[1] * 4 + 1
    got = run_gpu(native, q, kc, vc, tables, L, max_ctx=int(L.max()))
    assert torch.isnan(got[0]).all() and torch.isfinite(got[1]).all()


def test_long_single_text_many_segments(native):
    """One 20,000-token text split over many waves; the merge pass combines them."""
    q, kc, vc, tables, L = make_case(14, [20000, 3], 2, 2, 128, 16, "f16",
                                     kv_std=1 / math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    for T in (0, 256, 4096):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T)
        assert_close(got, want, "f16", f"T={T}")


def test_scale_argument(native):
    q, kc, vc, tables, L = make_case(15, [30, 61], 4, 4, 64, 8, "f32")
    want = decode_attention(q, kc, vc, tables, L, 8, scale=0.3)
    got = run_gpu(native, q, kc, vc, tables, L, scale=0.3)
    assert_close(got, want, "f32", "scale 0.3")


def test_repeated_launches_are_bit_identical(native):
    """Many segments per text and partials merged by whichever segment finishes last:
    thirty launches give the same bits (a race in the merge would show here)."""
    lens = [3000] * 6 + [17, 1, 250, 4096]
    q, kc, vc, tables, L = make_case(16, lens, 8, 8, 128, 16, "f16", kv_std=1 / math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(L).cuda()
    for T in (0, 32):
        ws = native.decode_workspace(len(lens), 8, 128, int(L.max()), T)
        outs = []
        for _ in range(30):
            out = torch.empty_like(qd)
            native.pa_decode_attention(out, qd, kd, vd, td, ld, int(L.max()), ws, partition_tokens=T)
            outs.append(out)
        torch.cuda.synchronize()
        first = outs[0].cpu()
        assert_close(first, want, "f16", f"T={T}")
        for o in outs[1:]:
            assert torch.equal(o.cpu().view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 2)])
def test_context_beyond_the_host_bound(native, H, Hkv):
    """context_lens above max_context_len (still within the tables) with 16-token
    partitions: the grid is sized for the smaller bound, so the segments lengthen to cover
    every unit and the merge stays inside the grid. Sharp scores (q x 32, V ~ N(0,1)):
    an output left stale (7.0) or a partial read from the wrong place would show."""
    lens = [300, 1000, 64, 777, 1]
    say(f"context beyond host bound H={H} Hkv={Hkv}")
    q, kc, vc, tables, L = make_case(31 + H, lens, H, Hkv, 128, 16, "f16",
                                     kv_std=1.0 / math.sqrt(128), q_std=32.0)
    vc = torch.where(torch.isnan(vc), vc, vc * math.sqrt(128))
    want = decode_attention(q, kc, vc, tables, L, 16)
    for T in (16, 48):
        got = run_gpu(native, q, kc, vc, tables, L, partition_tokens=T, max_ctx=100)
        assert torch.isfinite(got.float()).all()
        assert_close(got, want, "f16", f"T={T} max_context_len=100")


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 2), (32, 4)])
def test_merge_guess_and_general_path_agree_bit_for_bit(native, H, Hkv):
    """The merge loads a run's partials on the guess that every text attends
    max_context_len tokens. With max_context_len exact (the guess holds) and with a looser
    bound of the same grid (the guess fails: the general path), the outputs must be the
    same bits: both fold the same partials in the same order. Unequal lengths (the guess
    fails everywhere but the longest texts) must agree with the oracle as well."""
    D, B = 128, 16
    for lens in ([300] * 9, [300, 17, 300, 1, 288, 300, 0, 299, 300]):
        q, kc, vc, tables, L = make_case(11, lens, H, Hkv, D, B, "f16", kv_std=0.125)
        say(f"merge guess H={H} Hkv={Hkv} lens={lens}")
        exact = run_gpu(native, q, kc, vc, tables, L, max_ctx=300)
        loose = run_gpu(native, q, kc, vc, tables, L, max_ctx=300 + 3 * B)
        assert torch.equal(exact.view(torch.int16), loose.view(torch.int16))
        want = decode_attention(q, kc, vc, tables, L, B)
        assert_close(exact, want, "f16", f"lens {lens}")


def test_segment_search_past_4096_texts(native):
    """More than 4,096 texts: each wave's segment search takes three rounds (64 lane
    ranges of 66 texts, then their sub-ranges, then single texts). Short random lengths,
    empty texts included; every output against the oracle."""
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 25, 4200)]
    lens[::97] = [0] * len(lens[::97])
    H, Hkv, D, B = 2, 2, 64, 4
    q, kc, vc, tables, L = make_case(12, lens, H, Hkv, D, B, "f16", kv_std=0.125, extra=3)
    say(f"segment search, {len(lens)} texts")
    got = run_gpu(native, q, kc, vc, tables, L)
    want = decode_attention(q, kc, vc, tables, L, B)
    assert_close(got, want, "f16", "4,200 texts")


def test_merge_by_segment_boundary_with_runs_over_many_segments(native):
    """More runs than segments (600 texts x 2 heads over the 1,024 segments of a 256-CU
    part's auto grid), so the merge runs one wave per segment boundary. Three 6,000-token
    texts among short ones make runs that cross ~90 boundaries each: every such run must be
    merged once, by the wave of the first boundary it crosses, and every short run split
    across a boundary too. Sharp scores (q x 32, V ~ N(0,1)): a run merged twice from the
    wrong partials, or left unmerged (7.0), would show; a second launch gives the same bits."""
    rng = np.random.default_rng(21)
    lens = [int(x) for x in rng.integers(1, 21, 600)]
    for i in (5, 300, 599):
        lens[i] = 6000
    H, Hkv, D, B = 2, 2, 128, 16
    say(f"merge by segment boundary, {len(lens)} texts")
    q, kc, vc, tables, L = make_case(22, lens, H, Hkv, D, B, "f16", kv_std=1.0 / math.sqrt(D),
                                     q_std=32.0)
    vc = torch.where(torch.isnan(vc), vc, vc * math.sqrt(D))
    want = decode_attention(q, kc, vc, tables, L, B)
    got = run_gpu(native, q, kc, vc, tables, L)
    assert torch.isfinite(got.float()).all()
    assert_close(got, want, "f16", "600 texts, three of 6,000 tokens")
    again = run_gpu(native, q, kc, vc, tables, L)
    assert torch.equal(again.view(torch.int16), got.view(torch.int16))
