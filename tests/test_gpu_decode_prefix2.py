"""pa_decode_attention_prefix2 (shared blocks at two nested levels, each read once for all
the texts that hold it) on the GPU: the same attention as over every text's whole table,
within the decode tolerance of the fp64 oracle (attention.decode_attention over the full
tables)."""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def make_nested(seed, outer, H, Hkv, D, B, dtype, q_std=1.0, extra=5):
    """outer: list of (P1, inner) with P1 a block multiple (0: no outer group) and inner a
    list of (P2, [own tokens of each member]): the members of an inner entry share P2 more
    tokens (a block multiple, 0: none) after the outer group's P1. Returns q, pools, tables,
    lengths, and the outer and inner groups as (first, count, shared length) lists."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    n_blocks = extra
    for P1, inner in outer:
        n_blocks += P1 // B
        for P2, own in inner:
            n_blocks += P2 // B + sum((n + B - 1) // B for n in own)
    perm = list(rng.permutation(n_blocks))
    kc = torch.full((n_blocks, Hkv, B, D), float("nan"), dtype=TD[dtype])
    vc = torch.full((n_blocks, Hkv, B, D), float("nan"), dtype=TD[dtype])
    std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(D)

    def fill(blocks, ntok):
        k = (torch.randn((ntok, Hkv, D), generator=g) * std).to(TD[dtype])
        v = (torch.randn((ntok, Hkv, D), generator=g) * std).to(TD[dtype])
        for t in range(ntok):
            kc[blocks[t // B], :, t % B] = k[t]
            vc[blocks[t // B], :, t % B] = v[t]

    rows, lens, og, ig = [], [], [], []
    for P1, inner in outer:
        b1 = [perm.pop() for _ in range(P1 // B)]
        fill(b1, P1)
        first1 = len(rows)
        for P2, own in inner:
            b2 = [perm.pop() for _ in range(P2 // B)]
            fill(b2, P2)
            first2 = len(rows)
            for n in own:
                mine = [perm.pop() for _ in range((n + B - 1) // B)]
                fill(mine, n)
                rows.append(b1 + b2 + mine)
                lens.append(P1 + P2 + n)
            ig.append((first2, len(own), P1 + P2))
        og.append((first1, len(rows) - first1, P1))
    tables = np.full((len(rows), max(len(r) for r in rows)), -1, dtype=np.int32)
    for s, r in enumerate(rows):
        tables[s, :len(r)] = r
    q = (torch.randn((len(rows), H, D), generator=g) * q_std).to(TD[dtype])
    return q, kc, vc, tables, np.asarray(lens, dtype=np.int32), og, ig


def run_nested(native, q, kc, vc, tables, lens, og, ig, shift=0, inner_members=None):
    S, H, D = q.shape
    Hkv, B = kc.shape[1], kc.shape[2]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    arr = lambda gs, i: np.array([x[i] for x in gs], dtype=np.int32)
    max_ctx = int(lens.max())
    p1, p2 = arr(og, 2), arr(ig, 2) + shift
    m1, m2 = int(p1.max()), int(p2.max())
    im = inner_members or max(x[1] for x in ig)
    n = native.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, max_ctx, len(og), m1, len(ig),
                                                 m2, im, CODE[q.dtype])
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_prefix2(out, q.cuda(), kc.cuda(), vc.cuda(), dev(tables), dev(lens),
                                       max_ctx, dev(arr(og, 0)), dev(arr(og, 1)), dev(p1), m1,
                                       dev(arr(ig, 0)), dev(arr(ig, 1)), dev(p2), m2, im, ws)
    torch.cuda.synchronize()
    return out.cpu()


def check(native, dtype, case, what, shift=0, inner_members=None):
    q, kc, vc, tables, lens, og, ig = case
    got = run_nested(native, q, kc, vc, tables, lens, og, ig, shift, inner_members)
    want = decode_attention(q, kc, vc, tables, lens, kc.shape[2])
    assert np.isfinite(got.double().numpy()).all(), f"{what}: non-finite output"
    return assert_close(got, want, dtype, what)


SHAPES = [(dt, D, B) for dt in ("f32", "f16", "bf16") for D, B in ((64, 4), (128, 16), (128, 32))]


@pytest.mark.parametrize("dtype,D,B", SHAPES)
def test_nested_matches_whole_table_attention(native, dtype, D, B):
    """Beam-style pairs inside sampled groups: pairs sharing several blocks after the prompt,
    an inner part of zero, members with own parts of 0, 1, B - 1, B + 1 and more tokens, an
    inner group of one, texts in no group, and a group whose inner level is the only one."""
    outer = [(0, [(0, [37])]),
             (4 * 32, [(3 * 32, [5, 1]), (2 * 32, [B - 1, B + 1]), (0, [9, 70]), (32, [0, 3])]),
             (0, [(64, [11, 4])]),
             (8 * 32, [(5 * 32, [2, 40, 1]), (32, [17])]),
             (0, [(0, [128, 3])])]
    say(f"nested shared-prefix decode dtype={dtype} D={D} B={B}")
    case = make_nested(D * 10 + B, outer, 4, 4, D, B, dtype)
    check(native, dtype, case, f"{dtype} D={D} B={B}")


@pytest.mark.parametrize("H,Hkv", [(8, 4), (16, 4), (16, 2)])
def test_nested_with_shared_kv_heads(native, H, Hkv):
    """2, 4 and 8 query heads per key/value head (4, 2 and 1 members share a read)."""
    outer = [(64, [(48, [3, 17]), (16, [1, 40])]), (0, [(32, [20, 2])])]
    say(f"nested shared-prefix decode GQA H={H} Hkv={Hkv}")
    case = make_nested(H * 7 + Hkv, outer, H, Hkv, 128, 16, "f16")
    check(native, "f16", case, f"H={H} Hkv={Hkv}", inner_members=min(2, 8 * Hkv // H))


def test_nested_rounds_and_clamps(native):
    """Inner shared lengths off a block boundary round down; an inner length at or below the
    outer one leaves an empty inner part."""
    outer = [(64, [(32, [5, 6]), (16, [7, 8])]), (96, [(0, [1, 30])])]
    case = make_nested(5, outer, 4, 4, 128, 16, "bf16")
    check(native, "bf16", case, "inner + 7", shift=7)
    check(native, "bf16", case, "inner - 40", shift=-40)


def test_nested_sharp_scores(native):
    """Queries x32: a lost or doubled block at either level would show."""
    outer = [(256, [(128, [4, 40]), (64, [1, 100]), (32, [17, 3]), (0, [9, 60])])]
    case = make_nested(11, outer, 8, 8, 128, 16, "bf16", q_std=32.0)
    check(native, "bf16", case, "sharp")


@pytest.mark.parametrize("members", [1, 2, 3, 8])
def test_nested_inner_width(native, members):
    """The inner pass's width follows inner_members (1, 2, 4 and 8 query columns per
    key/value head); inner groups larger than it keep only their first members."""
    outer = [(64, [(32, [5, 6, 1]), (48, [2]), (16, [9, 3, 4, 30])])]
    case = make_nested(members, outer, 4, 4, 128, 16, "f16")
    check(native, "f16", case, f"inner_members={members}", inner_members=members)


def test_nested_rejects_too_wide_inner_groups(native):
    q, kc, vc, tables, lens, og, ig = make_nested(3, [(32, [(16, [3, 4])])], 8, 2, 64, 16, "f16")
    with pytest.raises(native.PagedKVError):
        run_nested(native, q, kc, vc, tables, lens, og, ig, inner_members=3)


def test_nested_inner_group_across_outer_groups(native):
    """An inner group whose members straddle two outer groups (and one text in none) keeps
    only the members whose outer part matches its first member's; the result is still the
    whole-table attention."""
    outer = [(64, [(32, [5, 6])]), (32, [(16, [7, 8])]), (0, [(0, [40])])]
    q, kc, vc, tables, lens, og, ig = make_nested(17, outer, 4, 4, 128, 16, "f16")
    # one inner group over texts 1 .. 4: text 1 in the first outer group, 2 and 3 in the
    # second, 4 in none (their tables agree on nothing beyond what the outer level covers)
    ig = [(0, 1, 64 + 32), (1, 4, 200)]
    check(native, "f16", (q, kc, vc, tables, lens, og, ig), "straddling inner group",
          inner_members=4)


def test_nested_inner_group_across_equal_outer_groups(native):
    """Two outer groups with the same shared length (the usual case: prompts of equal
    length) and an inner group straddling them: the members from the second outer group
    are left out of it (their outer group differs from the first member's, though their
    outer shared length is the same), so the result is still the whole-table attention.
    Sharp scores, so reading the first member's blocks for the others would show."""
    outer = [(64, [(32, [5, 6])]), (64, [(32, [7, 8])])]
    q, kc, vc, tables, lens, og, ig = make_nested(19, outer, 4, 4, 128, 16, "f16", q_std=32.0)
    # inner groups: text 0 alone, then texts 1 .. 3 (text 1 in the first outer group, texts
    # 2 and 3 in the second; all three have 64 outer tokens)
    ig = [(0, 1, 64 + 32), (1, 3, 64 + 32)]
    check(native, "f16", (q, kc, vc, tables, lens, og, ig), "inner group across equal outer groups",
          inner_members=4)


def test_nested_graph_replays_match_eager(native):
    """The whole call (start clear, both levels' set-ups and passes with their merges, the
    texts' own pass) captured into a HIP graph: every replay equals the eager call bit for
    bit, with eager work on the same buffers between replays."""
    case = make_nested(61, [(64, [(32, [5, 9]), (16, [3, 20])]), (32, [(48, [1, 4])])],
                       8, 4, 128, 16, "bf16")
    q, kc, vc, tables, lens, og, ig = case
    S, H, D = q.shape
    Hkv, B = kc.shape[1], kc.shape[2]
    say(f"prefix2 graph replay S={S} H={H}")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    arr = lambda gs, i: np.array([x[i] for x in gs], dtype=np.int32)
    max_ctx = int(lens.max())
    p1, p2 = arr(og, 2), arr(ig, 2)
    m1, m2, im = int(p1.max()), int(p2.max()), max(x[1] for x in ig)
    n = native.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, max_ctx, len(og), m1, len(ig),
                                                 m2, im, CODE[q.dtype])
    ins = (q.cuda(), kc.cuda(), vc.cuda(), dev(tables), dev(lens), max_ctx, dev(arr(og, 0)),
           dev(arr(og, 1)), dev(p1), m1, dev(arr(ig, 0)), dev(arr(ig, 1)), dev(p2), m2, im)
    ws_e = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    ws_g = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    out_e = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    out_g = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_prefix2(out_e, *ins, ws_e)
    native.pa_decode_attention_prefix2(out_g, *ins, ws_g)  # eager first: properties cached
    torch.cuda.synchronize()
    want = out_e.cpu()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        native.pa_decode_attention_prefix2(out_g, *ins, ws_g)
    torch.cuda.synchronize()
    for rep in range(4):
        out_g.fill_(float("nan"))
        ws_g.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out_g.cpu()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
    ref = decode_attention(q, kc, vc, tables, lens, B)
    assert_close(want, ref, "bf16", "prefix2 eager (graph test)")


def test_nested_past_the_one_launch_set_up(native):
    """More than 2,048 texts: the set-up runs as the clear and the two per-level kernels
    instead of the single set-up launch; the same attention as over the whole tables."""
    outer = [(16, [(16, [1 + (i + j) % 5, 2 + (i * j) % 4]) for j in range(4)]) for i in range(263)]
    case = make_nested(71, outer, 2, 2, 64, 16, "f16")
    assert case[0].shape[0] == 2104
    say("prefix2 with 2,104 texts (general set-up path)")
    check(native, "f16", case, "2,104 texts")


@pytest.mark.parametrize("dtype,H,Hkv", [("f16", 8, 4), ("bf16", 8, 8), ("f32", 4, 4)])
def test_nested_fused_write_equals_write_then_decode(native, dtype, H, Hkv):
    """pa_decode_attention_prefix2_write: outputs and whole pools bit for bit those of
    pa_kv_write then pa_decode_attention_prefix2, every text's newest key and value being
    new rows (stored by the texts' own pass); and the oracle over the written pools."""
    case = make_nested(81, [(32, [(16, [3, 7]), (16, [1, 17])]), (16, [(32, [2, 5]), (0, [9])])],
                       H, Hkv, 128, 16, dtype)
    q, kc, vc, tables, lens, og, ig = case
    S, _, D = q.shape
    B = kc.shape[2]
    say(f"prefix2 fused write {dtype} S={S} H={H} Hkv={Hkv}")
    g = torch.Generator().manual_seed(82)
    kn = (torch.randn((S, Hkv, D), generator=g) / math.sqrt(D)).to(TD[dtype])
    vn = (torch.randn((S, Hkv, D), generator=g) / math.sqrt(D)).to(TD[dtype])
    slots = torch.tensor([int(tables[s, (lens[s] - 1) // B]) * B + int(lens[s] - 1) % B
                          for s in range(S)], dtype=torch.int64)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    arr = lambda gs, i: np.array([x[i] for x in gs], dtype=np.int32)
    max_ctx = int(lens.max())
    p1, p2 = arr(og, 2), arr(ig, 2)
    m1, m2, im = int(p1.max()), int(p2.max()), max(x[1] for x in ig)
    n = native.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, max_ctx, len(og), m1, len(ig),
                                                 m2, im, CODE[q.dtype])
    groups = (dev(arr(og, 0)), dev(arr(og, 1)), dev(p1), m1, dev(arr(ig, 0)), dev(arr(ig, 1)),
              dev(p2), m2, im)
    qd, knd, vnd, sld = q.cuda(), kn.cuda(), vn.cuda(), slots.cuda()
    td, ld = dev(tables), dev(lens)
    # write, then decode
    ka, va = kc.cuda(), vc.cuda()
    out_a = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_kv_write(ka, va, knd, vnd, sld)
    native.pa_decode_attention_prefix2(out_a, qd, ka, va, td, ld, max_ctx, *groups,
                                       torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda"))
    # fused
    kb, vb = kc.cuda(), vc.cuda()
    out_b = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_prefix2_write(out_b, qd, kb, vb, knd, vnd, sld, td, ld, max_ctx,
                                             *groups,
                                             torch.full((n,), 0x5A, dtype=torch.uint8,
                                                        device="cuda"))
    torch.cuda.synchronize()
    bits = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}
    iv = lambda t: t.cpu().view(bits[t.dtype])
    assert torch.equal(iv(out_a), iv(out_b)), "outputs differ from write-then-decode"
    assert torch.equal(iv(ka), iv(kb)) and torch.equal(iv(va), iv(vb)), "pools differ"
    # the oracle over the pools with the new rows in place
    kw, vw = kc.clone(), vc.clone()
    for s in range(S):
        blk, off = int(slots[s]) // B, int(slots[s]) % B
        kw[blk, :, off] = kn[s]
        vw[blk, :, off] = vn[s]
    want = decode_attention(q, kw, vw, tables, lens, B)
    assert_close(out_b.cpu(), want, dtype, f"fused write {dtype}")


@pytest.mark.parametrize("dtype,H,Hkv", [("f16", 8, 4), ("bf16", 8, 8), ("f32", 4, 4)])
def test_nested_plan_once_runs_per_layer(native, dtype, H, Hkv):
    """pa_decode_prefix2_plan once, then pa_decode_attention_prefix2_run for three layers
    (each its own queries and pools), without and with new rows: bit for bit the one-call
    pa_decode_attention_prefix2 / _write of each layer (the runs leave the plan as it was);
    the last layer also against the oracle."""
    case = make_nested(83, [(32, [(16, [3, 7]), (16, [1, 17])]), (16, [(32, [2, 5]), (0, [9])])],
                       H, Hkv, 128, 16, dtype)
    q, kc, vc, tables, lens, og, ig = case
    S, _, D = q.shape
    B = kc.shape[2]
    say(f"prefix2 plan + runs {dtype} S={S} H={H} Hkv={Hkv}")
    g = torch.Generator().manual_seed(84)
    kn = (torch.randn((S, Hkv, D), generator=g) / math.sqrt(D)).to(TD[dtype])
    vn = (torch.randn((S, Hkv, D), generator=g) / math.sqrt(D)).to(TD[dtype])
    slots = torch.tensor([int(tables[s, (lens[s] - 1) // B]) * B + int(lens[s] - 1) % B
                          for s in range(S)], dtype=torch.int64)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    arr = lambda gs, i: np.array([x[i] for x in gs], dtype=np.int32)
    max_ctx = int(lens.max())
    p1, p2 = arr(og, 2), arr(ig, 2)
    m1, m2, im = int(p1.max()), int(p2.max()), max(x[1] for x in ig)
    n = native.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, max_ctx, len(og), m1, len(ig),
                                                 m2, im, CODE[q.dtype])
    groups = (dev(arr(og, 0)), dev(arr(og, 1)), dev(p1), m1, dev(arr(ig, 0)), dev(arr(ig, 1)),
              dev(p2), m2, im)
    counts = (len(og), m1, len(ig), m2, im)
    td, ld = dev(tables), dev(lens)
    knd, vnd, sld = kn.cuda(), vn.cuda(), slots.cuda()
    # layer l: heads of q rotated by l, keys negated and values halved on odd layers (exact in
    # every format; the pools' unused places stay NaN where they were)
    layers = []
    for li in range(3):
        sign, half = (-1.0, 0.5) if li % 2 else (1.0, 1.0)
        layers.append((q.roll(li, dims=1).contiguous(), kc * sign, vc * half))
    wsp = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    native.pa_decode_prefix2_plan(layers[0][0].cuda(), kc.cuda(), td, ld, max_ctx, *groups, wsp)
    bits = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}
    iv = lambda t: t.cpu().view(bits[t.dtype])
    for write in (False, True):
        for li, (ql, kl, vl) in enumerate(layers):
            qd = ql.cuda()
            ka, va, kb, vb = kl.cuda(), vl.cuda(), kl.cuda(), vl.cuda()
            out_a = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
            out_b = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
            ws1 = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
            if write:
                native.pa_decode_attention_prefix2_write(out_a, qd, ka, va, knd, vnd, sld, td, ld,
                                                         max_ctx, *groups, ws1)
                native.pa_decode_attention_prefix2_run(out_b, qd, kb, vb, td, ld, max_ctx, *counts,
                                                       wsp, k_new=knd, v_new=vnd, slots=sld)
            else:
                native.pa_decode_attention_prefix2(out_a, qd, ka, va, td, ld, max_ctx, *groups,
                                                   ws1)
                native.pa_decode_attention_prefix2_run(out_b, qd, kb, vb, td, ld, max_ctx, *counts,
                                                       wsp)
            torch.cuda.synchronize()
            what = f"layer {li}{' with new rows' if write else ''}"
            assert torch.equal(iv(out_a), iv(out_b)), f"{what}: outputs differ from one call"
            assert torch.equal(iv(ka), iv(kb)) and torch.equal(iv(va), iv(vb)), \
                f"{what}: pools differ"
    ql, kl, vl = layers[2]
    want = decode_attention(ql, kl, vl, tables, lens, B)
    assert_close(run_nested(native, ql, kl, vl, tables, lens, og, ig), want, dtype,
                 f"layer 2 {dtype}")


def test_nested_run_on_a_zeroed_workspace_decodes_whole_tables(native):
    """A zeroed workspace holds a plan of empty groups: every text starts at its first token
    with no shared state, so pa_decode_attention_prefix2_run without a plan call attends each
    text over its whole table (the oracle's result) and stays inside its arguments."""
    case = make_nested(85, [(32, [(16, [3, 7]), (16, [1, 17])]), (16, [(32, [2, 5]), (0, [9])])],
                       8, 8, 128, 16, "bf16")
    q, kc, vc, tables, lens, og, ig = case
    S, H, D = q.shape
    Hkv, B = kc.shape[1], kc.shape[2]
    say(f"prefix2 run on a zeroed workspace S={S}")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    max_ctx = int(lens.max())
    m1, m2, im = max(x[2] for x in og), max(x[2] for x in ig), max(x[1] for x in ig)
    n = native.pa_decode_prefix2_workspace_bytes(S, H, Hkv, D, B, max_ctx, len(og), m1, len(ig),
                                                 m2, im, CODE[q.dtype])
    ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_prefix2_run(out, q.cuda(), kc.cuda(), vc.cuda(), dev(tables),
                                           dev(lens), max_ctx, len(og), m1, len(ig), m2, im, ws)
    torch.cuda.synchronize()
    want = decode_attention(q, kc, vc, tables, lens, B)
    assert_close(out.cpu(), want, "bf16", "zeroed workspace")
