"""pa_decode_attention_prefix (decode over blocks shared by groups of texts, read once per
group) on the GPU: the same attention as over each text's whole table, within the decode
tolerance of the fp64 oracle (attention.decode_attention over the full tables)."""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def make_batch(seed, groups, H, Hkv, D, B, dtype, q_std=1.0, extra=7):
    """groups: list of (shared_tokens, [own tokens of each member]); shared_tokens is a
    block multiple, 0 for texts in no group. Members hold the same physical blocks for
    their first shared_tokens tokens and blocks of their own after them (randomly placed,
    unused places NaN). Returns q, pools, tables, lens and the members of each group."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nshared = [P // B for P, _ in groups]
    nown = [[(n + B - 1) // B for n in own] for _, own in groups]
    N = sum(nshared) + sum(sum(x) for x in nown) + extra
    perm = list(rng.permutation(N))
    kc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[dtype])
    vc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[dtype])
    std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(D)

    def fill(blocks, ntok):
        k = (torch.randn((ntok, Hkv, D), generator=g) * std).to(TD[dtype])
        v = (torch.randn((ntok, Hkv, D), generator=g) * std).to(TD[dtype])
        for t in range(ntok):
            kc[blocks[t // B], :, t % B] = k[t]
            vc[blocks[t // B], :, t % B] = v[t]

    rows, lens, members = [], [], []
    for (P, own), nb, no in zip(groups, nshared, nown):
        shared = [perm.pop() for _ in range(nb)]
        fill(shared, P)
        first = len(rows)
        for n, k in zip(own, no):
            mine = [perm.pop() for _ in range(k)]
            fill(mine, n)
            rows.append(shared + mine)
            lens.append(P + n)
        members.append((first, len(own), P))
    tables = np.full((len(rows), max(len(r) for r in rows)), -1, dtype=np.int32)
    for s, r in enumerate(rows):
        tables[s, :len(r)] = r
    q = (torch.randn((len(rows), H, D), generator=g) * q_std).to(TD[dtype])
    return q, kc, vc, tables, np.asarray(lens, dtype=np.int32), members


def run_prefix(native, q, kc, vc, tables, lens, first, count, prefix, max_prefix):
    S, H, D = q.shape
    Hkv, B = kc.shape[1], kc.shape[2]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    max_ctx = int(lens.max())
    n = native.pa_decode_prefix_workspace_bytes(S, H, Hkv, D, B, max_ctx, max(len(first), 1),
                                                max_prefix, CODE[q.dtype])
    # a workspace full of garbage: the call needs none of it initialized
    ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_prefix(out, q.cuda(), kc.cuda(), vc.cuda(), dev(tables),
                                      dev(lens), max_ctx, dev(first), dev(count), dev(prefix),
                                      max_prefix, ws)
    torch.cuda.synchronize()
    return out.cpu()


def check(native, dtype, case, what, prefix_shift=0, count_override=None):
    q, kc, vc, tables, lens, members = case
    grouped = [(f, n, P) for f, n, P in members if P > 0]
    first = np.array([f for f, _, _ in grouped], dtype=np.int32)
    count = np.array([n for _, n, _ in grouped], dtype=np.int32)
    if count_override is not None:
        count = np.array(count_override, dtype=np.int32)
    prefix = np.array([P + prefix_shift for _, _, P in grouped], dtype=np.int32)
    max_prefix = int(prefix.max()) if len(prefix) else 0
    got = run_prefix(native, q, kc, vc, tables, lens, first, count, prefix, max_prefix)
    want = decode_attention(q, kc, vc, tables, lens, kc.shape[2])
    assert np.isfinite(got.double().numpy()).all(), f"{what}: non-finite output"
    return assert_close(got, want, dtype, what)


SHAPES = [(dt, D, B) for dt in ("f32", "f16", "bf16") for D in (64, 128) for B in (4, 16, 32)]


@pytest.mark.parametrize("dtype,D,B", SHAPES)
def test_prefix_matches_whole_table_attention(native, dtype, D, B):
    """Eight members with own parts of 0 (the group then shares one block less), 1, B - 1,
    B, B + 1 and more tokens; a group of three (unused query columns); texts in no group
    before, between and after; a long shared part split over several segments."""
    P1, P2 = 4 * 32, 20 * 32
    groups = [(0, [37]),
              (P1, [0, 1, B - 1, B, B + 1, 3, 70, 2]),
              (0, [5, 1]),
              (P2, [9, 300, 1]),
              (0, [128])]
    say(f"shared-prefix decode dtype={dtype} D={D} B={B}")
    case = make_batch(D * 100 + B, groups, 4, 4, D, B, dtype)
    check(native, dtype, case, f"{dtype} D={D} B={B}")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("H,Hkv", [(8, 4), (12, 4), (16, 2), (6, 2)])
def test_prefix_with_shared_kv_heads(native, dtype, H, Hkv):
    """2, 3 and 8 query heads per key/value head: 4, 2 and 1 members share a read (the
    members past that decode on their own)."""
    groups = [(48, [3, 17, 1, 40, 5]), (0, [20]), (160, [1, 2])]
    say(f"shared-prefix decode GQA dtype={dtype} H={H} Hkv={Hkv}")
    case = make_batch(H * 13 + Hkv, groups, H, Hkv, 128, 16, dtype)
    check(native, dtype, case, f"H={H} Hkv={Hkv}")


def test_prefix_rounds_and_clamps_the_shared_length(native):
    """A shared length off a block boundary is rounded down; counts past the 8 columns
    (and past the batch) leave the extra members to decode on their own."""
    groups = [(64, [5, 6, 7, 8, 9, 10, 11, 12, 13, 14]), (96, [1, 30])]
    case = make_batch(5, groups, 4, 4, 128, 16, "f16")
    check(native, "f16", case, "shared length + 7", prefix_shift=7)
    check(native, "f16", case, "counts 10 and 9", count_override=[10, 9])


def test_prefix_sharp_scores(native):
    """Queries x32 (score spread ~2.8): softmax far from uniform, so a lost or doubled
    shared block would show."""
    groups = [(256, [4, 40, 1, 100, 17, 3, 9, 60]), (0, [33])]
    case = make_batch(11, groups, 8, 8, 128, 16, "bf16", q_std=32.0)
    check(native, "bf16", case, "sharp")


def test_prefix_without_groups_is_plain_decode(native):
    q, kc, vc, tables, lens, _ = make_batch(3, [(0, [50, 7, 300])], 4, 4, 64, 16, "f16")
    got = run_prefix(native, q, kc, vc, tables, lens, np.zeros(0, np.int32),
                     np.zeros(0, np.int32), np.zeros(0, np.int32), 0)
    assert_close(got, decode_attention(q, kc, vc, tables, lens, 16), "f16", "no groups")


def test_prefix_rejects_more_than_8_heads_per_kv_head(native):
    q, kc, vc, tables, lens, members = make_batch(2, [(32, [3, 4])], 16, 1, 64, 16, "f16")
    with pytest.raises(native.PagedKVError):
        run_prefix(native, q, kc, vc, tables, lens, np.array([0], np.int32),
                   np.array([2], np.int32), np.array([32], np.int32), 32)
