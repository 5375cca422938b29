"""The debug re-checks (pa_set_debug_checks) on the GPU, through the C ABI: each promise the
device calls take on trust is refused when broken, before anything is launched, and calls
that keep it give the same bits as with the checks off."""
import math

import numpy as np
import pytest
import torch

from gpu_common import say
from test_gpu_decode import make_case
from test_gpu_decode_prefix import make_batch, run_prefix
from test_gpu_decode_prefix2 import make_nested, run_nested

pytestmark = pytest.mark.gpu


@pytest.fixture
def checks(native):
    native.pa_set_debug_checks(True)
    assert native.pa_debug_checks()
    yield native
    native.pa_set_debug_checks(False)


def pools(N=8, Hkv=2, B=4, D=64):
    k = torch.full((N, Hkv, B, D), float("nan"), dtype=torch.float16, device="cuda")
    return k, k.clone()


def test_kv_write_slots(checks):
    L = checks
    kc, vc = pools()
    new = torch.randn((2, 2, 64), dtype=torch.float16, device="cuda")
    dup = torch.tensor([5, 5], dtype=torch.int64, device="cuda")
    with pytest.raises(L.PagedKVError, match="slot 5"):
        L.pa_kv_write(kc, vc, new, new, dup)
    torch.cuda.synchronize()
    assert torch.isnan(kc.float()).all(), "nothing may be written"
    # a slot outside the pool is skipped, not a duplicate
    L.pa_kv_write(kc, vc, new, new, torch.tensor([5, 10 ** 6], dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(kc[1, :, 1], new[0])


def test_copy_pairs(checks):
    L = checks
    kc, vc = pools()
    i32 = dict(dtype=torch.int32, device="cuda")
    for bad in ([[1, 2], [3, 2]], [[1, 2], [2, 3]], [[4, 4]]):
        with pytest.raises(L.PagedKVError):
            L.pa_copy_blocks(kc, vc, torch.tensor(bad, **i32))
    L.pa_copy_blocks(kc, vc, torch.tensor([[1, 2], [1, 3], [9, 0]], **i32))  # one source twice
    torch.cuda.synchronize()


def test_fused_write_slot_is_the_last_position(checks):
    L = checks
    lens = [5, 33, 17]
    q, kc, vc, tables, lens_np = make_case(3, lens, 4, 4, 64, 16, "f16", kv_std=0.125)
    S, H, D = q.shape
    slots = np.array([tables[s, (n - 1) // 16] * 16 + (n - 1) % 16 for s, n in enumerate(lens)],
                     dtype=np.int64)
    dev = lambda a: torch.from_numpy(a).cuda()
    kn = torch.randn((S, 4, D), dtype=torch.float16).cuda()
    ws = L.decode_workspace(S, H, D, max(lens))

    def run(sl):
        out = torch.empty_like(q).cuda()
        kd, vd = kc.cuda(), vc.cuda()
        L.pa_decode_attention_write(out, q.cuda(), kd, vd, kn, kn, dev(sl), dev(tables),
                                    dev(lens_np), max(lens), ws)
        torch.cuda.synchronize()
        return out.cpu()

    got = run(slots)
    L.pa_set_debug_checks(False)
    plain = run(slots)
    L.pa_set_debug_checks(True)
    assert torch.equal(got.view(torch.int16), plain.view(torch.int16))
    wrong = slots.copy()
    wrong[1] += 1
    with pytest.raises(L.PagedKVError, match="last position"):
        run(wrong)


def test_prefix_groups(checks):
    L = checks
    q, kc, vc, tables, lens, members = make_batch(21, [(64, [5, 9, 1]), (32, [7, 3])], 4, 4,
                                                   128, 16, "f16")
    f = np.array([m[0] for m in members], np.int32)
    c = np.array([m[1] for m in members], np.int32)
    p = np.array([m[2] for m in members], np.int32)
    got = run_prefix(L, q, kc, vc, tables, lens, f, c, p, 64)
    L.pa_set_debug_checks(False)
    plain = run_prefix(L, q, kc, vc, tables, lens, f, c, p, 64)
    L.pa_set_debug_checks(True)
    assert torch.equal(got.view(torch.int16), plain.view(torch.int16))
    # a member whose table does not begin with its group's blocks
    bad = tables.copy()
    bad[1, 2] = bad[4, 0]
    with pytest.raises(L.PagedKVError, match="group 0"):
        run_prefix(L, q, kc, vc, bad, lens, f, c, p, 64)
    # overlapping groups
    with pytest.raises(L.PagedKVError, match="groups"):
        run_prefix(L, q, kc, vc, tables, lens, np.array([0, 2], np.int32),
                   np.array([3, 2], np.int32), np.array([64, 32], np.int32), 64)


def test_nested_groups(checks):
    L = checks
    outer = [(64, [(32, [5, 6]), (16, [7, 8])])]
    q, kc, vc, tables, lens, og, ig = make_nested(23, outer, 4, 4, 128, 16, "f16")
    got = run_nested(L, q, kc, vc, tables, lens, og, ig)
    L.pa_set_debug_checks(False)
    plain = run_nested(L, q, kc, vc, tables, lens, og, ig)
    L.pa_set_debug_checks(True)
    assert torch.equal(got.view(torch.int16), plain.view(torch.int16))
    # an inner group claiming more blocks than its members share
    ig_bad = [(0, 4, 64 + 32)]
    with pytest.raises(L.PagedKVError, match="level 2"):
        run_nested(L, q, kc, vc, tables, lens, og, ig_bad, inner_members=4)
