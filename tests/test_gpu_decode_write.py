"""pa_decode_attention_write (the step's new-token write fused into decode attention)
on the GPU: bit for bit the result of pa_kv_write followed by pa_decode_attention, pools
included, and within the decode tolerance of the fp64 oracle (cache_ops.kv_write, then
attention.decode_attention)."""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle import cache_ops
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def make_step(seed, lens, H, Hkv, D, B, dtype, extra=5, q_std=1.0):
    """Texts attending lens[s] tokens this step: tokens 0 .. lens[s] - 2 already cached in
    randomly placed blocks (unused places NaN), the new token's place (position
    lens[s] - 1) in its block; k_new / v_new / q of the step."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nblk = [max(1, (L + B - 1) // B) for L in lens]
    N = sum(nblk) + extra
    kc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[dtype])
    vc = torch.full((N, Hkv, B, D), float("nan"), dtype=TD[dtype])
    perm = list(rng.permutation(N))
    tables = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
    slots = np.zeros(len(lens), dtype=np.int64)
    std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(D)
    for s, L in enumerate(lens):
        for j in range(nblk[s]):
            tables[s, j] = perm.pop()
        k = (torch.randn((max(L - 1, 0), Hkv, D), generator=g) * std).to(TD[dtype])
        v = (torch.randn((max(L - 1, 0), Hkv, D), generator=g) * std).to(TD[dtype])
        for t in range(L - 1):
            kc[tables[s, t // B], :, t % B] = k[t]
            vc[tables[s, t // B], :, t % B] = v[t]
        p = max(L - 1, 0)  # a text with an empty context still names a place (not written)
        slots[s] = int(tables[s, p // B]) * B + p % B
    kn = (torch.randn((len(lens), Hkv, D), generator=g) * std).to(TD[dtype])
    vn = (torch.randn((len(lens), Hkv, D), generator=g) * std).to(TD[dtype])
    q = (torch.randn((len(lens), H, D), generator=g) * q_std).to(TD[dtype])
    return q, kc, vc, kn, vn, slots, tables, np.asarray(lens, dtype=np.int32)


def run_both(native, q, kc, vc, kn, vn, slots, tables, lens, partition_tokens=0):
    S, H, D = q.shape
    max_ctx = int(lens.max())
    dev = lambda a: torch.from_numpy(a).cuda()
    # separate launches: the write skips texts with an empty context (slot -1)
    k1, v1 = kc.cuda(), vc.cuda()
    written = np.where(lens >= 1, slots, -1).astype(np.int64)
    native.pa_kv_write(k1, v1, kn.cuda(), vn.cuda(), dev(written))
    ws1 = native.decode_workspace(S, H, D, max_ctx, partition_tokens)
    o1 = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention(o1, q.cuda(), k1, v1, dev(tables), dev(lens), max_ctx, ws1,
                               partition_tokens=partition_tokens)
    # fused
    k2, v2 = kc.cuda(), vc.cuda()
    ws2 = native.decode_workspace(S, H, D, max_ctx, partition_tokens)
    o2 = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_write(o2, q.cuda(), k2, v2, kn.cuda(), vn.cuda(), dev(slots),
                                     dev(tables), dev(lens), max_ctx, ws2,
                                     partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    return (o1.cpu(), k1.cpu(), v1.cpu()), (o2.cpu(), k2.cpu(), v2.cpu()), written


def check(native, dtype, case, what, partition_tokens=0):
    q, kc, vc, kn, vn, slots, tables, lens = case
    B = kc.shape[2]
    (o1, k1, v1), (o2, k2, v2), written = run_both(native, q, kc, vc, kn, vn, slots, tables, lens,
                                                   partition_tokens)
    assert torch.equal(bits(o1), bits(o2)), f"{what}: outputs differ from write + decode"
    assert torch.equal(bits(k1), bits(k2)) and torch.equal(bits(v1), bits(v2)), \
        f"{what}: pools differ from write + decode"
    # the oracle: write the new rows into the pools, then attend
    kw, vw = kc.clone(), vc.clone()
    keep = [i for i in range(len(lens)) if written[i] >= 0]
    cache_ops.kv_write(kw, vw, kn[keep], vn[keep], written[keep], B)
    assert torch.equal(bits(kw), bits(k2)) and torch.equal(bits(vw), bits(v2)), \
        f"{what}: pools vs the oracle's write"
    want = decode_attention(q, kw, vw, tables, lens, B)
    assert_close(o2, want, dtype, what)


SHAPES = [(dt, D, B) for dt in ("f32", "f16", "bf16") for D in (64, 128) for B in (4, 8, 16, 32)]


@pytest.mark.parametrize("dtype,D,B", SHAPES)
def test_fused_equals_write_then_decode(native, dtype, D, B):
    lens = [1, 2, 16, 17, 40, 129, 300, 0, 33]
    say(f"decode+write dtype={dtype} D={D} B={B}")
    case = make_step(D * 10 + B, lens, 4, 4, D, B, dtype)
    check(native, dtype, case, f"{dtype} D={D} B={B}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("H,Hkv", [(8, 4), (12, 4), (16, 4), (32, 4), (64, 4), (6, 2)])
def test_fused_with_shared_kv_heads(native, dtype, H, Hkv):
    """2, 3, 4, 8 and 16 query heads per key/value head: vector and matrix-core kernels,
    and (16) two runs per key/value head, of which only the first writes."""
    lens = [5, 64, 65, 250, 1]
    say(f"decode+write GQA dtype={dtype} H={H} Hkv={Hkv}")
    case = make_step(H * 7 + Hkv, lens, H, Hkv, 128, 16, dtype)
    check(native, dtype, case, f"H={H} Hkv={Hkv}")


@pytest.mark.parametrize("T", [16, 48])
def test_fused_with_short_segments(native, T):
    """Fixed segment lengths: every run ends in another segment than it starts."""
    lens = [300, 17, 1000, 64]
    case = make_step(T, lens, 8, 8, 128, 16, "f16")
    check(native, "f16", case, f"partition_tokens={T}", partition_tokens=T)


def test_fused_rejects_e4m3_pools(native):
    q = torch.zeros((2, 4, 128), dtype=torch.float16, device="cuda")
    kc = torch.zeros((4, 4, 16, 128), dtype=torch.uint8, device="cuda")
    kn = torch.zeros((2, 4, 128), dtype=torch.float16, device="cuda")
    t = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    L = torch.ones(2, dtype=torch.int32, device="cuda")
    ws = native.decode_workspace(2, 4, 128, 1, 0)
    with pytest.raises((native.PagedKVError, AssertionError)):
        native.pa_decode_attention_write(q.clone(), q, kc, kc, kn, kn,
                                         torch.zeros(2, dtype=torch.int64, device="cuda"),
                                         t, L, 1, ws)
