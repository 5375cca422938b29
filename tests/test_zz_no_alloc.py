"""pa_decode_attention_noalloc (the library's own workspace, no allocation) against
pa_decode_attention with a caller workspace, through the C ABI: bit-identical outputs on
two calls in a row, the second smaller than the first, and within the decode bar of the
fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle.attention import decode_attention
from test_gpu_decode import make_case

pytestmark = pytest.mark.gpu


def both(native, q, kc, vc, tables, lens, T):
    S, H, D = q.shape
    max_ctx = int(lens.max())
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    td, ld = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    ws = native.decode_workspace(S, H, D, max_ctx, T)
    ref = torch.full(q.shape, 7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention(ref, qd, kd, vd, td, ld, max_ctx, ws, partition_tokens=T)
    got = torch.full(q.shape, -7.0, dtype=q.dtype, device="cuda")
    native.pa_decode_attention_noalloc(got, qd, kd, vd, td, ld, max_ctx, partition_tokens=T)
    torch.cuda.synchronize()
    return ref.cpu(), got.cpu()


@pytest.mark.parametrize("dtype,H,Hkv,T", [("f16", 40, 40, 0), ("bf16", 16, 2, 0),
                                           ("f32", 8, 8, 512)])
def test_noalloc_matches_workspace_call(native, dtype, H, Hkv, T):
    """A large call, then a smaller one (fewer texts, shorter contexts): the second must not
    see anything the first left in the shared array."""
    for step, lens in enumerate(([2048, 1500, 17, 1, 777, 0, 3000], [300, 5, 64])):
        say(f"noalloc dtype={dtype} H={H} Hkv={Hkv} T={T} call {step} lens={lens}")
        kv_std = 1.0 if dtype == "f32" else 1.0 / math.sqrt(128)
        q, kc, vc, tables, L = make_case(40 + step, lens, H, Hkv, 128, 16, dtype, kv_std=kv_std)
        ref, got = both(native, q, kc, vc, tables, L, T)
        bits = torch.int32 if dtype == "f32" else torch.int16
        assert torch.equal(ref.view(bits), got.view(bits)), f"call {step}: outputs differ"
        want = decode_attention(q, kc, vc, tables, L, 16)
        assert_close(got, want, dtype, f"call {step}")


def test_noalloc_refuses_a_launch_past_its_workspace(native):
    """A launch whose workspace would exceed the built-in array is refused before launch."""
    limit = native.pa_decode_noalloc_max_bytes()
    S, H, D, max_ctx, T = 64, 40, 128, 32768, 16
    assert native.pa_decode_workspace_bytes(S, H, D, max_ctx, T) > limit
    q = torch.zeros((S, H, D), dtype=torch.float16, device="cuda")
    kc = torch.zeros((4, H, 16, D), dtype=torch.float16, device="cuda")
    tables = torch.zeros((S, 2048), dtype=torch.int32, device="cuda")
    lens = torch.ones((S,), dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(native.PagedKVError):
        native.pa_decode_attention_noalloc(out, q, kc, kc, tables, lens, max_ctx,
                                           partition_tokens=T)
    torch.cuda.synchronize()
    assert (out == 7.0).all(), "nothing may be launched"
