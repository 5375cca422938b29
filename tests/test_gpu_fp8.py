"""The 8-bit (E4M3) key/value cache on the GPU against the oracle, through the C ABI.

pa_kv_write_fp8: every stored code bit-exact with the oracle's quantization.
E4M3 widening in the decode kernel: all 256 codes through single-token texts.
pa_decode_attention_fp8: against the fp64 oracle on the dequantized pools.
"""
import math

import numpy as np
import pytest
import torch

from gpu_common import assert_close, say
from oracle import cache_ops, fp8
from oracle.attention import decode_attention

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D,B", [(64, 4), (128, 16), (128, 32)])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.05, 3.0), (0.3, 0.0071)])
def test_kv_write_fp8_bit_exact(native, src, D, B, scales):
    ks, vs = scales
    say(f"kv_write_fp8 src={src} D={D} B={B} scales={scales}")
    g = torch.Generator().manual_seed(D + B)
    N, Hkv, T = 23, 3, 40
    kc = torch.randint(0, 256, (N, Hkv, B, D), generator=g, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (N, Hkv, B, D), generator=g, dtype=torch.int32).to(torch.uint8)
    kn = (torch.randn((T, Hkv, D), generator=g) * 4).to(TD[src])
    vn = (torch.randn((T, Hkv, D), generator=g) * 0.02).to(TD[src])
    # saturation, NaN, signed zero and values far below the smallest code
    kn[0, 0, :4] = torch.tensor([1e4, -1e4, float("nan"), -0.0]).to(TD[src])
    vn[1, 0, :3] = torch.tensor([1e-9, -1e-9, 600.0]).to(TD[src])
    slots = np.random.default_rng(D).choice(N * B, size=T, replace=False).astype(np.int64)
    kd, vd = kc.cuda(), vc.cuda()
    native.pa_kv_write_fp8(kd, vd, kn.cuda(), vn.cuda(), torch.from_numpy(slots).cuda(), ks, vs)
    ko, vo = kc.clone(), vc.clone()
    cache_ops.kv_write_fp8(ko, vo, kn, vn, slots, B, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), ko) and torch.equal(vd.cpu(), vo)


def test_kv_write_rejects_fp8_pools_and_bad_scales(native):
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.uint8, device="cuda")
    kn = torch.zeros((1, 2, 128), dtype=torch.float16, device="cuda")
    s = torch.zeros(1, dtype=torch.int64, device="cuda")
    with pytest.raises(native.PagedKVError):
        native.pa_kv_write(kc, kc.clone(), kn, kn, s)
    with pytest.raises(native.PagedKVError):
        native.pa_kv_write_fp8(kc, kc.clone(), kn, kn, s, 0.0, 1.0)


@pytest.mark.parametrize("qt", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_every_code_widens_exactly(native, qt, D):
    """Texts of one token: out = decode(v code) * v_scale exactly, for all 256 codes."""
    B = 16
    S = 256 // D
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(S, D)
    kc = torch.zeros((S, 1, B, D), dtype=torch.uint8)
    vc = torch.zeros((S, 1, B, D), dtype=torch.uint8)
    vc[:, 0, 0, :] = codes
    tables = np.arange(S, dtype=np.int32).reshape(S, 1)
    lens = np.ones(S, dtype=np.int32)
    q = torch.randn((S, 1, D)).to(TD[qt])
    ws = native.decode_workspace(S, 1, D, 1, 0)
    out = torch.empty((S, 1, D), dtype=TD[qt], device="cuda")
    native.pa_decode_attention_fp8(out, q.cuda(), kc.cuda(), vc.cuda(), torch.from_numpy(tables).cuda(),
                                   torch.from_numpy(lens).cuda(), 1, ws, 1.0, 1.0)
    torch.cuda.synchronize()
    got = out.cpu().double().reshape(-1).numpy()
    want = fp8.DECODE_TABLE
    nan = np.isnan(want)
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan], want[~nan])


def make_fp8_case(seed, lens, H, Hkv, D, B, qt, k_scale, v_scale, extra=5):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    nblk = [(L + B - 1) // B for L in lens]
    N = sum(nblk) + extra
    kc = torch.full((N, Hkv, B, D), 0x7F, dtype=torch.uint8)   # NaN codes where unused
    vc = torch.full((N, Hkv, B, D), 0x7F, dtype=torch.uint8)
    perm = list(rng.permutation(N))
    tables = np.full((len(lens), max(1, max(nblk))), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        k = torch.randn((L, Hkv, D), generator=g) * 0.3
        v = torch.randn((L, Hkv, D), generator=g) * 0.3
        kq = cache_ops.quantize_rows(k, k_scale).reshape(L, Hkv, D)
        vq = cache_ops.quantize_rows(v, v_scale).reshape(L, Hkv, D)
        for j in range(nblk[s]):
            tables[s, j] = perm.pop()
        for t in range(L):
            kc[tables[s, t // B], :, t % B] = kq[t]
            vc[tables[s, t // B], :, t % B] = vq[t]
    q = torch.randn((len(lens), H, D), generator=g).to(TD[qt])
    return q, kc, vc, tables, np.asarray(lens, dtype=np.int32)


@pytest.mark.parametrize("qt", ["f16", "bf16"])
@pytest.mark.parametrize("D,B,H,Hkv", [(128, 16, 8, 8), (64, 4, 4, 2), (128, 32, 16, 2),
                                       (64, 16, 8, 1), (128, 8, 40, 40)])
def test_decode_fp8_matches_oracle(native, qt, D, B, H, Hkv):
    lens = [1, 15, 16, 33, 300, 1000]
    ks, vs = 0.02, 0.05
    say(f"decode_fp8 qt={qt} D={D} B={B} H={H} Hkv={Hkv}")
    q, kc, vc, tables, L = make_fp8_case(D + B + H, lens, H, Hkv, D, B, qt, ks, vs)
    want = decode_attention(q, kc, vc, tables, L, B, k_scale=ks, v_scale=vs)
    for T in (0, 32):
        ws = native.decode_workspace(len(lens), H, D, int(L.max()), T)
        out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
        native.pa_decode_attention_fp8(out, q.cuda(), kc.cuda(), vc.cuda(),
                                       torch.from_numpy(tables).cuda(), torch.from_numpy(L).cuda(),
                                       int(L.max()), ws, ks, vs, partition_tokens=T)
        torch.cuda.synchronize()
        assert_close(out.cpu(), want, qt, f"T={T}")


def test_copy_blocks_fp8_bit_exact(native):
    g = torch.Generator().manual_seed(9)
    kc = torch.randint(0, 256, (12, 4, 16, 128), generator=g, dtype=torch.int32).to(torch.uint8)
    vc = torch.randint(0, 256, (12, 4, 16, 128), generator=g, dtype=torch.int32).to(torch.uint8)
    pairs = [(1, 7), (3, 9), (0, 11)]
    kd, vd = kc.cuda(), vc.cuda()
    native.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32).cuda())
    ko, vo = kc.clone(), vc.clone()
    cache_ops.copy_blocks(ko, vo, pairs)
    torch.cuda.synchronize()
    assert torch.equal(kd.cpu(), ko) and torch.equal(vd.cpu(), vo)
