"""pa_kv_write and pa_copy_blocks on the GPU: whole pools bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from gpu_common import say
from oracle import cache_ops

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def random_pool(shape, dtype, g):
    # arbitrary bit patterns (NaN payloads, subnormals, -0.0 included)
    n = int(np.prod(shape)) * (4 if dtype == "f32" else 2)
    raw = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)
    return raw.view(TD[dtype]).reshape(shape).clone()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [4, 16, 32])
def test_kv_write_bit_exact(native, dtype, D, B):
    say(f"kv_write dtype={dtype} D={D} B={B}")
    g = torch.Generator().manual_seed(1000 + D + B)
    N, Hkv, T = 37, 3, 50
    kc, vc = random_pool((N, Hkv, B, D), dtype, g), random_pool((N, Hkv, B, D), dtype, g)
    kn, vn = random_pool((T, Hkv, D), dtype, g), random_pool((T, Hkv, D), dtype, g)
    rng = np.random.default_rng(D * B)
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int64)
    slots[3] = -1            # outside the pool: skipped by the kernel
    slots[7] = N * B + 5
    kd, vd = kc.cuda(), vc.cuda()
    native.pa_kv_write(kd, vd, kn.cuda(), vn.cuda(), torch.from_numpy(slots).cuda())
    keep = [i for i in range(T) if 0 <= slots[i] < N * B]
    ko, vo = kc.clone(), vc.clone()
    cache_ops.kv_write(ko, vo, kn[keep], vn[keep], slots[keep], B)
    torch.cuda.synchronize()
    assert torch.equal(bits(kd), bits(ko))
    assert torch.equal(bits(vd), bits(vo))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D,B", [(64, 4), (128, 16), (128, 32)])
def test_copy_blocks_bit_exact(native, dtype, D, B):
    say(f"copy_blocks dtype={dtype} D={D} B={B}")
    g = torch.Generator().manual_seed(2000 + D + B)
    N, Hkv = 40, 5
    kc, vc = random_pool((N, Hkv, B, D), dtype, g), random_pool((N, Hkv, B, D), dtype, g)
    rng = np.random.default_rng(B)
    blocks = rng.permutation(N)
    pairs = [(int(blocks[i]), int(blocks[i + 12])) for i in range(12)]  # disjoint src / dst
    pairs.append((5, N + 3))  # destination outside the pool: skipped
    kd, vd = kc.cuda(), vc.cuda()
    native.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32).cuda())
    ko, vo = kc.clone(), vc.clone()
    cache_ops.copy_blocks(ko, vo, pairs[:-1])
    torch.cuda.synchronize()
    assert torch.equal(bits(kd), bits(ko))
    assert torch.equal(bits(vd), bits(vo))


def test_empty_calls_are_no_ops(native):
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    empty = torch.zeros((0,), dtype=torch.int64, device="cuda")
    native.pa_kv_write(kc, vc, None, None, empty)
    native.pa_copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0 and int(vc.abs().sum()) == 0
