"""The measurement helpers read (and copy) exactly the bytes they claim: the XOR of every
32-bit word they read, folded into their sink, matches the same XOR taken on the host."""
import numpy as np
import pytest
import torch

from gpu_common import say

pytestmark = pytest.mark.gpu


def xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel()))


def sink_xor(sink) -> int:
    return xor_words(sink.cpu().numpy())


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 << 20, (16 << 20) + 48,
                                    (40 << 20) + 3 * 4096 + 16])
def test_stream_read_probe_reads_every_word(native, nbytes):
    say(f"stream read probe {nbytes} B")
    g = torch.Generator().manual_seed(nbytes)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    sink = torch.zeros(native.pa_probe_sink_bytes(0), dtype=torch.uint8, device="cuda")
    native.pa_stream_read_probe(buf.cuda(), sink)
    torch.cuda.synchronize()
    assert sink_xor(sink) == xor_words(buf.numpy())


@pytest.mark.parametrize("tile", [2048, 4096, 8192, 16384])
def test_tile_read_probe_reads_the_listed_tiles(native, tile):
    say(f"tile read probe tile={tile}")
    g = torch.Generator().manual_seed(tile)
    ntiles = 300
    buf = torch.randint(0, 256, (ntiles * tile,), dtype=torch.uint8, generator=g)
    ids = torch.randint(0, ntiles, (1037,), dtype=torch.int32, generator=g)
    ids[5] = -3            # clamped to tile 0
    ids[9] = ntiles + 7    # clamped to the last tile
    sink = torch.zeros(native.pa_probe_sink_bytes(4), dtype=torch.uint8, device="cuda")
    native.pa_tile_read_probe(buf.cuda(), tile, ids.cuda(), sink)
    torch.cuda.synchronize()
    tiles = buf.numpy().reshape(ntiles, tile)
    want = 0
    for i in np.clip(ids.numpy(), 0, ntiles - 1):
        want ^= xor_words(tiles[i])
    assert sink_xor(sink) == want


def test_tile_read_probe_rejects_other_tile_sizes(native):
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(native.pa_probe_sink_bytes(4), dtype=torch.uint8, device="cuda")
    with pytest.raises(native.PagedKVError):
        native.pa_tile_read_probe(buf, 1024, ids, sink)


def test_copy_probe_copies(native):
    g = torch.Generator().manual_seed(3)
    src = torch.randint(0, 256, ((1 << 20) + 32,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros_like(src)
    native.pa_copy_probe(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
