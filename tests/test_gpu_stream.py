"""GPU check of the stream probe (a measurement helper): every written 16-byte
chunk of tile t is the XOR of the tile's read chunks at the same lane, plus the
write index; reads and writes cover whole tiles, ragged tile counts included."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_fine_nf4_amd as nf4  # noqa: E402

DEV = "cuda:0"


@pytest.mark.parametrize("rd,wr", [(4, 1), (1, 4), (1, 0)])
@pytest.mark.parametrize("tiles", [1, 3, 4099])
@pytest.mark.parametrize("depth,blocks", [(2, 0), (1, 5), (4, 0), (8, 1)])
def test_stream_probe(rd, wr, tiles, depth, blocks):
    print(f"stream probe rd={rd} wr={wr} tiles={tiles} depth={depth} blocks={blocks}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(tiles * 7 + rd)
    src = torch.randint(0, 2**31 - 1, (tiles * 256 * rd,), dtype=torch.int32, device=DEV, generator=g)
    dst = torch.zeros(max(4, tiles * 256 * wr), dtype=torch.int32, device=DEV)
    nf4.qlora_stream_probe(rd, wr, src, dst, tiles, depth=depth, blocks=blocks)
    torch.cuda.synchronize()
    if wr == 0:
        return
    s = src.cpu().numpy().view(np.uint32).reshape(tiles, rd, 64, 4)
    x = s[:, 0]
    for j in range(1, rd):
        x = x ^ s[:, j]
    d = dst.cpu().numpy().view(np.uint32).reshape(tiles, wr, 64, 4)
    for k in range(wr):
        assert np.array_equal(d[:, k], (x + np.uint32(k)).astype(np.uint32))
