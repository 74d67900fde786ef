"""ds_copy, the same-pattern copy the scan is measured against: the copied
bytes equal the source and nothing past nbytes is written, at sizes that
end inside a wave segment, at a tile boundary and past it."""
import numpy as np
import pytest
import torch

import primitives_device_scan_amd as ds
from gpu_util import say, stream_handle

pytestmark = pytest.mark.gpu


def test_copy_sizes():
    tile = ds.lib.ds_tile_elems(ds.DS_UINT32, 0) * 4      # bytes per workgroup tile (4-byte scan)
    seg = tile // 4                                        # bytes per wave segment
    sizes = [16, 1008, seg - 16, seg, seg + 16, tile - 16, tile, tile + 16, 3 * tile + seg + 48,
             100_000_000 // 16 * 16]
    src = torch.randint(-2**31, 2**31 - 1, (max(sizes) // 4 + 64,), dtype=torch.int32, device="cuda")
    for nbytes in sizes:
        say("ds_copy", nbytes, "bytes")
        dst = torch.full_like(src, -1)
        assert ds.lib.ds_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream_handle()) == 0
        torch.cuda.synchronize()
        k = nbytes // 4
        assert torch.equal(dst[:k], src[:k]), nbytes
        assert bool((dst[k:] == -1).all()), f"{nbytes}: written past nbytes"
