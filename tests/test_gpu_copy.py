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



def _read_half_expected(src_vecs, nvec, vpt):
    """Where the read-half probes put each vector: workgroup b's thread
    t = 64 w + l loads vector b*256*vpt + w*64*vpt + k*64 + l as its k-th, and
    the first vpt/2 of them go to vector b*128*vpt + k*256 + t."""
    out = {}
    per = 256 * vpt
    for b in range((nvec + per - 1) // per):
        for k in range(vpt // 2):
            for t in range(256):
                w, l = divmod(t, 64)
                src = b * per + w * 64 * vpt + k * 64 + l
                dst = b * per // 2 + k * 256 + t
                if src < nvec and dst < nvec:
                    out[dst] = src
    return out


@pytest.mark.parametrize("mode", ["copy", "copy_held", "read_half", "read_half_held"])
def test_bandwidth_pattern_bytes(mode):
    """The ceiling probes move the bytes they claim: the copies equal the
    source, the read-half forms place each workgroup's first vpt/2 vectors per
    thread at the workgroup's compacted position, and nothing else is written.
    Values below 2^24 keep the held forms' gate (a fold of the tile compared
    with a constant above 2^24) shut."""
    code = ds._binding.PATTERNS[mode]
    vpt = 16
    tile = 256 * vpt * 16                                  # bytes per workgroup
    for nbytes in (tile, 5 * tile, 2 * tile + 4096 + 512):
        say("ds_bandwidth_pattern", mode, nbytes, "bytes")
        k = nbytes // 4
        src = torch.randint(0, 1 << 24, (k + 64,), dtype=torch.int32, device="cuda")
        dst = torch.full_like(src, -1)
        assert ds.lib.ds_bandwidth_pattern(code, vpt, 0, src.data_ptr(), dst.data_ptr(), nbytes, stream_handle()) == 0
        torch.cuda.synchronize()
        if mode.startswith("copy"):
            assert torch.equal(dst[:k], src[:k]), nbytes
            assert bool((dst[k:] == -1).all()), f"{nbytes}: written past nbytes"
        else:
            s = src.cpu().numpy().reshape(-1, 4)
            d = dst.cpu().numpy().reshape(-1, 4)
            want = np.full_like(d, -1)
            for dv, sv in _read_half_expected(s, nbytes // 16, vpt).items():
                want[dv] = s[sv]
            assert np.array_equal(d, want), nbytes
