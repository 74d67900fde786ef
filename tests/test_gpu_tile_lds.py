"""Parity of the 4,096-element LDS tile scans and of the three-kernel
pipeline built on them (through the C ABI) with the oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import CODE, assert_fp32_close, assert_int_equal, from_dev, sentinel_fill, stream_handle, to_dev

pytestmark = pytest.mark.gpu

TILE = 4096
VARIANTS = ["tree", "tree_pad1", "tree_pad2", "hillis_steele"]


def gpu_tile_scan(x, variant, in_place=False):
    n = x.size
    xin = to_dev(x)
    out = xin if in_place else torch.empty_like(xin)
    if not in_place:
        sentinel_fill(out)
    tiles = (n + TILE - 1) // TILE
    sums = torch.empty(max(tiles, 1), dtype=xin.dtype, device="cuda")
    st = ds.lib.ds_tile_scan(CODE[x.dtype], ds.TILE_VARIANTS[variant], xin.data_ptr(), out.data_ptr(),
                             sums.data_ptr(), n, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    return from_dev(out, x.dtype, 0, n), from_dev(sums, x.dtype, 0, tiles)


def gpu_pipeline(x, variant, in_place=False):
    xin = to_dev(x)
    out = xin if in_place else torch.empty_like(xin)
    st = ds.lib.ds_tile_pipeline(CODE[x.dtype], ds.TILE_VARIANTS[variant], xin.data_ptr(), out.data_ptr(), x.size,
                                 stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    return from_dev(out, x.dtype, 0, x.size)


def per_tile_oracle(x):
    n = x.size
    ys, ss, tots = [], [], []
    for t in range(0, n, TILE):
        chunk = x[t:t + TILE]
        if x.dtype == np.float32:
            y, s = oracle.scan(chunk, False)
            inc, _ = oracle.scan(chunk, True)
            ys.append(y), ss.append(s), tots.append(inc[-1])
        else:
            ys.append(oracle.scan(chunk, False))
            tots.append(oracle.scan(chunk, True)[-1])
    if x.dtype == np.float32:
        return np.concatenate(ys), np.concatenate(ss), np.array(tots)
    return np.concatenate(ys), None, np.array(tots, dtype=x.dtype)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dt", [np.int32, np.uint32, np.float32], ids=lambda d: np.dtype(d).name)
def test_tile_scan(dt, variant):
    for n in (1, 5, TILE - 1, TILE, TILE + 1, 7 * TILE + 123, 300 * TILE + 9):
        if dt == np.float32:
            x = datagen.normal_f32(900 + n, n)
        elif dt == np.int32:
            x = datagen.uniform_int(900 + n, n, -1000, 1000)
        else:
            x = datagen.keys_u32(900 + n, n)
        got, sums = gpu_tile_scan(x, variant)
        y, s, tots = per_tile_oracle(x)
        if dt == np.float32:
            assert_fp32_close(got, y, s, f"{variant} n={n}")
            assert np.all(np.abs(sums.astype(np.float64) - tots) <= 1e-5 * np.add.reduceat(np.abs(x.astype(np.float64)),
                                                                                            np.arange(0, n, TILE)))
        else:
            assert_int_equal(got, y, f"{variant} n={n}")
            assert_int_equal(sums, tots, f"{variant} n={n} tile totals")


@pytest.mark.parametrize("variant", VARIANTS)
def test_pipeline_exact_quarter_twos_10m(variant):
    """The page's exact check: 1.0 with every fourth element 2.0, n = 10,000,000."""
    n = 10_000_000
    x = datagen.quarter_twos_f32(n)
    i = np.arange(n, dtype=np.int64)
    got = gpu_pipeline(x, variant)
    assert_int_equal(got.astype(np.int64), i + i // 4, f"pipeline {variant}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_pipeline_random(variant):
    for n in (1, TILE, TILE + 1, 2442 * TILE - 5, 3_000_017):
        x = datagen.uniform_int(31 + n, n, -1000, 1000)
        assert_int_equal(gpu_pipeline(x, variant), oracle.scan(x, False), f"pipeline {variant} n={n}")
        f = datagen.normal_f32(32 + n, n)
        y, s = oracle.scan(f, False)
        assert_fp32_close(gpu_pipeline(f, variant), y, s, f"pipeline fp32 {variant} n={n}")


def test_in_place_and_errors():
    n = 5 * TILE + 7
    x = datagen.uniform_int(3, n, 0, 9)
    got, _ = gpu_tile_scan(x, "tree_pad2", in_place=True)
    assert_int_equal(got, per_tile_oracle(x)[0], "tile scan in place")
    assert_int_equal(gpu_pipeline(x, "tree", in_place=True), oracle.scan(x, False), "pipeline in place")
    t = torch.zeros(16, dtype=torch.int64, device="cuda")
    assert ds.lib.ds_tile_scan(3, 0, t.data_ptr(), t.data_ptr(), None, 16, None) == 2   # 8-byte types refused
    assert ds.lib.ds_tile_scan(0, 4, t.data_ptr(), t.data_ptr(), None, 16, None) == 1   # bad variant
