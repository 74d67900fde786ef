"""ds_scan_seeded: one shard of a longer scan, through the C ABI.

A sequence is cut into contiguous shards, as a scan split over several GPUs
would be. On the GPU, each shard's total is taken (the last element of its
inclusive scan), the totals are scanned (exclusive), and each shard is then
scanned seeded with its offset read from device memory. The concatenated
result must equal the oracle's scan of the whole sequence: bit-exact for
integers (wrapping), within 1e-5 * S_i for fp32. The shards run one after the
other here, on one GPU, at the per-GPU shape of an eight-way split.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import CODE, FP32_TOL, STORAGE, assert_int_equal, from_dev, say, stream_handle, to_dev

pytestmark = pytest.mark.gpu


def cut(n: int, shards: int, seed: int):
    """Shard boundaries 0 = b_0 <= ... <= b_shards = n: uneven, one shard empty and one of a single
    element when there is room, starts mostly off 16-byte alignment."""
    rng = np.random.default_rng(seed)
    inner = np.sort(rng.choice(np.arange(1, n), size=shards - 1, replace=False)) if n > shards else \
        np.linspace(0, n, shards + 1)[1:-1].astype(np.int64)
    b = [0, *inner.tolist(), n]
    if n > 1000 and shards >= 4:
        b[2] = b[1]          # an empty shard
        b[3] = b[2] + 1      # a one-element shard
    return b


def sharded_scan(x: np.ndarray, inclusive: bool, bounds) -> np.ndarray:
    code = CODE[x.dtype]
    snp, st = STORAGE[x.dtype]
    k = len(bounds) - 1
    sh = stream_handle()
    dx = to_dev(x)
    tmp = torch.empty_like(dx)
    totals = torch.zeros(k, dtype=st, device="cuda")
    for g in range(k):
        a, b = bounds[g], bounds[g + 1]
        if b > a:
            assert ds.lib.ds_scan(code, 1, 0, dx[a:].data_ptr(), tmp[a:].data_ptr(), b - a, sh) == 0
            totals[g:g + 1].copy_(tmp[b - 1:b])
    seeds = torch.empty_like(totals)
    assert ds.lib.ds_scan(code, 0, 0, totals.data_ptr(), seeds.data_ptr(), k, sh) == 0
    out = torch.empty_like(dx)
    for g in range(k):
        a, b = bounds[g], bounds[g + 1]
        st_ = ds.lib.ds_scan_seeded(code, int(inclusive), dx[a:].data_ptr(), out[a:].data_ptr(), b - a,
                                    seeds[g:].data_ptr(), sh)
        assert st_ == 0, ds.lib.ds_status_string(st_)
    assert not ds.query_timeout()
    return from_dev(out, x.dtype)


CASES = [
    ("int32 wrapping", lambda n: datagen.uniform_int(41, n, -(1 << 30), 1 << 30), 10_000_019),
    ("uint32", lambda n: datagen.keys_u32(42, n), 10_000_019),
    ("int64 wrapping", lambda n: datagen.uniform_i64(43, n, 62), 10_000_019),
    ("fp32", lambda n: datagen.normal_f32(44, n), 10_000_019),
    ("int32 small", lambda n: datagen.uniform_int(45, n, -1000, 1000), 5_000),
    ("int32 at the 100M shape", lambda n: datagen.workload("int32_100m", n), 100_000_007),
]


@pytest.mark.parametrize("inclusive", [False, True])
@pytest.mark.parametrize("name,make,n", CASES, ids=[c[0] for c in CASES])
def test_sharded_scan_equals_the_whole_scan(name, make, n, inclusive):
    say("seeded shards:", name, "n =", n, "inclusive =", inclusive)
    x = make(n)
    bounds = cut(n, 8, n % 1000)
    got = sharded_scan(x, inclusive, bounds)
    want = oracle.scan(x, inclusive)
    if x.dtype == np.float32:
        y, s = want
        err = np.abs(got.astype(np.float64) - y)
        assert np.all(err <= FP32_TOL * s), f"{name}: max |err|/S = {np.max(err / np.maximum(s, 1e-300))}"
    else:
        assert_int_equal(got, want, f"{name} inclusive={inclusive}")


def test_null_seed_is_the_plain_scan():
    n = 3 * 24_576 + 77
    x = datagen.uniform_int(46, n, -1000, 1000)
    dx = to_dev(x)
    out = torch.empty_like(dx)
    assert ds.lib.ds_scan_seeded(0, 0, dx.data_ptr(), out.data_ptr(), n, None, stream_handle()) == 0
    assert_int_equal(from_dev(out, np.int32), oracle.scan(x, False), "null seed")


def test_seed_on_a_single_tile_and_in_place():
    # one tile (no look-back) takes the seed as its prefix; the output may be the input
    x = datagen.uniform_int(47, 1000, 0, 9)
    seed = np.array([123456], dtype=np.int32)
    for inclusive in (False, True):
        dx, dseed = to_dev(x), to_dev(seed)
        assert ds.lib.ds_scan_seeded(0, int(inclusive), dx.data_ptr(), dx.data_ptr(), x.size, dseed.data_ptr(),
                                     stream_handle()) == 0
        want = oracle.scan(x, inclusive) + np.int32(123456)
        assert_int_equal(from_dev(dx, np.int32), want, f"single tile inclusive={inclusive}")


def test_binding():
    x = torch.arange(1, 50_001, dtype=torch.int64, device="cuda")
    seed = torch.tensor([1000], dtype=torch.int64, device="cuda")
    y = ds.scan_seeded(x, True, seed).cpu().numpy()
    k = np.arange(1, 50_001, dtype=np.int64)
    assert np.array_equal(y, 1000 + k * (k + 1) // 2)
    with pytest.raises(ValueError):
        ds.scan_seeded(x, True, seed.to(torch.int32))
