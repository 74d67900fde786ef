"""ds_scan_noalloc (the look-back scan with its control block and status
words in the library's fixed device array) against the allocating entry
point, ds_scan with DS_ALGO_LOOKBACK, through the C ABI: integers bit-exact
and equal to the oracle, fp32 within 1e-5 * sum|x| of the fp64 oracle; two
calls in a row with the second input smaller, then a refused size, then one
more call. "Prefix sum and other parallel patterns", section "A device-level
scan: scan then propagate"."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import CODE, assert_fp32_close, assert_int_equal, from_dev, say, scan_tile, stream_handle, to_dev

pytestmark = pytest.mark.gpu


def _both(x: np.ndarray, inclusive: bool):
    """(noalloc output, allocating output) for x."""
    n = x.size
    xin = to_dev(x)
    a = torch.empty_like(xin)
    b = torch.empty_like(xin)
    a.view(torch.uint8).fill_(0xA5)
    b.view(torch.uint8).fill_(0x5A)
    h = stream_handle()
    st = ds.lib.ds_scan_noalloc(CODE[x.dtype], int(inclusive), xin.data_ptr(), a.data_ptr(), n, h)
    assert st == ds.DS_OK, ds.lib.ds_status_string(st)
    st = ds.lib.ds_scan(CODE[x.dtype], int(inclusive), ds.ALGO["lookback"], xin.data_ptr(), b.data_ptr(), n, h)
    assert st == ds.DS_OK, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    assert ds.query_timeout() is False
    return from_dev(a, x.dtype), from_dev(b, x.dtype)


def _check(x: np.ndarray, inclusive: bool, what: str):
    got, ref = _both(x, inclusive)
    if x.dtype == np.float32:
        y, s = oracle.scan(x, inclusive)
        r1 = assert_fp32_close(got, y, s, what + " (noalloc)")
        assert_fp32_close(ref, y, s, what + " (allocating)")
        say(f"{what}: fp32 max err/S {r1:.2e}")
    else:
        want = oracle.scan(x, inclusive)
        assert_int_equal(got, ref, what + ": noalloc vs allocating")
        assert_int_equal(got, want, what + ": noalloc vs oracle")


@pytest.mark.parametrize("inclusive", [False, True])
def test_noalloc_matches_allocating_entry_two_calls(inclusive):
    say(f"ds_scan_noalloc, inclusive={inclusive}")
    big = 100 * scan_tile(np.int32, inclusive, 3_000_000) + 17       # ragged, many tiles
    x1 = datagen.uniform_int(81, big, -1000, 1000)
    _check(x1, inclusive, f"int32 n={big}")
    small = 7 * scan_tile(np.int32, inclusive, 100_000) + 3           # second call: smaller input
    x2 = datagen.uniform_int(82, small, -1000, 1000)
    _check(x2, inclusive, f"int32 n={small}")


def test_noalloc_other_types_and_sizes():
    _check(datagen.normal_f32(83, 2_000_003), False, "fp32 n=2000003")
    _check(datagen.uniform_i64(84, 1_500_001, 40), True, "int64 n=1500001")
    _check(datagen.uniform_int(85, 4096, 0, 9), False, "int32 one tile")
    x = datagen.workload("int32_100m")
    _check(x, False, "int32 n=100000007")
    # a size beyond the fixed array is refused before any launch; the next call works
    xin = to_dev(datagen.uniform_int(86, 16, 0, 9))
    st = ds.lib.ds_scan_noalloc(0, 0, xin.data_ptr(), xin.data_ptr(), 1_200_000_000, stream_handle())
    assert st == ds.DS_ERR_TOO_LARGE
    _check(datagen.uniform_int(87, 333_333, 0, 100), True, "int32 n=333333 after a refused call")
