"""The look-back scan with the blocked tile layout (DS_ALGO_LOOKBACK_BLOCKED:
each tile transposed through padded LDS so that a thread scans contiguous
elements), against the oracle through the C ABI: bit-exact integers, fp32
within 1e-5 * sum|x|. Sizes around its two tiles (8 and 12 vectors per thread;
"Day 32 -- The CUDA scan algorithm", section "The stride doubles, and so does
the conflict"), the pages' worked examples, the workloads at their full sizes,
misaligned and in-place calls, and the refusal of 8-byte types."""
import numpy as np
import pytest
import torch

import datagen
import pins
import primitives_device_scan_amd as ds
from gpu_util import CODE, check_scan, gpu_scan, say, stream_handle, to_dev

pytestmark = pytest.mark.gpu
ALGO = "lookback_blocked"
SMALL_T = 256 * 8 * 4    # elements per tile up to 8 MiB of input
BIG_T = 256 * 12 * 4     # beyond


def _input(dt, n, seed):
    if np.dtype(dt) == np.float32:
        return datagen.normal_f32(seed, n)
    if np.dtype(dt) == np.uint32:
        return datagen.keys_u32(seed, n)
    return datagen.uniform_int(seed, n, -1000, 1000)


@pytest.mark.parametrize("dt", [np.int32, np.uint32, np.float32], ids=lambda d: np.dtype(d).name)
def test_worked_examples(dt):
    for ex in pins.parse_golden_examples():
        x = np.array(ex["input"], dtype=dt)
        for kind in ("inclusive", "exclusive"):
            if kind in ex:
                got = gpu_scan(x, kind == "inclusive", ALGO)
                assert [int(v) for v in got] == ex[kind], (ex["name"], kind, got)


@pytest.mark.parametrize("dt", [np.int32, np.uint32, np.float32], ids=lambda d: np.dtype(d).name)
def test_tile_boundaries(dt):
    small_max = (8 << 20) // 4
    k = small_max // BIG_T + 2
    sizes = [1, 2, 63, 64, 65, 1023, 1025, SMALL_T - 1, SMALL_T, SMALL_T + 1, 3 * SMALL_T + 7, 64 * SMALL_T + 5,
             small_max, small_max + 1, k * BIG_T - 1, k * BIG_T, k * BIG_T + 1]
    for n in sizes:
        x = _input(dt, n, 4000 + n % 991)
        for inc in (False, True):
            check_scan(x, inc, gpu_scan(x, inc, ALGO), f"blocked {np.dtype(dt).name} n={n} inc={inc}")


def test_workloads_full_size():
    for name, inc in (("one_tile", False), ("mid", False), ("mid", True), ("fp32_10m", True), ("int32_100m", False),
                      ("fp32_100m", False)):
        x = datagen.workload(name)
        say(f"blocked {name} inclusive={inc}")
        r = check_scan(x, inc, gpu_scan(x, inc, ALGO), f"blocked {name} inc={inc}")
        if x.dtype == np.float32:
            say(f"  fp32 max err/S {r:.2e}")


def test_misaligned_and_in_place():
    n = 5 * BIG_T + 777 + (8 << 20) // 4
    x = _input(np.int32, n, 4242)
    for inc in (False, True):
        check_scan(x, inc, gpu_scan(x, inc, ALGO, offset=1), f"blocked misaligned inc={inc}")
        check_scan(x, inc, gpu_scan(x, inc, ALGO, in_place=True), f"blocked in place inc={inc}")


def test_eight_byte_types_refused():
    x = to_dev(datagen.uniform_i64(5, 1000, 40))
    y = torch.empty_like(x)
    for dt in (np.int64, np.uint64):
        st = ds.lib.ds_scan(CODE[np.dtype(dt)], 0, ds.ALGO[ALGO], x.data_ptr(), y.data_ptr(), 1000, stream_handle())
        assert st == ds.DS_ERR_UNSUPPORTED_DTYPE
