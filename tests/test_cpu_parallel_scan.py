"""The threaded CPU comparison scan (oracle/parallel_scan.c) against the oracle.

CPU only. Integer results must be bit-identical to the oracle's (both wrap
modulo 2^32); fp32 results must lie within the fp32 tolerance of the oracle's
fp64 prefix, |y_i - ref_i| <= 1e-5 * S_i.
"""
import numpy as np
import pytest

import datagen
import oracle


@pytest.fixture(scope="module")
def par():
    oracle.build()
    return oracle.ParallelScan()


SIZES = [0, 1, 2, 7, 1000, 100_003]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("threads", [1, 3, 8, 300])
@pytest.mark.parametrize("inclusive", [False, True])
def test_int32_bit_exact(par, n, threads, inclusive):
    x = datagen.uniform_int(11, n, -1000, 1000)
    want = oracle.scan(x, inclusive)
    got = par.scan(x, inclusive, threads)
    assert got.dtype == np.int32 and np.array_equal(got, want)


@pytest.mark.parametrize("inclusive", [False, True])
def test_int32_wraps_like_the_oracle(par, inclusive):
    x = np.full(10_000, 1 << 30, dtype=np.int32)
    got = par.scan(x, inclusive, 8)
    assert np.array_equal(got, oracle.scan(x, inclusive))
    # closed form: the k-th prefix is k * 2^30 modulo 2^32
    k = np.arange(x.size, dtype=np.uint64) + (1 if inclusive else 0)
    assert np.array_equal(got.view(np.uint32), ((k << np.uint64(30)) & np.uint64(0xFFFFFFFF)).astype(np.uint32))


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("threads", [1, 5, 16])
@pytest.mark.parametrize("inclusive", [False, True])
def test_fp32_within_tolerance(par, n, threads, inclusive):
    x = datagen.normal_f32(12, n)
    ref, s = oracle.scan(x, inclusive)
    got = par.scan(x, inclusive, threads)
    assert got.dtype == np.float32
    assert np.all(np.abs(got.astype(np.float64) - ref) <= 1e-5 * s)


def test_in_place(par):
    x = datagen.uniform_int(13, 50_001, 0, 9)
    want = oracle.scan(x, False)
    par.scan(x, False, 7, out=x)
    assert np.array_equal(x, want)


def test_host_threads_is_capped():
    assert 1 <= oracle.host_threads() <= 16
