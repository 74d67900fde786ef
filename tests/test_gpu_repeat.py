"""Many launches of the multi-tile kernels on one input, every result compared
on the device with the first (itself checked against the oracle).

Integer results are unique, so any launch whose look-back took a wrong
prefix -- a status word read before it was written, a stale epoch accepted,
a lost update -- would differ. Runs a few hundred launches in well under a
second of GPU time.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import assert_int_equal, cached_workload, from_dev, say, stream_handle, to_dev

pytestmark = pytest.mark.gpu


def test_scan_100m_int32_repeated():
    x = datagen.workload("int32_100m")
    n = x.size
    say("repeat: 200 launches, int32 exclusive scan, n =", n)
    dx = to_dev(x)
    first, y = torch.empty_like(dx), torch.empty_like(dx)
    sh = stream_handle()
    assert ds.lib.scan_exclusive(0, dx.data_ptr(), first.data_ptr(), n, sh) == 0
    torch.cuda.synchronize()
    assert_int_equal(from_dev(first, np.int32), oracle.scan(x, False), "first launch")
    bad = []
    for i in range(200):
        assert ds.lib.scan_exclusive(0, dx.data_ptr(), y.data_ptr(), n, sh) == 0
        if not torch.equal(y, first):
            bad.append(i)
    torch.cuda.synchronize()
    assert not bad, f"launches {bad[:10]} differ from the first"
    assert not ds.query_timeout()


@pytest.mark.parametrize("inclusive", [False, True])
def test_scan_int64_and_mid_sizes_repeated(inclusive):
    # several tile regimes, 8-byte status words
    sh = stream_handle()
    for n, dt in ((1_048_576, np.int32), (30_000_001, np.int32), (10_000_019, np.int64)):
        x = datagen.uniform_int(77, n, -1000, 1000) if dt == np.int32 else datagen.uniform_i64(78, n, 62)
        code = 0 if dt == np.int32 else 3
        dx = to_dev(x)
        first, y = torch.empty_like(dx), torch.empty_like(dx)
        assert ds.lib.ds_scan(code, int(inclusive), 0, dx.data_ptr(), first.data_ptr(), n, sh) == 0
        torch.cuda.synchronize()
        assert_int_equal(from_dev(first, dt), oracle.scan(x, inclusive), f"n={n} first launch")
        for i in range(100):
            assert ds.lib.ds_scan(code, int(inclusive), 0, dx.data_ptr(), y.data_ptr(), n, sh) == 0
            assert torch.equal(y, first), f"n={n} launch {i} differs"
    assert not ds.query_timeout()


def test_compaction_and_radix_pass_repeated():
    keys = cached_workload("compact_256m")
    n = keys.size
    say("repeat: compact_if x 30 and radix pass x 10 over", n, "keys")
    sh = stream_handle()
    dk = to_dev(keys)
    out, cnt = torch.empty_like(dk), torch.empty(1, dtype=torch.int64, device="cuda")
    assert ds.lib.compact_if(1, dk.data_ptr(), out.data_ptr(), cnt.data_ptr(), n, 0, 1 << 31, sh) == 0
    torch.cuda.synchronize()
    k = int(cnt.item())
    first = out[:k].clone()
    want = oracle.compact(keys, "<", 1 << 31)
    assert k == want.size
    assert_int_equal(from_dev(first, np.uint32), want, "compact_if first launch")
    for i in range(30):
        assert ds.lib.compact_if(1, dk.data_ptr(), out.data_ptr(), cnt.data_ptr(), n, 0, 1 << 31, sh) == 0
        assert int(cnt.item()) == k and torch.equal(out[:k], first), f"compact_if launch {i} differs"
    del out, first
    ko = torch.empty_like(dk)
    assert ds.lib.ds_radix_pass(dk.data_ptr(), ko.data_ptr(), None, None, n, 8, 8, sh) == 0
    torch.cuda.synchronize()
    rfirst = ko.clone()
    wk, _ = oracle.radix_pass(keys, 8, 8)
    assert_int_equal(from_dev(rfirst, np.uint32), wk, "radix pass first launch")
    for i in range(10):
        assert ds.lib.ds_radix_pass(dk.data_ptr(), ko.data_ptr(), None, None, n, 8, 8, sh) == 0
        assert torch.equal(ko, rfirst), f"radix pass launch {i} differs"
    assert not ds.query_timeout()
