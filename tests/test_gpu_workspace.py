"""Workspace edge paths through the C ABI: a refused workspace allocation
comes back as DS_ERR_OUT_OF_MEMORY with nothing launched, and the next call
on the same stream allocates and is correct; a capture that would have to
allocate is refused with DS_ERR_STREAM_CAPTURING, and after one eager call
the same capture records and replays correctly. (The testing hook is
ds_fail_next_allocations; the pages ask for every call to be checked and for
the workspace to be cached: "Parallel Prefix Sum (Scan) for NVIDIA T4
(sm_75)", sections "Key Features" and "Optimisation Journey".)"""
import numpy as np
import pytest
import torch

import datagen
import primitives_device_scan_amd as ds
from gpu_util import check_scan, say, tile_of, to_dev

pytestmark = pytest.mark.gpu


def test_refused_allocation_then_success():
    n = 40 * tile_of(np.int32) + 3
    x = datagen.uniform_int(71, n, -1000, 1000)
    xin = to_dev(x)
    out = torch.full_like(xin, 0x5A5A5A5A)
    s = torch.cuda.Stream()  # a stream with no workspace yet
    ds.lib.ds_fail_next_allocations(1)
    try:
        st = ds.lib.scan_exclusive(0, xin.data_ptr(), out.data_ptr(), n, s.cuda_stream)
        say(f"refused allocation: status {st}")
        assert st == ds.DS_ERR_OUT_OF_MEMORY, ds.lib.ds_status_string(st)
        s.synchronize()
        assert torch.all(out == 0x5A5A5A5A)  # nothing was launched
        cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
        ds.lib.ds_fail_next_allocations(1)
        st = ds.lib.compact_if(0, xin.data_ptr(), out.data_ptr(), cnt.data_ptr(), n, ds.CMP["<"], 0, s.cuda_stream)
        assert st == ds.DS_ERR_OUT_OF_MEMORY
    finally:
        ds.lib.ds_fail_next_allocations(0)
    st = ds.lib.scan_exclusive(0, xin.data_ptr(), out.data_ptr(), n, s.cuda_stream)
    assert st == ds.DS_OK, ds.lib.ds_status_string(st)
    s.synchronize()
    check_scan(x, False, out.cpu().numpy(), "after a refused allocation")
    assert ds.query_timeout(stream=s) is False


def test_capture_that_would_allocate_is_refused():
    n = 12 * tile_of(np.int32) + 5
    x = datagen.uniform_int(72, n, 0, 100)
    xin = to_dev(x)
    out = torch.empty_like(xin)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        st = ds.lib.scan_exclusive(0, xin.data_ptr(), out.data_ptr(), n, cap.cuda_stream)
    say(f"capture before any eager call: status {st}")
    assert st == ds.DS_ERR_STREAM_CAPTURING, ds.lib.ds_status_string(st)
    del g
    # one eager call sizes the workspace; the capture then records the kernel only
    with torch.cuda.stream(cap):
        assert ds.lib.scan_exclusive(0, xin.data_ptr(), out.data_ptr(), n, cap.cuda_stream) == ds.DS_OK
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        st = ds.lib.scan_exclusive(0, xin.data_ptr(), out.data_ptr(), n, cap.cuda_stream)
    assert st == ds.DS_OK
    for r in range(3):
        out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        check_scan(x, False, out.cpu().numpy(), f"replay {r}")
    assert ds.query_timeout(stream=cap) is False
