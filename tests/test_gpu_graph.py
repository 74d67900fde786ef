"""Scans captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every replay, with the program's own eager work and synchronisations between
the replays, must equal the eager result bit for bit. The look-back's launch
epoch lives in device memory and the last tile of each launch advances it, so
replayed launches retire the previous launch's status words exactly as eager
ones do. The captured calls find their workspace already allocated (a
warm-up call on the capture stream), so nothing but kernel launches is
recorded.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import assert_int_equal, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

CALLS_PER_GRAPH = 3
REPLAYS = 5


@pytest.mark.parametrize("inclusive", [False, True])
@pytest.mark.parametrize("n", [4096, 1_048_576, 10_000_019])
def test_scan_graph_replays(n, inclusive):
    say("graph: int32 scan, n =", n, "inclusive =", inclusive)
    fn = ds.lib.scan_inclusive if inclusive else ds.lib.scan_exclusive
    x = datagen.uniform_int(300 + n % 97, n, -1000, 1000)
    want = oracle.scan(x, inclusive)
    other = datagen.uniform_int(7, 3 * n + 5, 0, 9)
    other_want = oracle.scan(other, inclusive)
    dx, dy = to_dev(x), to_dev(np.zeros(n, dtype=np.int32))
    ox, oy = to_dev(other), to_dev(np.zeros(other.size, dtype=np.int32))

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        assert fn(ds.DS_INT32, dx.data_ptr(), dy.data_ptr(), n, cap.cuda_stream) == 0  # allocates the workspace
    cap.synchronize()
    assert_int_equal(from_dev(dy, np.int32), want, "eager on the capture stream")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for _ in range(CALLS_PER_GRAPH):
            st = fn(ds.DS_INT32, dx.data_ptr(), dy.data_ptr(), n, cap.cuda_stream)
            assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()

    main = torch.cuda.current_stream().cuda_stream
    for r in range(REPLAYS):
        dy.fill_(0)
        # eager work between replays: another scan, on this thread's stream
        assert fn(ds.DS_INT32, ox.data_ptr(), oy.data_ptr(), other.size, main) == 0
        torch.cuda.synchronize()
        assert_int_equal(from_dev(oy, np.int32), other_want, f"eager scan before replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert_int_equal(from_dev(dy, np.int32), want, f"replay {r}")
    timed_out = ds.query_timeout(stream=cap)
    assert not timed_out, "a look-back wait gave up during the replays"
    del g


@pytest.mark.parametrize("name", ["moe_decode", "moe_64k"])
def test_moe_align_graph_replays(name):
    # one-launch (256 x 8 ids) and three-launch (65,536 x 8) alignment replayed from a graph
    t, k, e, block, _, _ = datagen.MOE_WORKLOADS[name]
    say("graph: MoE alignment", name)
    ids = datagen.moe_workload(name).ravel()
    wc, wo, ws = oracle.moe_align(ids, e, block)
    n = ids.size
    cap_n = n + e * (block - 1)
    d_ids = to_dev(ids)
    counts = torch.empty(e, dtype=torch.int32, device="cuda")
    offsets = torch.empty(e + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(cap_n, dtype=torch.int32, device="cuda")

    def call(stream):
        return ds.lib.ds_moe_align(d_ids.data_ptr(), n, e, block, counts.data_ptr(), offsets.data_ptr(),
                                   srt.data_ptr(), cap_n, stream)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        assert call(cap.cuda_stream) == 0  # allocates the table and workspace
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for _ in range(CALLS_PER_GRAPH):
            assert call(cap.cuda_stream) == 0
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t_ in (counts, offsets, srt):
            t_.fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        total = int(wo[-1])
        assert_int_equal(counts.cpu().numpy(), wc, f"replay {r} counts")
        assert_int_equal(offsets.cpu().numpy(), wo, f"replay {r} offsets")
        assert_int_equal(srt.cpu().numpy()[:total], ws, f"replay {r} sorted ids")
    assert not ds.query_timeout(stream=cap)
    del g
