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
