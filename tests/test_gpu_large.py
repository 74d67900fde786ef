"""The scans and compact_if past 2^31 elements, where every element index
and tile offset needs 64 bits. Inputs are made on the device with closed-form
results (all ones: y_i = i or i + 1 mod 2^32; the keys 0, 1, 2, ...: the
kept prefix is 0 .. k-1), checked in full, chunk by chunk, on the device."""
import pytest
import torch

import primitives_device_scan_amd as ds
from gpu_util import say, stream_handle

pytestmark = pytest.mark.gpu

N = (1 << 31) + 24_579  # past 2^31, ragged last tile
CHUNK = 1 << 28


def expect_iota(y: torch.Tensor, n: int, first: int, what: str):
    """y[i] == (first + i) mod 2^32 for every i < n, as int32 bits."""
    for start in range(0, n, CHUNK):
        end = min(n, start + CHUNK)
        want = (torch.arange(start, end, dtype=torch.int64, device=y.device) + first).to(torch.int32)
        if not torch.equal(y[start:end], want):
            bad = torch.nonzero(y[start:end] != want)[0].item() + start
            raise AssertionError(f"{what}: first mismatch at {bad}: got {int(y[bad])}, want {int(want[bad - start])}")


@pytest.mark.parametrize("algo", ["lookback", "three_pass"])
def test_scan_beyond_2_31_elements(algo):
    say(f"int32 scans of {N} ones, {algo}")
    x = torch.ones(N, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    for inc in (0, 1):
        st = ds.lib.ds_scan(ds.DS_INT32, inc, ds.ALGO[algo], x.data_ptr(), y.data_ptr(), N, stream_handle())
        assert st == 0, ds.lib.ds_status_string(st)
        torch.cuda.synchronize()
        expect_iota(y, N, inc, f"{algo} inclusive={inc}")
    assert not ds.query_timeout()


def test_compact_beyond_2_31_elements():
    say(f"compact_if of {N} keys 0, 1, 2, ... keeping key < 2^31 + 5")
    x = torch.empty(N, dtype=torch.int32, device="cuda")
    for start in range(0, N, CHUNK):
        end = min(N, start + CHUNK)
        x[start:end] = torch.arange(start, end, dtype=torch.int64, device="cuda").to(torch.int32)
    out = torch.empty_like(x)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    keep = (1 << 31) + 5
    st = ds.lib.compact_if(ds.DS_UINT32, x.data_ptr(), out.data_ptr(), cnt.data_ptr(), N, ds.CMP["<"], keep,
                           stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    assert int(cnt.item()) == keep
    expect_iota(out, keep, 0, "compact_if kept keys")


def test_radix_pass_beyond_2_31_keys():
    # keys 0, 1, 2, ... ordered by their low byte: digit d holds d, d + 256, d + 512, ... in that order
    say(f"radix pass of {N} keys 0, 1, 2, ... by the low byte, with values")
    x = torch.empty(N, dtype=torch.int32, device="cuda")
    for start in range(0, N, CHUNK):
        end = min(N, start + CHUNK)
        x[start:end] = torch.arange(start, end, dtype=torch.int64, device="cuda").to(torch.int32)
    ko, vo = torch.empty_like(x), torch.empty_like(x)
    st = ds.lib.ds_radix_pass(x.data_ptr(), ko.data_ptr(), x.data_ptr(), vo.data_ptr(), N, 0, 8, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    del x
    q, r = N // 256, N % 256  # digits below r occur q + 1 times, the others q times
    for start in range(0, N, CHUNK):
        end = min(N, start + CHUNK)
        p = torch.arange(start, end, dtype=torch.int64, device="cuda")
        head = p < r * (q + 1)
        d = torch.where(head, p // (q + 1), r + (p - r * (q + 1)) // q)
        m = torch.where(head, p % (q + 1), (p - r * (q + 1)) % q)
        want = (d + 256 * m).to(torch.int32)
        assert torch.equal(ko[start:end], want), f"keys differ in [{start}, {end})"
        assert torch.equal(vo[start:end], want), f"values differ in [{start}, {end})"
