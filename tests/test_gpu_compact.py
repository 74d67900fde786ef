"""Parity of compact_if (through the C ABI) with the oracle: the count and
the kept elements in order, bit-exact."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import pins
from gpu_util import assert_int_equal, cached_workload, gpu_compact, say, tile_of

pytestmark = pytest.mark.gpu


def test_compact_256m_keys_below_2_31():
    x = cached_workload("compact_256m")
    say("compact_256m uint32 keep key < 2^31")
    out, k = gpu_compact(x, "<", 1 << 31)
    want = oracle.compact(x, "<", 1 << 31)
    assert k == want.size, (k, want.size)
    assert_int_equal(out[:k], want, "compact_256m kept keys")
    flags = (x < np.uint32(1 << 31)).astype(np.uint32)
    pos = oracle.scan(flags, False)
    assert k == int(pos[-1]) + int(flags[-1])


@pytest.mark.parametrize("case", range(len(pins.COMPACT_CASES)))
def test_compact_dtypes_ops(case):
    dt, gen, operands = pins.COMPACT_CASES[case]
    T = tile_of(dt, compact=True)
    for n in (1, 7, 64, T - 1, T, T + 1, 3 * T + 5, 70 * T + 3):
        x = gen(500 + n, n).astype(dt)
        for c in operands:
            for op in ("<", "<=", ">", ">=", "==", "!="):
                out, k = gpu_compact(x, op, c)
                want = oracle.compact(x, op, c)
                assert k == want.size, (np.dtype(dt).name, n, op, c, k, want.size)
                assert_int_equal(out[:k].view(want.dtype), want, f"{np.dtype(dt).name} n={n} {op} {c}")


def test_compact_nan_and_edges():
    x = np.array([1.0, np.nan, -2.0, np.nan, 0.0], dtype=np.float32)
    out, k = gpu_compact(x, "<", 5.0)
    assert k == 3 and out[:3].tolist() == [1.0, -2.0, 0.0]
    out, k = gpu_compact(x, "!=", 0.0)
    assert k == 4
    out, k = gpu_compact(x, "==", float("nan"))
    assert k == 0
    out, k = gpu_compact(np.zeros(0, dtype=np.int32), ">", 0)
    assert k == 0
    out, k = gpu_compact(np.array([5], dtype=np.int32), ">", 0)
    assert k == 1 and out[0] == 5


def test_compact_in_place():
    n = 40 * tile_of(np.uint32, compact=True) + 17
    x = datagen.keys_u32(31, n)
    out, k = gpu_compact(x, ">=", 3 << 30, in_place=True)
    want = oracle.compact(x, ">=", 3 << 30)
    assert k == want.size
    assert_int_equal(out[:k], want, "in place")


def test_compact_all_and_none():
    n = 9 * tile_of(np.int32, compact=True) + 1
    x = datagen.uniform_int(8, n, 0, 9)
    out, k = gpu_compact(x, ">=", 0)
    assert k == n and np.array_equal(out[:k], x)
    out, k = gpu_compact(x, ">", 9)
    assert k == 0


@pytest.mark.parametrize("dt", [np.uint32, np.float32, np.int64])
def test_compact_misaligned(dt):
    # input and output one element off 16-byte alignment
    T = tile_of(dt, compact=True)
    case = [c for c in pins.COMPACT_CASES if c[0] == dt][0]
    for n in (T - 1, 5 * T + 3):
        x = case[1](910 + n, n).astype(dt)
        c = case[2][1]
        out, k = gpu_compact(x, ">", c, offset=1)
        want = oracle.compact(x, ">", c)
        assert k == want.size
        assert_int_equal(out[:k].view(want.dtype), want, f"{np.dtype(dt).name} n={n} misaligned")


@pytest.mark.parametrize("dt", [np.uint32, np.int64])
def test_compact_misaligned_phases(dt):
    # input and output at different offsets from 16-byte alignment; the output
    # buffer keeps its sentinel below the output and past the kept elements
    import primitives_device_scan_amd as ds
    from gpu_util import CODE, STORAGE, sentinel_fill, stream_handle, to_dev
    T = tile_of(dt, compact=True)
    case = [c for c in pins.COMPACT_CASES if c[0] == dt][0]
    n = 6 * T + 7
    x = case[1](4321, n).astype(dt)
    c = case[2][1]
    want = oracle.compact(x, ">", c)
    esz = np.dtype(dt).itemsize
    per_vec = 16 // esz
    bits = ds.operand_bits(torch.int64, c)
    if dt == np.uint32:
        bits &= 0xFFFFFFFF
    for in_off, out_off in [(a, b) for a in range(per_vec) for b in range(per_vec) if a != b]:
        xin = to_dev(x, extra=in_off + 5, offset=in_off)
        out = torch.empty(n + out_off + 5, dtype=STORAGE[np.dtype(dt)][1], device="cuda")
        sentinel_fill(out)
        cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
        st = ds.lib.compact_if(CODE[np.dtype(dt)], xin.data_ptr() + in_off * esz, out.data_ptr() + out_off * esz,
                               cnt.data_ptr(), n, ds.CMP[">"], bits, stream_handle())
        assert st == 0, ds.lib.ds_status_string(st)
        torch.cuda.synchronize()
        k = int(cnt.item())
        assert k == want.size, (in_off, out_off)
        raw = out.view(torch.uint8).cpu().numpy()
        got = raw[out_off * esz:(out_off + k) * esz].view(want.dtype)
        assert_int_equal(got, want, f"in +{in_off} out +{out_off}")
        assert np.all(raw[:out_off * esz] == 0xA5), "written below the output"
        assert np.all(raw[(out_off + k) * esz:] == 0xA5), "written past the kept elements"
