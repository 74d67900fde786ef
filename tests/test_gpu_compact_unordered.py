"""Parity of ds_compact_unordered (through the C ABI) with the oracle. The
output order is unspecified, so what is unique is compared: the count, and
the kept elements as a multiset (both sides sorted by bit pattern), bit-exact;
the rest of the output buffer must be untouched."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import pins
import primitives_device_scan_amd as ds
from gpu_util import CODE, assert_int_equal, cached_workload, from_dev, say, sentinel_fill, stream_handle, tile_of, \
    to_dev

pytestmark = pytest.mark.gpu

CLAIMS = ("wave", "workgroup")


def gpu_compact_unordered(x: np.ndarray, op: str, operand, claim: str, offset: int = 0):
    n = x.size
    xin = to_dev(x, extra=offset, offset=offset)[offset:]
    out = torch.empty_like(xin)
    sentinel_fill(out)
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    bits = ds.operand_bits({np.dtype(np.int32): torch.int32, np.dtype(np.uint32): torch.int64,
                            np.dtype(np.float32): torch.float32, np.dtype(np.int64): torch.int64,
                            np.dtype(np.uint64): torch.int64}[x.dtype], operand)
    if x.dtype == np.uint32:
        bits &= 0xFFFFFFFF
    st = ds.lib.ds_compact_unordered(CODE[x.dtype], xin.data_ptr(), out.data_ptr(), cnt.data_ptr(), n,
                                     ds.CMP[op], bits, ds._binding.CLAIM[claim], stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    return from_dev(out, x.dtype, 0, n), int(cnt.item())


def bits_sorted(a: np.ndarray) -> np.ndarray:
    return np.sort(a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint64))


def check_multiset(got: np.ndarray, k: int, want: np.ndarray, what: str):
    assert k == want.size, (what, k, want.size)
    assert_int_equal(bits_sorted(got[:k]), bits_sorted(want), what + " (sorted bit patterns)")
    rest = got[k:].view(np.uint8)
    assert np.all(rest == 0xA5), what + ": written past the count"


@pytest.mark.parametrize("claim", CLAIMS)
def test_unordered_256m_keys_below_2_31(claim):
    x = cached_workload("compact_256m")
    say("compact_256m uint32 unordered keep key < 2^31, claim per", claim)
    got, k = gpu_compact_unordered(x, "<", 1 << 31, claim)
    want = oracle.compact(x, "<", 1 << 31)
    check_multiset(got, k, want, f"compact_256m claim per {claim}")


@pytest.mark.parametrize("claim", CLAIMS)
@pytest.mark.parametrize("case", range(len(pins.COMPACT_CASES)))
def test_unordered_dtypes_ops(case, claim):
    dt, gen, operands = pins.COMPACT_CASES[case]
    T = tile_of(dt, compact=True)
    for n in (1, 7, 64, T - 1, T, T + 1, 3 * T + 5, 40 * T + 3):
        x = gen(700 + n, n).astype(dt)
        for c in operands:
            for op in ("<", ">=", "==", "!="):
                got, k = gpu_compact_unordered(x, op, c, claim)
                check_multiset(got, k, oracle.compact(x, op, c), f"{np.dtype(dt).name} n={n} {op} {c} {claim}")


@pytest.mark.parametrize("claim", CLAIMS)
def test_unordered_edges(claim):
    x = np.array([1.0, np.nan, -2.0, np.nan, 0.0], dtype=np.float32)
    got, k = gpu_compact_unordered(x, "<", 5.0, claim)
    assert k == 3 and sorted(got[:3].tolist()) == [-2.0, 0.0, 1.0]
    got, k = gpu_compact_unordered(x, "!=", 0.0, claim)
    assert k == 4
    got, k = gpu_compact_unordered(x, "==", float("nan"), claim)
    assert k == 0
    got, k = gpu_compact_unordered(np.zeros(0, dtype=np.int32), ">", 0, claim)
    assert k == 0
    got, k = gpu_compact_unordered(np.array([5], dtype=np.int32), ">", 0, claim)
    assert k == 1 and got[0] == 5
    n = 9 * tile_of(np.int32, compact=True) + 1
    x = datagen.uniform_int(8, n, 0, 9)
    got, k = gpu_compact_unordered(x, ">=", 0, claim)
    check_multiset(got, k, x, "all kept")
    got, k = gpu_compact_unordered(x, ">", 9, claim)
    assert k == 0


def test_unordered_count_reused_across_calls():
    # The counter is the claim target: a second call on the same buffer must start from zero.
    x = datagen.keys_u32(41, 5 * tile_of(np.uint32, compact=True) + 9)
    xin = to_dev(x)
    out = torch.empty_like(xin)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    want = oracle.compact(x, ">", 1 << 30)
    for claim in (0, 1, 0):
        st = ds.lib.ds_compact_unordered(CODE[x.dtype], xin.data_ptr(), out.data_ptr(), cnt.data_ptr(), x.size,
                                         ds.CMP[">"], 1 << 30, claim, stream_handle())
        assert st == 0
        torch.cuda.synchronize()
        assert int(cnt.item()) == want.size


def test_unordered_binding():
    x = torch.from_numpy(datagen.uniform_int(3, 100003, -50, 50)).cuda()
    out, cnt = ds.compact_unordered(x, "<", 0, claim="wave")
    torch.cuda.synchronize()
    want = oracle.compact(x.cpu().numpy(), "<", 0)
    k = int(cnt.item())
    assert k == want.size
    assert_int_equal(np.sort(out[:k].cpu().numpy()), np.sort(want), "binding")


@pytest.mark.parametrize("claim", CLAIMS)
def test_unordered_misaligned(claim):
    T = tile_of(np.uint32, compact=True)
    n = 7 * T + 13
    x = datagen.keys_u32(55, n)
    got, k = gpu_compact_unordered(x, "<", 1 << 30, claim, offset=1)
    check_multiset(got, k, oracle.compact(x, "<", 1 << 30), f"misaligned claim per {claim}")
