"""Helpers of the GPU parity tests: move numpy inputs to the GPU, call the C
ABI of libdevscan.so with an explicit ds_dtype code, bring results back, and
compare them with the oracle element by element."""
from __future__ import annotations

import ctypes
import functools
import sys

import numpy as np
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds

CODE = {np.dtype(np.int32): 0, np.dtype(np.uint32): 1, np.dtype(np.float32): 2,
        np.dtype(np.int64): 3, np.dtype(np.uint64): 4}
STORAGE = {np.dtype(np.int32): (np.int32, torch.int32), np.dtype(np.uint32): (np.int32, torch.int32),
           np.dtype(np.float32): (np.float32, torch.float32), np.dtype(np.int64): (np.int64, torch.int64),
           np.dtype(np.uint64): (np.int64, torch.int64)}
FP32_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, extra: int = 0, offset: int = 0) -> torch.Tensor:
    """x on the GPU in a buffer of x.size + extra elements, starting at `offset` elements."""
    snp, st = STORAGE[x.dtype]
    t = torch.zeros(x.size + extra, dtype=st, device="cuda")
    if x.size:
        t[offset:offset + x.size].copy_(torch.from_numpy(np.ascontiguousarray(x).view(snp)))
    return t


def from_dev(t: torch.Tensor, dtype, start: int = 0, count: int | None = None) -> np.ndarray:
    count = t.numel() - start if count is None else count
    return t[start:start + count].cpu().numpy().view(dtype)


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def sentinel_fill(t: torch.Tensor):
    """Fill an output buffer with a recognisable pattern so unwritten elements show."""
    t.view(torch.uint8).fill_(0xA5)


def gpu_scan(x: np.ndarray, inclusive: bool, algo: str = "default", in_place: bool = False, offset: int = 0,
             entry: str = "ds_scan") -> np.ndarray:
    """Scan x through the C ABI; offset > 0 shifts both buffers off 16-byte alignment."""
    n = x.size
    xin = to_dev(x, extra=offset, offset=offset)
    if in_place:
        out = xin
    else:
        out = torch.empty_like(xin)
        sentinel_fill(out)
    esz = x.dtype.itemsize
    pin = xin.data_ptr() + offset * esz
    pout = out.data_ptr() + offset * esz
    if entry == "ds_scan":
        st = ds.lib.ds_scan(CODE[x.dtype], int(inclusive), ds.ALGO[algo], pin, pout, n, stream_handle())
    else:
        f = ds.lib.scan_inclusive if inclusive else ds.lib.scan_exclusive
        st = f(CODE[x.dtype], pin, pout, n, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    assert ds.query_timeout() is False, "a look-back wait gave up: the output is not valid"
    return from_dev(out, x.dtype, offset, n)


def gpu_compact(x: np.ndarray, op: str, operand, in_place: bool = False, offset: int = 0):
    """compact_if through the C ABI; offset > 0 moves input and output off 16-byte alignment."""
    n = x.size
    xin = to_dev(x, extra=offset, offset=offset)
    out = xin if in_place else torch.empty_like(xin)
    if not in_place:
        sentinel_fill(out)
    esz = x.dtype.itemsize
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    bits = ds.operand_bits({np.dtype(np.int32): torch.int32, np.dtype(np.uint32): torch.int64,
                            np.dtype(np.float32): torch.float32, np.dtype(np.int64): torch.int64,
                            np.dtype(np.uint64): torch.int64}[x.dtype], operand)
    if x.dtype == np.uint32:
        bits &= 0xFFFFFFFF
    st = ds.lib.compact_if(CODE[x.dtype], xin.data_ptr() + offset * esz, out.data_ptr() + offset * esz,
                           cnt.data_ptr(), n, ds.CMP[op], bits, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    assert ds.query_timeout() is False, "a look-back wait gave up: the output is not valid"
    k = int(cnt.item())
    return from_dev(out, x.dtype, offset, n), k


def tile_of(dtype, compact: bool = False, entry: str | None = None) -> int:
    """Elements per workgroup tile, as the library reports it (ds_tile_elems);
    by default the smaller of the exclusive and inclusive scan tiles."""
    if entry is None and not compact:
        return min(tile_of(dtype, entry="scan_exclusive"), tile_of(dtype, entry="scan_inclusive"))
    entry = entry or "compact"
    return int(ds.lib.ds_tile_elems(CODE[np.dtype(dtype)], ds._binding.TILE_OF[entry]))


def scan_tile(dtype, inclusive: bool, n: int) -> int:
    """Elements per look-back tile for an input of n elements (ds_scan_tile_elems)."""
    return int(ds.lib.ds_scan_tile_elems(CODE[np.dtype(dtype)], int(inclusive), n))


def assert_int_equal(got: np.ndarray, want: np.ndarray, what: str):
    if got.shape == want.shape and np.array_equal(got, want):
        return
    bad = np.nonzero(got != want)[0] if got.shape == want.shape else np.array([0])
    i = int(bad[0])
    T = tile_of(want.dtype)
    raise AssertionError(f"{what}: {bad.size} mismatches of {want.size}; first at {i} "
                         f"(tile {i // T}, position {i % T}): got {got[i]} want {want[i]}")


def assert_fp32_close(got: np.ndarray, y: np.ndarray, s_abs: np.ndarray, what: str, tol: float = FP32_TOL):
    """|got_i - y_i| <= tol * S_i (and got_i == 0 where S_i == 0). Returns the max err/S ratio."""
    err = np.abs(got.astype(np.float64) - y)
    zero = s_abs == 0
    if np.any(zero) and np.any(got[zero] != 0):
        i = int(np.nonzero(zero & (got != 0))[0][0])
        raise AssertionError(f"{what}: element {i} should be exactly 0, got {got[i]}")
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, s_abs))
    if not np.all(np.isfinite(got)) or np.any(ratio > tol):
        bad = np.nonzero(~np.isfinite(got) | (ratio > tol))[0]
        i = int(bad[0])
        T = tile_of(np.float32)
        raise AssertionError(f"{what}: {bad.size} elements outside {tol}*S; first at {i} (tile {i // T}, "
                             f"position {i % T}): got {got[i]} want {y[i]} S {s_abs[i]}")
    return float(ratio.max()) if ratio.size else 0.0


def check_scan(x: np.ndarray, inclusive: bool, got: np.ndarray, what: str):
    if x.dtype == np.float32:
        y, s = oracle.scan(x, inclusive)
        return assert_fp32_close(got, y, s, what)
    assert_int_equal(got, oracle.scan(x, inclusive), what)
    return 0.0


@functools.lru_cache(maxsize=4)
def cached_workload(name: str) -> np.ndarray:
    x = datagen.workload(name)
    x.setflags(write=False)
    return x
