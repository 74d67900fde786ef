"""Sequential CPU oracle for device-wide prefix sums, stream compaction, the
counting-sort pass of a radix sort and MoE alignment.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library. The arithmetic
lives in ``oracle.c`` (plain C, one loop per function); this module only
compiles it with gcc, loads it and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
PAR_SRC = os.path.join(HERE, "parallel_scan.c")
PAR_LIB = os.path.join(HERE, "libparallel_scan.so")

OPS = {"<": 0, "<=": 1, ">": 2, ">=": 3, "==": 4, "!=": 5}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction); with the
    default paths, also the threaded CPU comparison scan."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-o", tmp, src], check=True)
    os.replace(tmp, out)
    if src == SRC and out == LIB:
        tmp = PAR_LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                        "-fno-fast-math", "-o", tmp, PAR_SRC], check=True)
        os.replace(tmp, PAR_LIB)
    return out


class Oracle:
    """numpy front end for one compiled copy of oracle.c."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path) if path == LIB else None
        self.lib = ctypes.CDLL(path)
        L = self.lib
        for name in ("oracle_scan_u32", "oracle_scan_u64"):
            getattr(L, name).argtypes = [_P, _P, _I64, ctypes.c_int]
            getattr(L, name).restype = None
        L.oracle_scan_f32.argtypes = [_P, _P, _P, _I64, ctypes.c_int]
        L.oracle_scan_f32.restype = None
        for name, ct in (("u32", ctypes.c_uint32), ("i32", ctypes.c_int32), ("f32", ctypes.c_float),
                         ("i64", ctypes.c_int64), ("u64", ctypes.c_uint64)):
            f = getattr(L, "oracle_compact_" + name)
            f.argtypes = [_P, _P, _I64, ctypes.c_int, ct]
            f.restype = ctypes.c_int64
        if hasattr(L, "oracle_radix_pass_u32"):
            L.oracle_radix_pass_u32.argtypes = [_P, _P, _P, _P, _I64, ctypes.c_int, ctypes.c_int]
            L.oracle_radix_pass_u32.restype = None
        if hasattr(L, "oracle_moe_align"):
            L.oracle_moe_align.argtypes = [_P, _I64, ctypes.c_int, ctypes.c_int, _P, _P, _P, _I64]
            L.oracle_moe_align.restype = ctypes.c_int64

    def scan(self, x: np.ndarray, inclusive: bool):
        """Integer input: the scan in x's dtype (wrapping). fp32 input: (y, s_abs) in fp64."""
        x = np.ascontiguousarray(x)
        n = x.size
        if x.dtype in (np.int32, np.uint32):
            y = np.empty_like(x)
            self.lib.oracle_scan_u32(x.ctypes.data, y.ctypes.data, n, int(inclusive))
            return y
        if x.dtype in (np.int64, np.uint64):
            y = np.empty_like(x)
            self.lib.oracle_scan_u64(x.ctypes.data, y.ctypes.data, n, int(inclusive))
            return y
        if x.dtype == np.float32:
            y = np.empty(n, dtype=np.float64)
            s = np.empty(n, dtype=np.float64)
            self.lib.oracle_scan_f32(x.ctypes.data, y.ctypes.data, s.ctypes.data, n, int(inclusive))
            return y, s
        raise TypeError(f"unsupported dtype {x.dtype}")

    def compact(self, x: np.ndarray, op: str, operand) -> np.ndarray:
        """The in-order subsequence of x whose elements satisfy (x_i op operand)."""
        x = np.ascontiguousarray(x)
        out = np.empty_like(x)
        names = {np.dtype(np.uint32): "u32", np.dtype(np.int32): "i32", np.dtype(np.float32): "f32",
                 np.dtype(np.int64): "i64", np.dtype(np.uint64): "u64"}
        f = getattr(self.lib, "oracle_compact_" + names[x.dtype])
        c = x.dtype.type(operand).item()
        k = f(x.ctypes.data, out.ctypes.data, x.size, OPS[op], c)
        return out[:k]


    def radix_pass(self, keys: np.ndarray, shift: int, bits: int, vals: np.ndarray | None = None):
        """Keys (uint32) ordered stably by the digit (key >> shift) & (2^bits - 1); vals follow."""
        keys = np.ascontiguousarray(keys, dtype=np.uint32)
        ko = np.empty_like(keys)
        vo = None
        vp = None
        if vals is not None:
            vals = np.ascontiguousarray(vals, dtype=np.uint32)
            assert vals.size == keys.size
            vo = np.empty_like(vals)
            vp = vals.ctypes.data
        self.lib.oracle_radix_pass_u32(keys.ctypes.data, vp, ko.ctypes.data, None if vo is None else vo.ctypes.data,
                                       keys.size, shift, bits)
        return ko, vo

    def moe_align(self, ids: np.ndarray, num_experts: int, block: int):
        """(counts[E], offsets[E+1], sorted[offsets[E]]) for int32 expert ids."""
        ids = np.ascontiguousarray(ids, dtype=np.int32).ravel()
        n = ids.size
        counts = np.empty(num_experts, dtype=np.int32)
        offsets = np.empty(num_experts + 1, dtype=np.int32)
        cap = n + num_experts * (block - 1)
        srt = np.empty(max(cap, 1), dtype=np.int32)
        total = self.lib.oracle_moe_align(ids.ctypes.data, n, num_experts, block, counts.ctypes.data,
                                          offsets.ctypes.data, srt.ctypes.data, cap)
        assert total >= 0
        return counts, offsets, srt[:total]


class ParallelScan:
    """The two-pass blocked scan on host threads (``parallel_scan.c``): a CPU
    comparison row for the benchmark, checked against the oracle, never used
    as one."""

    def __init__(self, path: str = PAR_LIB):
        if not os.path.exists(path):
            build()
        self.lib = ctypes.CDLL(path)
        for name in ("par_scan_u32", "par_scan_f32"):
            getattr(self.lib, name).argtypes = [_P, _P, _I64, ctypes.c_int, ctypes.c_int]
            getattr(self.lib, name).restype = ctypes.c_int

    def scan(self, x: np.ndarray, inclusive: bool, threads: int, out: np.ndarray | None = None) -> np.ndarray:
        """int32/uint32 (wrapping) or fp32 (fp64 accumulation, fp32 result) scan of x, in x's dtype."""
        x = np.ascontiguousarray(x)
        y = np.empty_like(x) if out is None else out
        assert y.dtype == x.dtype and y.size == x.size and y.flags.c_contiguous
        if x.dtype in (np.int32, np.uint32):
            rc = self.lib.par_scan_u32(x.ctypes.data, y.ctypes.data, x.size, int(inclusive), threads)
        elif x.dtype == np.float32:
            rc = self.lib.par_scan_f32(x.ctypes.data, y.ctypes.data, x.size, int(inclusive), threads)
        else:
            raise TypeError(f"unsupported dtype {x.dtype}")
        if rc != 0:
            raise RuntimeError("parallel_scan: could not start its threads")
        return y


def host_threads() -> int:
    """Cores this process may run on, capped at 16 (a one-GPU share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scan(x: np.ndarray, inclusive: bool):
    return default().scan(x, inclusive)


def compact(x: np.ndarray, op: str, operand) -> np.ndarray:
    return default().compact(x, op, operand)


def radix_pass(keys: np.ndarray, shift: int, bits: int, vals: np.ndarray | None = None):
    return default().radix_pass(keys, shift, bits, vals)


def moe_align(ids: np.ndarray, num_experts: int, block: int):
    return default().moe_align(ids, num_experts, block)
