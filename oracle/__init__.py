"""Sequential CPU oracle for device-wide prefix sums and stream compaction.

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

OPS = {"<": 0, "<=": 1, ">": 2, ">=": 3, "==": 4, "!=": 5}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-o", tmp, src], check=True)
    os.replace(tmp, out)
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
