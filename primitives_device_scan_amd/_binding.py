"""ctypes binding of libdevscan.so (include/devscan.h).

Argument marshalling only: every step of a scan or compaction runs in the HIP
kernels of the library. torch provides device memory and streams. Importing
this module fails with ImportError when the library has not been built; there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import struct

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdevscan.so")

# ds_dtype, ds_cmp, ds_algo, ds_status (include/devscan.h)
DS_INT32, DS_UINT32, DS_FP32, DS_INT64, DS_UINT64 = range(5)
CMP = {"<": 0, "<=": 1, ">": 2, ">=": 3, "==": 4, "!=": 5}
ALGO = {"default": 0, "lookback": 1, "three_pass": 2, "lookback_blocked": 3}
DS_OK = 0
DS_ERR_INVALID_VALUE = 1
DS_ERR_UNSUPPORTED_DTYPE = 2
DS_ERR_OVERLAP = 3
DS_ERR_OUT_OF_MEMORY = 4
DS_ERR_HIP = 5
DS_ERR_MISALIGNED = 6
DS_ERR_TOO_LARGE = 7
DS_ERR_STREAM_CAPTURING = 8

EXPORTS = ["scan_exclusive", "scan_inclusive", "ds_scan", "ds_scan_seeded", "ds_scan_noalloc", "compact_if", "ds_compact_unordered", "ds_radix_pass",
           "ds_moe_align", "ds_copy", "ds_bandwidth_pattern", "ds_tile_scan", "ds_tile_pipeline",
           "ds_tile_elems", "ds_scan_tile_elems", "ds_query_timeout", "ds_fail_next_allocations", "ds_set_spin_limit",
           "ds_status_string", "ds_release_workspace", "ds_version"]
TILE_OF = {"scan_exclusive": 0, "scan_inclusive": 1, "three_pass": 2, "compact": 3, "lds_tile_scan": 4,
           "counting_sort": 5, "counting_sort_values": 6, "moe_align": 7}
TILE_VARIANTS = {"tree": 0, "tree_pad1": 1, "tree_pad2": 2, "hillis_steele": 3}
PATTERNS = {"read": 0, "write": 1, "copy": 2, "read_half": 3, "read_half_held": 4, "copy_held": 5}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python primitives_device_scan_amd/build.py` "
                          "(or __graft_entry__.build()); there is no CPU fallback")
    L = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("scan_exclusive", "scan_inclusive"):
        getattr(L, name).argtypes = [I, P, P, I64, P]
        getattr(L, name).restype = I
    L.ds_scan.argtypes = [I, I, I, P, P, I64, P]
    L.ds_scan.restype = I
    L.ds_scan_seeded.argtypes = [I, I, P, P, I64, P, P]
    L.ds_scan_seeded.restype = I
    L.ds_scan_noalloc.argtypes = [I, I, P, P, I64, P]
    L.ds_scan_noalloc.restype = I
    L.compact_if.argtypes = [I, P, P, P, I64, I, ctypes.c_uint64, P]
    L.compact_if.restype = I
    L.ds_compact_unordered.argtypes = [I, P, P, P, I64, I, ctypes.c_uint64, I, P]
    L.ds_compact_unordered.restype = I
    L.ds_radix_pass.argtypes = [P, P, P, P, I64, I, I, P]
    L.ds_radix_pass.restype = I
    L.ds_moe_align.argtypes = [P, I64, I, I, P, P, P, I64, P]
    L.ds_moe_align.restype = I
    L.ds_copy.argtypes = [P, P, I64, P]
    L.ds_copy.restype = I
    L.ds_bandwidth_pattern.argtypes = [I, I, I, P, P, I64, P]
    L.ds_bandwidth_pattern.restype = I
    L.ds_tile_scan.argtypes = [I, I, P, P, P, I64, P]
    L.ds_tile_scan.restype = I
    L.ds_tile_pipeline.argtypes = [I, I, P, P, I64, P]
    L.ds_tile_pipeline.restype = I
    L.ds_query_timeout.argtypes = [P, ctypes.POINTER(I)]
    L.ds_query_timeout.restype = I
    L.ds_fail_next_allocations.argtypes = [I]
    L.ds_fail_next_allocations.restype = I
    L.ds_set_spin_limit.argtypes = [ctypes.c_uint32]
    L.ds_set_spin_limit.restype = I
    L.ds_status_string.argtypes = [I]
    L.ds_status_string.restype = ctypes.c_char_p
    L.ds_release_workspace.argtypes = []
    L.ds_release_workspace.restype = None
    L.ds_tile_elems.argtypes = [I, I]
    L.ds_tile_elems.restype = I64
    L.ds_scan_tile_elems.argtypes = [I, I, I64]
    L.ds_scan_tile_elems.restype = I64
    L.ds_version.argtypes = []
    L.ds_version.restype = I
    return L


lib = load_library()


class DevscanError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.ds_status_string(status).decode()}")


def _check(status: int, what: str):
    if status != DS_OK:
        raise DevscanError(status, what)


_DTYPES = {torch.int32: DS_INT32, torch.float32: DS_FP32, torch.int64: DS_INT64}
if hasattr(torch, "uint32"):
    _DTYPES[torch.uint32] = DS_UINT32
if hasattr(torch, "uint64"):
    _DTYPES[torch.uint64] = DS_UINT64


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}; one of {list(_DTYPES)}")
    return _DTYPES[dt]


def _stream_handle(x: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensor(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def scan(x: torch.Tensor, inclusive: bool, out: torch.Tensor | None = None, *, algo: str = "default",
         stream=None) -> torch.Tensor:
    """Exclusive or inclusive scan of the 1-D contiguous GPU tensor x (into out, may be x)."""
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out")
    if out.dtype != x.dtype or out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must match x in dtype, size and device")
    with torch.cuda.device(x.device):
        _check(lib.ds_scan(code, int(bool(inclusive)), ALGO[algo], x.data_ptr(), out.data_ptr(), x.numel(),
                           _stream_handle(x, stream)), "ds_scan")
    return out


def scan_seeded(x: torch.Tensor, inclusive: bool, seed: torch.Tensor | None, out: torch.Tensor | None = None, *,
                stream=None) -> torch.Tensor:
    """One shard of a longer scan: the scan of x with every prefix offset by seed
    (a one-element GPU tensor of x's dtype, or None for 0)."""
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out")
    if out.dtype != x.dtype or out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must match x in dtype, size and device")
    if seed is not None and (seed.dtype != x.dtype or seed.numel() != 1 or seed.device != x.device):
        raise ValueError("seed must be one element of x's dtype on x's device")
    with torch.cuda.device(x.device):
        _check(lib.ds_scan_seeded(code, int(bool(inclusive)), x.data_ptr(), out.data_ptr(), x.numel(),
                                  None if seed is None else seed.data_ptr(), _stream_handle(x, stream)),
               "ds_scan_seeded")
    return out


def scan_exclusive(x: torch.Tensor, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    _check_tensor(x, "x")
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out")
    if out.dtype != x.dtype or out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must match x in dtype, size and device")
    with torch.cuda.device(x.device):
        _check(lib.scan_exclusive(dtype_code(x.dtype), x.data_ptr(), out.data_ptr(), x.numel(),
                                  _stream_handle(x, stream)), "scan_exclusive")
    return out


def scan_inclusive(x: torch.Tensor, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    _check_tensor(x, "x")
    if out is None:
        out = torch.empty_like(x)
    _check_tensor(out, "out")
    if out.dtype != x.dtype or out.numel() != x.numel() or out.device != x.device:
        raise ValueError("out must match x in dtype, size and device")
    with torch.cuda.device(x.device):
        _check(lib.scan_inclusive(dtype_code(x.dtype), x.data_ptr(), out.data_ptr(), x.numel(),
                                  _stream_handle(x, stream)), "scan_inclusive")
    return out


def operand_bits(dtype: torch.dtype, value) -> int:
    """The bit pattern compact_if expects for `value` in `dtype`."""
    code = dtype_code(dtype)
    if code == DS_FP32:
        return struct.unpack("<I", struct.pack("<f", float(value)))[0]
    if code in (DS_INT32, DS_UINT32):
        return int(value) & 0xFFFFFFFF
    return int(value) & 0xFFFFFFFFFFFFFFFF


def compact_if(x: torch.Tensor, cmp: str, operand, out: torch.Tensor | None = None,
               num_selected: torch.Tensor | None = None, *, stream=None):
    """Order-preserving compaction of x by (x_i cmp operand).

    Returns (out, num_selected): out holds the kept elements in out[:k], and
    num_selected is a one-element int64 GPU tensor holding k.
    """
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if num_selected is None:
        num_selected = torch.empty(1, dtype=torch.int64, device=x.device)
    _check_tensor(out, "out")
    _check_tensor(num_selected, "num_selected")
    if out.dtype != x.dtype or out.numel() < x.numel() or out.device != x.device:
        raise ValueError("out must match x in dtype and device and hold x.numel() elements")
    if num_selected.dtype != torch.int64 or num_selected.numel() < 1:
        raise ValueError("num_selected must be an int64 tensor of at least one element")
    with torch.cuda.device(x.device):
        _check(lib.compact_if(code, x.data_ptr(), out.data_ptr(), num_selected.data_ptr(), x.numel(), CMP[cmp],
                              operand_bits(x.dtype, operand), _stream_handle(x, stream)), "compact_if")
    return out, num_selected


CLAIM = {"wave": 0, "workgroup": 1}


def compact_unordered(x: torch.Tensor, cmp: str, operand, out: torch.Tensor | None = None,
                      num_selected: torch.Tensor | None = None, *, claim: str = "workgroup", stream=None):
    """Compaction in no particular order (atomic space claims); returns (out, num_selected)."""
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    out = torch.empty_like(x) if out is None else out
    num_selected = torch.empty(1, dtype=torch.int64, device=x.device) if num_selected is None else num_selected
    _check_tensor(out, "out")
    _check_tensor(num_selected, "num_selected")
    if out.dtype != x.dtype or out.numel() < x.numel() or num_selected.dtype != torch.int64:
        raise ValueError("out must match x and hold x.numel() elements; num_selected must be int64")
    with torch.cuda.device(x.device):
        _check(lib.ds_compact_unordered(code, x.data_ptr(), out.data_ptr(), num_selected.data_ptr(), x.numel(),
                                        CMP[cmp], operand_bits(x.dtype, operand), CLAIM[claim],
                                        _stream_handle(x, stream)), "ds_compact_unordered")
    return out, num_selected


def radix_pass(keys: torch.Tensor, shift: int, bits: int, vals: torch.Tensor | None = None,
               keys_out: torch.Tensor | None = None, vals_out: torch.Tensor | None = None, *, stream=None):
    """One stable counting-sort pass over the digit (key >> shift) & (2^bits - 1) of 32-bit keys
    (int32 or uint32 storage, compared as unsigned); returns (keys_out, vals_out or None)."""
    _check_tensor(keys, "keys")
    if keys.element_size() != 4 or keys.is_floating_point():
        raise TypeError("keys must be 32-bit integers")
    keys_out = torch.empty_like(keys) if keys_out is None else keys_out
    _check_tensor(keys_out, "keys_out")
    if vals is not None:
        _check_tensor(vals, "vals")
        vals_out = torch.empty_like(vals) if vals_out is None else vals_out
        _check_tensor(vals_out, "vals_out")
        if vals.element_size() != 4 or vals.numel() != keys.numel() or vals_out.numel() < keys.numel():
            raise ValueError("vals must hold one 32-bit value per key")
    if keys_out.numel() < keys.numel():
        raise ValueError("keys_out is too small")
    with torch.cuda.device(keys.device):
        _check(lib.ds_radix_pass(keys.data_ptr(), keys_out.data_ptr(), None if vals is None else vals.data_ptr(),
                                 None if vals is None else vals_out.data_ptr(), keys.numel(), shift, bits,
                                 _stream_handle(keys, stream)), "ds_radix_pass")
    return keys_out, (vals_out if vals is not None else None)


def moe_align(topk_ids: torch.Tensor, num_experts: int, block: int, *, stream=None):
    """MoE alignment of int32 expert ids [tokens, top_k]: returns (counts[E], offsets[E+1],
    sorted_ids[capacity]); the first offsets[E] entries of sorted_ids are written."""
    _check_tensor(topk_ids, "topk_ids")
    if topk_ids.dtype != torch.int32:
        raise TypeError("topk_ids must be int32")
    n = topk_ids.numel()
    cap = max(1, n + num_experts * (block - 1))
    dev = topk_ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        _check(lib.ds_moe_align(topk_ids.data_ptr(), n, num_experts, block, counts.data_ptr(), offsets.data_ptr(),
                                sorted_ids.data_ptr(), cap, _stream_handle(topk_ids, stream)), "ds_moe_align")
    return counts, offsets, sorted_ids


def copy(src: torch.Tensor, dst: torch.Tensor, *, stream=None) -> torch.Tensor:
    """The copy kernel with the scan's access pattern (bandwidth ceiling)."""
    _check_tensor(src, "src")
    _check_tensor(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    with torch.cuda.device(src.device):
        _check(lib.ds_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream_handle(src, stream)), "ds_copy")
    return dst


def tile_scan(x: torch.Tensor, variant: str, out: torch.Tensor | None = None,
              tile_sums: torch.Tensor | None = None, *, stream=None):
    """Block-level exclusive scan of every 4,096-element tile of x in LDS; returns (out, tile_sums)."""
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    out = torch.empty_like(x) if out is None else out
    tiles = (x.numel() + 4095) // 4096
    tile_sums = torch.empty(tiles, dtype=x.dtype, device=x.device) if tile_sums is None else tile_sums
    _check_tensor(out, "out")
    _check_tensor(tile_sums, "tile_sums")
    if tile_sums.numel() < tiles or tile_sums.dtype != x.dtype or out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x; tile_sums must hold ceil(n/4096) elements of x's dtype")
    with torch.cuda.device(x.device):
        _check(lib.ds_tile_scan(code, TILE_VARIANTS[variant], x.data_ptr(), out.data_ptr(), tile_sums.data_ptr(),
                                x.numel(), _stream_handle(x, stream)), "ds_tile_scan")
    return out, tile_sums


def tile_pipeline(x: torch.Tensor, variant: str, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """Device-wide exclusive scan by the three-kernel pipeline over LDS tile scans."""
    _check_tensor(x, "x")
    code = dtype_code(x.dtype)
    out = torch.empty_like(x) if out is None else out
    _check_tensor(out, "out")
    if out.numel() != x.numel() or out.dtype != x.dtype:
        raise ValueError("out must match x")
    with torch.cuda.device(x.device):
        _check(lib.ds_tile_pipeline(code, TILE_VARIANTS[variant], x.data_ptr(), out.data_ptr(), x.numel(),
                                    _stream_handle(x, stream)), "ds_tile_pipeline")
    return out


def query_timeout(device=None, stream=None) -> bool:
    """Waits for the stream; True if a look-back wait gave up since the last query."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        s = torch.cuda.current_stream(dev) if stream is None else stream
        flag = ctypes.c_int(0)
        _check(lib.ds_query_timeout(s.cuda_stream if hasattr(s, "cuda_stream") else int(s), ctypes.byref(flag)),
               "ds_query_timeout")
    return bool(flag.value)


def set_spin_limit(polls: int):
    _check(lib.ds_set_spin_limit(int(polls)), "ds_set_spin_limit")


def release_workspace():
    lib.ds_release_workspace()
