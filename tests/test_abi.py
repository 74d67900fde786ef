"""The C-ABI library loads, exports every function include/*.h declares, and
rejects bad arguments on the host before any HIP call (CPU only: none of
these calls reaches a kernel launch)."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "primitives_device_scan_amd", "libdevscan.so")


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.append(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    from primitives_device_scan_amd import _binding
    return _binding.load_library(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("scan_exclusive", "scan_inclusive", "compact_if", "ds_scan", "ds_copy"):
        assert want in names, names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in include/ but not exported"
    from primitives_device_scan_amd import _binding
    assert sorted(_binding.EXPORTS) == sorted(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.ds_version() == 1
    for s in range(8):
        assert lib.ds_status_string(s).startswith(b"DS_")
    assert b"unknown" in lib.ds_status_string(99)


# Fake, never-dereferenced addresses: validation must reject these on the host.
A = 0x7F0000000000
B = 0x7F0000100000


@pytest.mark.parametrize("fn", ["scan_exclusive", "scan_inclusive"])
def test_scan_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(7, A, B, 10, None) == 2            # DS_ERR_UNSUPPORTED_DTYPE
    assert f(-1, A, B, 10, None) == 2
    assert f(0, A, B, -1, None) == 1            # n < 0
    assert f(0, None, B, 10, None) == 1         # null with n > 0
    assert f(0, A, None, 10, None) == 1
    assert f(0, None, None, 0, None) == 0       # n == 0: nothing to do, no launch
    assert f(0, A, A + 4, 10, None) == 3        # partial overlap
    assert f(0, A + 4, A, 10, None) == 3
    assert f(0, A + 2, B, 10, None) == 4        # misaligned for int32
    assert f(3, A + 4, B, 10, None) == 4        # misaligned for int64
    assert f(0, A, B, 1 << 40, None) == 7       # beyond the grid limit


def test_ds_scan_validation(lib):
    assert lib.ds_scan(0, 2, 0, A, B, 10, None) == 1   # inclusive not 0/1
    assert lib.ds_scan(0, 0, 3, A, B, 10, None) == 1   # bad algo
    assert lib.ds_scan(0, 0, -1, A, B, 10, None) == 1
    assert lib.ds_scan(2, 1, 2, A, A + 8, 10, None) == 3


def test_scan_seeded_validation(lib):
    f = lib.ds_scan_seeded
    S = 0x7F0000200000
    assert f(7, 0, A, B, 10, S, None) == 2         # DS_ERR_UNSUPPORTED_DTYPE
    assert f(0, 2, A, B, 10, S, None) == 1         # inclusive not 0/1
    assert f(0, 0, A, B, -1, S, None) == 1
    assert f(0, 0, None, None, 0, S, None) == 0    # n == 0: nothing to do
    assert f(0, 0, A, B, 10, S + 2, None) == 4     # seed misaligned for int32
    assert f(3, 0, A, B, 10, S + 4, None) == 4     # ... and for int64
    assert f(0, 0, A, B, 10, B + 8, None) == 3     # seed inside the output
    assert f(0, 0, A, A + 4, 10, S, None) == 3     # partial overlap of in and out
    assert f(0, 0, A, B, 1 << 40, S, None) == 7


def test_compact_validation(lib):
    C = 0x7F0000200000
    assert lib.compact_if(9, A, B, C, 10, 0, 0, None) == 2
    assert lib.compact_if(0, A, B, C, 10, 6, 0, None) == 1   # bad cmp
    assert lib.compact_if(0, A, B, C, 10, -1, 0, None) == 1
    assert lib.compact_if(0, A, B, None, 10, 0, 0, None) == 1
    assert lib.compact_if(0, A, B, C, -3, 0, 0, None) == 1
    assert lib.compact_if(0, A, B, C + 4, 10, 0, 0, None) == 4
    assert lib.compact_if(0, A, B, C, 1 << 32, 0, 0, None) == 7
    assert lib.compact_if(0, A, A + 4, C, 10, 0, 0, None) == 3
    assert lib.compact_if(0, None, B, C, 10, 0, 0, None) == 1


def test_compact_unordered_validation(lib):
    C = 0x7F0000200000
    f = lib.ds_compact_unordered
    assert f(9, A, B, C, 10, 0, 0, 0, None) == 2
    assert f(0, A, B, C, 10, 6, 0, 0, None) == 1     # bad cmp
    assert f(0, A, B, C, 10, 0, 0, 2, None) == 1     # bad claim
    assert f(0, A, B, C, 10, 0, 0, -1, None) == 1
    assert f(0, A, B, None, 10, 0, 0, 1, None) == 1
    assert f(0, A, B, C, -3, 0, 0, 1, None) == 1
    assert f(0, A, B, C + 4, 10, 0, 0, 1, None) == 4
    assert f(0, A, B, C, 1 << 32, 0, 0, 1, None) == 7
    assert f(0, A, A, C, 10, 0, 0, 1, None) == 3     # never in place: the order is not kept
    assert f(0, A, A + 4, C, 10, 0, 0, 0, None) == 3
    assert f(0, None, B, C, 10, 0, 0, 0, None) == 1


def test_radix_pass_validation(lib):
    f = lib.ds_radix_pass
    C, D = 0x7F0000200000, 0x7F0000300000
    assert f(A, B, None, None, 10, 0, 0, None) == 1      # bits 0
    assert f(A, B, None, None, 10, 0, 9, None) == 1      # bits 9
    assert f(A, B, None, None, 10, -1, 8, None) == 1
    assert f(A, B, None, None, 10, 32, 1, None) == 1
    assert f(A, B, None, None, 10, 28, 8, None) == 1     # shift + bits > 32
    assert f(A, B, C, None, 10, 0, 8, None) == 1         # values in without values out
    assert f(A, B, None, None, -1, 0, 8, None) == 1
    assert f(None, None, None, None, 0, 0, 8, None) == 0  # n == 0: nothing to do
    assert f(A, B, None, None, 1 << 32, 0, 8, None) == 7
    assert f(None, B, None, None, 10, 0, 8, None) == 1
    assert f(A + 2, B, None, None, 10, 0, 8, None) == 4
    assert f(A, B, C + 2, D, 10, 0, 8, None) == 4
    assert f(A, A, None, None, 10, 0, 8, None) == 3      # never in place
    assert f(A, A + 8, None, None, 10, 0, 8, None) == 3
    assert f(A, B, C, B + 4, 10, 0, 8, None) == 3        # values out over keys out


def test_moe_align_validation(lib):
    f = lib.ds_moe_align
    C, D, E = 0x7F0000200000, 0x7F0000300000, 0x7F0000400000
    assert f(A, 100, 0, 64, B, C, D, 10000, None) == 1     # no experts
    assert f(A, 100, 512, 64, B, C, D, 100000, None) == 1  # more experts than buckets
    assert f(A, 100, 8, 0, B, C, D, 10000, None) == 1      # block 0
    assert f(A, -1, 8, 64, B, C, D, 10000, None) == 1
    assert f(A, 100, 8, 64, None, C, D, 10000, None) == 1
    assert f(None, 100, 8, 64, B, C, D, 10000, None) == 1
    assert f(A, 100, 8, 64, B, C, D, 100 + 8 * 63 - 1, None) == 1   # capacity below the worst case
    assert f(A, 1 << 31, 8, 64, B, C, D, 1 << 32, None) == 7
    assert f(A + 2, 100, 8, 64, B, C, D, 10000, None) == 4
    assert f(A, 100, 8, 64, B, C, A + 200, 10000, None) == 3        # sorted ids over the input
    assert f(A, 100, 8, 64, B, B + 16, D, 10000, None) == 3         # offsets over counts


def test_copy_validation(lib):
    assert lib.ds_copy(A, B, 17, None) == 1
    assert lib.ds_copy(A, B, -16, None) == 1
    assert lib.ds_copy(A, B, 0, None) == 0
    assert lib.ds_copy(A + 4, B, 32, None) == 4
    assert lib.ds_copy(A, A + 16, 64, None) == 3


def test_tile_queries(lib):
    from primitives_device_scan_amd import _binding
    # host-only queries: every tile is whole waves of a 256-thread workgroup;
    # the counting-sort tiles exist for 4-byte keys only
    for entry in _binding.TILE_OF.values():
        t = lib.ds_tile_elems(1, entry)
        assert t > 0 and t % 256 == 0, (entry, t)
    for name in ("counting_sort", "counting_sort_values", "moe_align", "lds_tile_scan"):
        assert lib.ds_tile_elems(3, _binding.TILE_OF[name]) == -1, name
    assert lib.ds_tile_elems(1, max(_binding.TILE_OF.values()) + 1) == -1
    assert lib.ds_tile_elems(1, -1) == -1
    assert lib.ds_tile_elems(9, 0) == -1
    for n in (0, 1, 4096, 1 << 20, 1 << 23, 100_000_007):
        t = lib.ds_scan_tile_elems(1, 0, n)
        assert t > 0 and t % 256 == 0, (n, t)
    assert lib.ds_scan_tile_elems(1, 2, 10) == -1 and lib.ds_scan_tile_elems(1, 0, -1) == -1


def test_query_timeout_null(lib):
    assert lib.ds_query_timeout(None, None) == 1


def test_binding_refuses_a_missing_library(tmp_path):
    from primitives_device_scan_amd import _binding
    with pytest.raises(ImportError):
        _binding.load_library(str(tmp_path / "nope.so"))


def test_binding_operand_bits():
    import torch
    from primitives_device_scan_amd import _binding
    assert _binding.operand_bits(torch.float32, 1.0) == 0x3F800000
    assert _binding.operand_bits(torch.int32, -1) == 0xFFFFFFFF
    assert _binding.operand_bits(torch.int64, -2) == 0xFFFFFFFFFFFFFFFE
