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
    assert lib.ds_version() == 2
    for s in range(9):
        assert lib.ds_status_string(s).startswith(b"DS_")
    assert b"unknown" in lib.ds_status_string(99)


# ds_status values (include/devscan.h)
OK, INV, DTY, OVL, OOM, HIPERR, MIS, BIG, CAPT = range(9)


def test_status_values_match_the_header():
    """The binding's constants are the header's enum, value by value."""
    from primitives_device_scan_amd import _binding
    text = open(os.path.join(ROOT, "include", "devscan.h")).read()
    enum = text[text.index("DS_OK = 0"):text.index("} ds_status;")]
    pairs = dict((m.group(1), int(m.group(2))) for m in re.finditer(r"(DS_[A-Z_]+)\s*=\s*(\d+)", enum))
    assert pairs["DS_ERR_OUT_OF_MEMORY"] == 4 and pairs["DS_ERR_HIP"] == 5
    for name, value in pairs.items():
        assert getattr(_binding, name) == value, name
    assert [OK, INV, DTY, OVL, OOM, HIPERR, MIS, BIG, CAPT] == [pairs[k] for k in (
        "DS_OK", "DS_ERR_INVALID_VALUE", "DS_ERR_UNSUPPORTED_DTYPE", "DS_ERR_OVERLAP", "DS_ERR_OUT_OF_MEMORY",
        "DS_ERR_HIP", "DS_ERR_MISALIGNED", "DS_ERR_TOO_LARGE", "DS_ERR_STREAM_CAPTURING")]


def test_scan_noalloc_validation(lib):
    f = lib.ds_scan_noalloc
    assert f(7, 0, A, B, 10, None) == DTY
    assert f(0, 2, A, B, 10, None) == INV         # inclusive not 0/1
    assert f(0, 0, A, B, -1, None) == INV
    assert f(0, 0, None, B, 10, None) == INV
    assert f(0, 0, None, None, 0, None) == OK     # n == 0: nothing to do
    assert f(0, 0, A + 2, B, 10, None) == MIS
    assert f(0, 0, A, A + 4, 10, None) == OVL
    far = A + (16 << 30)                           # no overlap with A at these sizes
    assert f(0, 0, A, far, 1_200_000_000, None) == BIG   # more tiles than the fixed scratch holds
    assert f(3, 1, A, far, 600_000_000, None) == BIG


def test_fail_next_allocations_arguments(lib):
    assert lib.ds_fail_next_allocations(-1) == INV
    assert lib.ds_fail_next_allocations(0) == OK


# Fake, never-dereferenced addresses: validation must reject these on the host.
A = 0x7F0000000000
B = 0x7F0000100000


@pytest.mark.parametrize("fn", ["scan_exclusive", "scan_inclusive"])
def test_scan_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(7, A, B, 10, None) == DTY            # DS_ERR_UNSUPPORTED_DTYPE
    assert f(-1, A, B, 10, None) == DTY
    assert f(0, A, B, -1, None) == INV            # n < 0
    assert f(0, None, B, 10, None) == INV         # null with n > 0
    assert f(0, A, None, 10, None) == INV
    assert f(0, None, None, 0, None) == OK       # n == 0: nothing to do, no launch
    assert f(0, A, A + 4, 10, None) == OVL        # partial overlap
    assert f(0, A + 4, A, 10, None) == OVL
    assert f(0, A + 2, B, 10, None) == MIS        # misaligned for int32
    assert f(3, A + 4, B, 10, None) == MIS        # misaligned for int64
    assert f(0, A, B, 1 << 40, None) == BIG       # beyond the grid limit


def test_ds_scan_validation(lib):
    assert lib.ds_scan(0, 2, 0, A, B, 10, None) == INV   # inclusive not 0/1
    assert lib.ds_scan(0, 0, 4, A, B, 10, None) == INV   # bad algo
    assert lib.ds_scan(3, 0, 3, A, B, 10, None) == DTY   # blocked layout: 4-byte types only
    assert lib.ds_scan(0, 0, -1, A, B, 10, None) == INV
    assert lib.ds_scan(2, 1, 2, A, A + 8, 10, None) == OVL


def test_scan_seeded_validation(lib):
    f = lib.ds_scan_seeded
    S = 0x7F0000200000
    assert f(7, 0, A, B, 10, S, None) == DTY         # DS_ERR_UNSUPPORTED_DTYPE
    assert f(0, 2, A, B, 10, S, None) == INV         # inclusive not 0/1
    assert f(0, 0, A, B, -1, S, None) == INV
    assert f(0, 0, None, None, 0, S, None) == OK    # n == 0: nothing to do
    assert f(0, 0, A, B, 10, S + 2, None) == MIS     # seed misaligned for int32
    assert f(3, 0, A, B, 10, S + 4, None) == MIS     # ... and for int64
    assert f(0, 0, A, B, 10, B + 8, None) == OVL     # seed inside the output
    assert f(0, 0, A, A + 4, 10, S, None) == OVL     # partial overlap of in and out
    assert f(0, 0, A, B, 1 << 40, S, None) == BIG


def test_compact_validation(lib):
    C = 0x7F0000200000
    assert lib.compact_if(9, A, B, C, 10, 0, 0, None) == DTY
    assert lib.compact_if(0, A, B, C, 10, 6, 0, None) == INV   # bad cmp
    assert lib.compact_if(0, A, B, C, 10, -1, 0, None) == INV
    assert lib.compact_if(0, A, B, None, 10, 0, 0, None) == INV
    assert lib.compact_if(0, A, B, C, -3, 0, 0, None) == INV
    assert lib.compact_if(0, A, B, C + 4, 10, 0, 0, None) == MIS
    assert lib.compact_if(0, A, B, C, 1 << 32, 0, 0, None) == BIG
    assert lib.compact_if(0, A, A + 4, C, 10, 0, 0, None) == OVL
    assert lib.compact_if(0, None, B, C, 10, 0, 0, None) == INV


def test_compact_unordered_validation(lib):
    C = 0x7F0000200000
    f = lib.ds_compact_unordered
    assert f(9, A, B, C, 10, 0, 0, 0, None) == DTY
    assert f(0, A, B, C, 10, 6, 0, 0, None) == INV     # bad cmp
    assert f(0, A, B, C, 10, 0, 0, 2, None) == INV     # bad claim
    assert f(0, A, B, C, 10, 0, 0, -1, None) == INV
    assert f(0, A, B, None, 10, 0, 0, 1, None) == INV
    assert f(0, A, B, C, -3, 0, 0, 1, None) == INV
    assert f(0, A, B, C + 4, 10, 0, 0, 1, None) == MIS
    assert f(0, A, B, C, 1 << 32, 0, 0, 1, None) == BIG
    assert f(0, A, A, C, 10, 0, 0, 1, None) == OVL     # never in place: the order is not kept
    assert f(0, A, A + 4, C, 10, 0, 0, 0, None) == OVL
    assert f(0, None, B, C, 10, 0, 0, 0, None) == INV


def test_radix_pass_validation(lib):
    f = lib.ds_radix_pass
    C, D = 0x7F0000200000, 0x7F0000300000
    assert f(A, B, None, None, 10, 0, 0, None) == INV      # bits 0
    assert f(A, B, None, None, 10, 0, 9, None) == INV      # bits 9
    assert f(A, B, None, None, 10, -1, 8, None) == INV
    assert f(A, B, None, None, 10, 32, 1, None) == INV
    assert f(A, B, None, None, 10, 28, 8, None) == INV     # shift + bits > 32
    assert f(A, B, C, None, 10, 0, 8, None) == INV         # values in without values out
    assert f(A, B, None, None, -1, 0, 8, None) == INV
    assert f(None, None, None, None, 0, 0, 8, None) == OK  # n == 0: nothing to do
    assert f(A, B, None, None, 1 << 32, 0, 8, None) == BIG
    assert f(None, B, None, None, 10, 0, 8, None) == INV
    assert f(A + 2, B, None, None, 10, 0, 8, None) == MIS
    assert f(A, B, C + 2, D, 10, 0, 8, None) == MIS
    assert f(A, A, None, None, 10, 0, 8, None) == OVL      # never in place
    assert f(A, A + 8, None, None, 10, 0, 8, None) == OVL
    assert f(A, B, C, B + 4, 10, 0, 8, None) == OVL        # values out over keys out


def test_moe_align_validation(lib):
    f = lib.ds_moe_align
    C, D, E = 0x7F0000200000, 0x7F0000300000, 0x7F0000400000
    assert f(A, 100, 0, 64, B, C, D, 10000, None) == INV     # no experts
    assert f(A, 100, 512, 64, B, C, D, 100000, None) == INV  # more experts than buckets
    assert f(A, 100, 8, 0, B, C, D, 10000, None) == INV      # block 0
    assert f(A, -1, 8, 64, B, C, D, 10000, None) == INV
    assert f(A, 100, 8, 64, None, C, D, 10000, None) == INV
    assert f(None, 100, 8, 64, B, C, D, 10000, None) == INV
    assert f(A, 100, 8, 64, B, C, D, 100 + 8 * 63 - 1, None) == INV   # capacity below the worst case
    assert f(A, 1 << 31, 8, 64, B, C, D, 1 << 32, None) == BIG
    assert f(A + 2, 100, 8, 64, B, C, D, 10000, None) == MIS
    assert f(A, 100, 8, 64, B, C, A + 200, 10000, None) == OVL        # sorted ids over the input
    assert f(A, 100, 8, 64, B, B + 16, D, 10000, None) == OVL         # offsets over counts


def test_copy_validation(lib):
    assert lib.ds_copy(A, B, 17, None) == INV
    assert lib.ds_copy(A, B, -16, None) == INV
    assert lib.ds_copy(A, B, 0, None) == OK
    assert lib.ds_copy(A + 4, B, 32, None) == MIS
    assert lib.ds_copy(A, A + 16, 64, None) == OVL


def test_bandwidth_pattern_validation(lib):
    f = lib.ds_bandwidth_pattern
    assert f(6, 1, 0, A, B, 4096, None) == INV       # bad mode
    assert f(-1, 1, 0, A, B, 4096, None) == INV
    assert f(0, 3, 0, A, B, 4096, None) == INV       # vectors per thread not offered
    assert f(0, 1, 2, A, B, 4096, None) == INV       # bad layout
    assert f(0, 1, 0, A, B, 4100, None) == INV       # not whole vectors
    assert f(0, 1, 0, A, B, 0, None) == OK           # nothing to do
    assert f(0, 1, 0, None, B, 4096, None) == INV
    assert f(0, 1, 0, A + 4, B, 4096, None) == MIS
    assert f(2, 4, 1, A, A + 16, 4096, None) == OVL
    assert f(1, 4, 1, None, B, 1 << 50, None) == BIG  # write only: no input needed


def test_tile_queries(lib):
    from primitives_device_scan_amd import _binding
    # host-only queries: every tile is whole waves of a 256-thread workgroup;
    # the counting-sort tiles exist for 4-byte keys only
    for entry in _binding.TILE_OF.values():
        t = lib.ds_tile_elems(1, entry)
        assert t > 0 and t % 256 == OK, (entry, t)
    for name in ("counting_sort", "counting_sort_values", "moe_align", "lds_tile_scan"):
        assert lib.ds_tile_elems(3, _binding.TILE_OF[name]) == -1, name
    assert lib.ds_tile_elems(1, max(_binding.TILE_OF.values()) + 1) == -1
    assert lib.ds_tile_elems(1, -1) == -1
    assert lib.ds_tile_elems(9, 0) == -1
    for n in (0, 1, 4096, 1 << 20, 1 << 23, 100_000_007):
        t = lib.ds_scan_tile_elems(1, 0, n)
        assert t > 0 and t % 256 == OK, (n, t)
    assert lib.ds_scan_tile_elems(1, 2, 10) == -1 and lib.ds_scan_tile_elems(1, 0, -1) == -1


def test_query_timeout_null(lib):
    assert lib.ds_query_timeout(None, None) == INV


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
