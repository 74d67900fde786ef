"""Device-wide prefix sums (exclusive / inclusive scan), stream compaction and
the scan's counting-sort users (a radix-sort pass, MoE alignment) for AMD
Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of
include/devscan.h (libdevscan.so, built in-tree by
``python primitives_device_scan_amd/build.py``). This package is its Python
binding: argument checks and marshalling, with torch for device memory and
streams. Importing it fails when the library is missing.
"""
from ._binding import (ALGO, CMP, DS_ERR_HIP, DS_ERR_INVALID_VALUE, DS_ERR_MISALIGNED, DS_ERR_OUT_OF_MEMORY,
                       DS_ERR_OVERLAP, DS_ERR_STREAM_CAPTURING, DS_ERR_TOO_LARGE, DS_ERR_UNSUPPORTED_DTYPE, DS_FP32,
                       DS_INT32, DS_INT64, DS_OK, DS_UINT32, DS_UINT64, EXPORTS, LIB_PATH,
                       TILE_VARIANTS, DevscanError, compact_if, compact_unordered, copy, dtype_code, lib,
                       load_library, moe_align, operand_bits, query_timeout, radix_pass, release_workspace, scan,
                       scan_exclusive, scan_inclusive, scan_seeded, set_spin_limit, tile_pipeline, tile_scan)

__all__ = ["scan", "scan_exclusive", "scan_inclusive", "scan_seeded", "compact_if", "compact_unordered",
           "radix_pass", "moe_align", "copy", "tile_scan", "tile_pipeline", "query_timeout", "set_spin_limit",
           "release_workspace", "DevscanError", "lib", "LIB_PATH", "EXPORTS", "ALGO", "CMP", "TILE_VARIANTS"]
