// launch.hpp -- host-side launchers of the kernels in csrc/*.hip, called by
// the C ABI (api.hip) after it has validated the arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds {

struct Ctrl;

// Device memory of one workspace.
struct DevWs {
    Ctrl* ctrl;          // control words (epoch, give-up flag)
    uint64_t* status;    // 2 x 64-bit words per tile (look-back status)
    void* totals;        // 8 bytes per tile (three-pass tile totals)
};

enum ElemKind { kU32 = 0, kF32 = 1, kU64 = 2, kI32 = 3, kI64 = 4 };

int64_t tile_elems(ElemKind kind, bool inclusive, int64_t n);  // look-back scan tile for n elements
int64_t three_pass_tile_elems(int elem_bytes);  // three-pass scan tile
int64_t compact_tile_elems(int elem_bytes);     // compaction tile
int64_t tile_bytes();

// seed: null, or one element of the scan's type in device memory added to
// every prefix (a seeded scan: one shard of a longer sequence).
hipError_t launch_lookback_scan(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                const DevWs& ws, uint32_t spin_limit, hipStream_t stream,
                                const void* seed = nullptr);

// The look-back scan with the tile transposed through LDS (blocked layout;
// 4-byte types only) and its tile for n elements.
hipError_t launch_lookback_blocked(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                   const DevWs& ws, uint32_t spin_limit, hipStream_t stream);
int64_t blocked_tile_elems(int64_t n);

hipError_t launch_three_pass_scan(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                  const DevWs& ws, hipStream_t stream);

hipError_t launch_compact(ElemKind kind, const void* in, void* out, int64_t* num_selected, int64_t n,
                          int cmp, uint64_t operand_bits, const DevWs& ws, uint32_t spin_limit,
                          hipStream_t stream);

// Writes v to *p with a one-thread kernel (a count when there is nothing to scan).
hipError_t launch_write_count(int64_t* p, int64_t v, hipStream_t stream);

hipError_t launch_compact_unordered(ElemKind kind, const void* in, void* out, int64_t* count, int64_t n, int cmp,
                                    uint64_t operand_bits, bool per_workgroup, hipStream_t stream);

hipError_t launch_copy(const void* in, void* out, int64_t nbytes, hipStream_t stream);

// Access-pattern probes (ds_bandwidth_pattern): mode 0 read, 1 write, 2 copy,
// 3 read all / write half; vpt 1, 2, 4, 8, 16, 20 or 28; layout 0 contiguous,
// 1 4 KiB chunks at a 32 KiB stride.
bool pattern_vpt_ok(int vpt);
hipError_t launch_pattern(int mode, int vpt, int layout, const void* in, void* out, int64_t nbytes,
                          hipStream_t stream);

// Counting-sort pass (radix sort step, MoE alignment): keys per workgroup
// tile, and the most real buckets a pass can have.
int64_t moe_one_launch_max();          // MoE inputs up to this many ids take one single-workgroup launch
int64_t sort_tile_elems(bool values);  // radix pass, keys only or with values
int64_t sort_table_columns(bool values, int64_t n);  // radix pass: entries per digit in its count table
int64_t sort_aux_words(bool values, int64_t n, int bits);  // radix pass: its table and group prefixes
int64_t moe_tile_elems();              // MoE alignment
int sort_max_buckets();

// table: (1 << bits) * tiles 32-bit words of scratch (the digit-major counts,
// scanned in place); ws: look-back workspace for a scan of that many words.
hipError_t launch_radix_pass(const uint32_t* keys, const uint32_t* vals_in, uint32_t* keys_out, uint32_t* vals_out,
                             int64_t n, int shift, int bits, uint32_t* table, const DevWs& ws, uint32_t spin_limit,
                             hipStream_t stream);

struct MoeOut {
    int32_t* counts;    // [experts]
    int32_t* offsets;   // [experts + 1]
    int32_t* sorted;    // [capacity]
    int block;
    int64_t capacity;
};

// hist, slots: experts * tiles 32-bit words each of scratch.
hipError_t launch_moe_align(const int32_t* ids, int64_t n, int experts, const MoeOut& out, uint32_t* hist,
                            uint32_t* slots, const DevWs& ws, uint32_t spin_limit, hipStream_t stream);

// Exclusive scan of `count` tile totals in place (one workgroup, carried sum).
hipError_t launch_scan_totals(ElemKind kind, void* totals, int64_t count, hipStream_t stream);

// 4,096-element tile scans in LDS and the three-kernel pipeline built on them.
int64_t lds_tile_elems();
hipError_t launch_tile_scan(ElemKind kind, int variant, const void* in, void* out, void* tile_sums, int64_t n,
                            hipStream_t stream);
hipError_t launch_tile_pipeline(ElemKind kind, int variant, const void* in, void* out, int64_t n,
                                const DevWs& ws, hipStream_t stream);

}  // namespace ds
