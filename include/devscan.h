/*
 * devscan.h -- device-wide prefix sums (scans), stream compaction and two
 * users of the scan built on one counting-sort pass (a radix-sort pass, MoE
 * token alignment) for AMD Instinct MI355X (gfx950), as a plain C ABI.
 *
 * Every entry point takes device pointers and an element count, enqueues its
 * work on `stream` and returns without waiting for it. The caller owns every
 * pointer it passes and keeps the memory alive until the stream work is done.
 * The library owns only a small workspace per (device, stream): per-tile
 * status words, a launch epoch, for the three-pass form the tile totals, and
 * for the counting-sort pass its digit-by-tile table. It grows on demand and
 * is freed by ds_release_workspace().
 *
 * Errors. Argument errors are found on the host before any HIP call and
 * returned at once (DS_ERR_*); launch failures return DS_ERR_HIP. A fault
 * inside a kernel surfaces, as usual in HIP, at the caller's next
 * synchronisation of the stream.
 *
 * Bounded waits. The single-pass kernels wait for earlier tiles' status
 * words; every wait gives up after a spin limit (ds_set_spin_limit), so a
 * kernel always finishes. A call in which any wait gave up has produced
 * invalid outputs (compact_if writes -1 as its count when its last tile saw
 * the give-up); ds_query_timeout reports it and restores the workspace.
 *
 * Graph capture. A call records only kernel launches once the workspace of
 * its (device, stream) is large enough, so make one call of at least the
 * captured size on the stream before capturing it; otherwise the call
 * returns DS_ERR_STREAM_CAPTURING and records nothing. Status words carry a
 * 30-bit launch number that the kernels advance themselves, and the host
 * clears them every 2^29 eager launches; a captured graph therefore may be
 * replayed at most 2^29 times before ds_release_workspace() (or one eager
 * call after 2^29 launches) clears them again.
 *
 * Element types: DS_INT32 / DS_UINT32 / DS_FP32 (4 bytes) and DS_INT64 /
 * DS_UINT64 (8 bytes), stored contiguously. Integer sums wrap modulo 2^32 or
 * 2^64 (signed and unsigned give the same bits). fp32 sums are fp32 additions
 * in an order the library chooses; they meet |y_i - exact_i| <= 1e-5 *
 * sum_{j<=i} |x_j| at the sizes the tests cover, and may differ in the last
 * bits from run to run (the look-back can stop at different tiles).
 * Pointers must be aligned to the element size (DS_ERR_MISALIGNED
 * otherwise). Any such pointer takes the 16-byte vector path (a slice that
 * starts mid-vector, x + 1 say, costs a few percent); only the ragged end of
 * the data goes element by element.
 */
#ifndef DEVSCAN_H
#define DEVSCAN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DS_INT32 = 0,
    DS_UINT32 = 1,
    DS_FP32 = 2,
    DS_INT64 = 3,
    DS_UINT64 = 4
} ds_dtype;

/* Comparison for compact_if: keep x_i when (x_i OP operand). */
typedef enum { DS_LT = 0, DS_LE = 1, DS_GT = 2, DS_GE = 3, DS_EQ = 4, DS_NE = 5 } ds_cmp;

/* Device-level algorithm for ds_scan. */
typedef enum {
    DS_ALGO_DEFAULT = 0,   /* the single-pass look-back scan */
    DS_ALGO_LOOKBACK = 1,  /* one launch: tiles publish aggregates / inclusive prefixes and look back */
    DS_ALGO_THREE_PASS = 2, /* three launches: reduce tiles, scan tile totals, rescan tiles seeded */
    DS_ALGO_LOOKBACK_BLOCKED = 3 /* the look-back scan with each tile transposed through LDS so that a
                                    thread scans contiguous elements (4-byte types only; a measured
                                    alternative to the default striped tile) */
} ds_algo;

/* Block-level tile scan held in LDS, for ds_tile_scan / ds_tile_pipeline. */
typedef enum {
    DS_TILE_TREE = 0,      /* work-efficient up-sweep / down-sweep tree, word i at i */
    DS_TILE_TREE_PAD1 = 1, /* same tree, word i at i + i/32 */
    DS_TILE_TREE_PAD2 = 2, /* same tree, word i at i + i/32 + i/1024 */
    DS_TILE_HS = 3         /* Hillis-Steele, double-buffered */
} ds_tile_variant;

typedef enum {
    DS_OK = 0,
    DS_ERR_INVALID_VALUE = 1,     /* n < 0, null pointer with n > 0, bad enum value */
    DS_ERR_UNSUPPORTED_DTYPE = 2, /* dtype not one of ds_dtype */
    DS_ERR_OVERLAP = 3,           /* input and output overlap without being the same buffer */
    DS_ERR_OUT_OF_MEMORY = 4,     /* workspace allocation failed */
    DS_ERR_HIP = 5,               /* a HIP runtime call or kernel launch failed */
    DS_ERR_MISALIGNED = 6,        /* a pointer not aligned to the element size */
    DS_ERR_TOO_LARGE = 7,         /* n beyond what the entry point supports */
    DS_ERR_STREAM_CAPTURING = 8   /* the workspace would have to be allocated, grown or cleared while
                                     `stream` is being captured into a graph */
} ds_status;

/*
 * Exclusive scan: d_out[0] = 0, d_out[i] = d_in[0] + ... + d_in[i-1].
 * Defined in "Prefix sum and other parallel patterns" (section "Definitions")
 * and "Day 31 -- CUDA prefix sum, the Hillis-Steele scan" (section "Two scans,
 * and which one hands you the total"). Single pass with decoupled look-back
 * ("Prefix sum and other parallel patterns", section "A device-level scan:
 * scan then propagate").
 *   dtype   one of ds_dtype
 *   d_in    device pointer to n elements (read)
 *   d_out   device pointer to n elements (written); may equal d_in (in place),
 *           must not otherwise overlap it
 *   n       element count, n >= 0; n == 0 enqueues nothing; n <= 68,719,472,640
 *           (2^24 - 1 blocks of 4,096: the grid of any entry point stays below
 *           2^32 work-items), DS_ERR_TOO_LARGE beyond
 *   stream  HIP stream of the current device (0 = null stream)
 * Returns DS_OK or a ds_status error.
 */
int scan_exclusive(int dtype, const void* d_in, void* d_out, int64_t n, hipStream_t stream);

/*
 * Inclusive scan: d_out[i] = d_in[0] + ... + d_in[i]. Same sources, arguments
 * and errors as scan_exclusive.
 */
int scan_inclusive(int dtype, const void* d_in, void* d_out, int64_t n, hipStream_t stream);

/*
 * Either scan with an explicit device-level algorithm: `inclusive` 0 or 1,
 * `algo` one of ds_algo. DS_ALGO_THREE_PASS is the multi-block scheme of
 * "Day 32 -- The CUDA scan algorithm: the tree and the three kernels"
 * (section "One block scans 4,096. Ten million needs three kernels.") in its
 * reduce-then-scan form: pass 1 only reads (tile totals), pass 2 scans the
 * totals in one workgroup, pass 3 rescans each tile seeded with its offset.
 * DS_ALGO_LOOKBACK_BLOCKED returns DS_ERR_UNSUPPORTED_DTYPE for 8-byte types.
 * Other arguments and errors as scan_exclusive.
 */
int ds_scan(int dtype, int inclusive, int algo, const void* d_in, void* d_out, int64_t n,
            hipStream_t stream);

/*
 * One shard of a longer scan: the look-back scan of d_in (`inclusive` 0 or 1)
 * with every prefix offset by *d_seed, the sum of all elements before this
 * shard. This is what each GPU would run when a scan is split into
 * contiguous shards over several GPUs (each reduces its shard, the shard
 * totals are exchanged and scanned, each scans its shard seeded with its
 * offset): the multi-block scheme of "Prefix sum and other parallel
 * patterns" (section "A device-level scan: scan then propagate") one level
 * up, with the shard offset in the role of a block's starting offset.
 *   d_seed  NULL (a seed of 0), or one element of `dtype` in device memory,
 *           aligned to its size and outside d_out (DS_ERR_MISALIGNED,
 *           DS_ERR_OVERLAP); read by the kernel when it runs, so earlier work
 *           on the same stream may produce it. Integers wrap as in the scan;
 *           an fp32 seed is added in fp32.
 * Other arguments and errors as scan_exclusive.
 */
int ds_scan_seeded(int dtype, int inclusive, const void* d_in, void* d_out, int64_t n, const void* d_seed,
                   hipStream_t stream);

/*
 * The look-back scan (as ds_scan with DS_ALGO_LOOKBACK, `inclusive` 0 or 1)
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It calls no
 * allocating routine: its control block and status words live in a fixed
 * 4 MiB array in the library's own device memory, one per GPU, held until the
 * process ends, with room for 32,766 tiles (n up to 1.07G 4-byte and 537M
 * 8-byte elements; DS_ERR_TOO_LARGE beyond). Every call on a GPU shares
 * that GPU's array, so calls that overlap in time on one GPU (different
 * streams, no ordering between them) race and give wrong results; order them
 * on one stream. The first call on a device enqueues a kernel that clears
 * the array. ds_query_timeout reports a give-up of these calls too (once
 * they have finished). Other arguments and errors as scan_exclusive.
 */
int ds_scan_noalloc(int dtype, int inclusive, const void* d_in, void* d_out, int64_t n, hipStream_t stream);

/*
 * Order-preserving stream compaction: writes, in input order, every d_in[i]
 * with (d_in[i] CMP operand) to d_out[0 .. k) and k to *d_num_selected (one
 * int64 in device memory; -1 if the last tile saw a look-back wait give up). "Prefix sum and other parallel patterns", section
 * "Stream compaction" and its first exercise: the write position of a kept
 * element is the exclusive scan of the keep flags, k = pos[n-1] + flag[n-1].
 * Flags, positions and the scan of them stay on chip (one launch).
 *   dtype          one of ds_dtype; comparison in that type's own order
 *                  (signed, unsigned, IEEE: NaN compares false except DS_NE)
 *   d_out          room for n elements; may equal d_in, must not otherwise
 *                  overlap it; elements past k are left untouched
 *   d_num_selected device pointer to one int64_t (written)
 *   n              0 <= n < 2^32
 *   cmp            one of ds_cmp
 *   operand_bits   the operand's bit pattern in the low 4 or 8 bytes
 *                  (e.g. the uint32 bits of a float operand)
 * Returns DS_OK or a ds_status error (DS_ERR_TOO_LARGE for n >= 2^32).
 */
int compact_if(int dtype, const void* d_in, void* d_out, int64_t* d_num_selected, int64_t n,
               int cmp, uint64_t operand_bits, hipStream_t stream);

/* Granularity of the space claims of ds_compact_unordered. */
typedef enum {
    DS_CLAIM_PER_WAVE = 0,     /* one atomic add per 64-lane wave, as the pages' warp-aggregated atomic */
    DS_CLAIM_PER_WORKGROUP = 1 /* the four waves' counts summed in LDS, one atomic add per workgroup */
} ds_claim;

/*
 * Stream compaction that does not keep the input order: d_out[0 .. k) holds
 * every kept element, in an unspecified order, and k goes to
 * *d_num_selected. Each wave ranks its kept elements with a ballot and claims
 * room for them with one atomic add on *d_num_selected ("Prefix sum and other
 * parallel patterns", section "Stream compaction", warp-aggregated atomic).
 * Arguments as compact_if, plus `claim` (ds_claim); d_out must not overlap
 * d_in at all. *d_num_selected is the claim counter, cleared by the call.
 */
int ds_compact_unordered(int dtype, const void* d_in, void* d_out, int64_t* d_num_selected, int64_t n,
                         int cmp, uint64_t operand_bits, int claim, hipStream_t stream);

/*
 * One stable counting-sort pass, the step a radix sort repeats once per digit
 * ("Day 32 -- The CUDA scan algorithm", closing section; "Prefix sum and other
 * parallel patterns", opening paragraph): d_keys_out holds the n uint32 keys
 * ordered by the digit (key >> shift) & (2^bits - 1), keys with equal digits
 * in input order. d_vals_in / d_vals_out (both NULL, or both n uint32
 * values) carry a value with each key. Three launches: digit counts per
 * group of four tiles into a digit-major table (with each later tile's counts
 * within its group), the device-wide exclusive scan of that table, then a
 * stable scatter. Four-byte aligned device pointers; an output may
 * not overlap any other buffer (DS_ERR_OVERLAP), the two inputs may share
 * memory. 1 <= bits <= 8, 0 <= shift,
 * shift + bits <= 32 (else DS_ERR_INVALID_VALUE); n < 2^32 (else
 * DS_ERR_TOO_LARGE). Scratch: 2^bits x (groups + tiles) 32-bit words, a
 * tile being ds_tile_elems(DS_UINT32, DS_TILE_OF_COUNTING_SORT) keys, or
 * DS_TILE_OF_COUNTING_SORT_VALUES with values, and a group four tiles; cached
 * per (device, stream) like the scan workspace.
 */
int ds_radix_pass(const uint32_t* d_keys_in, uint32_t* d_keys_out, const uint32_t* d_vals_in,
                  uint32_t* d_vals_out, int64_t n, int shift, int bits, hipStream_t stream);

/*
 * MoE token alignment ("Prefix sum and other parallel patterns", section "In
 * LLMs: MoE token dispatch" and exercise 2). d_topk_ids: n int32 expert ids,
 * token-major (n = tokens x top_k); an id outside [0, num_experts) is
 * dropped. Writes d_counts[e] = assignments of expert e, d_offsets[0] = 0 and
 * d_offsets[e + 1] = d_offsets[e] + d_counts[e] rounded up to a multiple of
 * `block` (the grouped GEMM's tile), and d_sorted_ids[d_offsets[e] + j] = the
 * index i (into d_topk_ids) of expert e's j-th assignment in input order, the
 * rest of expert e's segment = n (the padding mark). Entries of d_sorted_ids
 * from d_offsets[num_experts] on are not written. The same counting-sort
 * pass as ds_radix_pass with the expert id as the digit (tiles of
 * ds_tile_elems(DS_INT32, DS_TILE_OF_MOE_ALIGN) ids), each scatter workgroup
 * deriving the rounded offsets from the scanned table; up to 8,192 ids, one
 * launch of one workgroup does all of it. 1 <= num_experts <= 511, block >= 1,
 * capacity >= n + num_experts * (block - 1) (else DS_ERR_INVALID_VALUE); that
 * bound < 2^31 (else DS_ERR_TOO_LARGE). Buffers must not overlap.
 */
int ds_moe_align(const int32_t* d_topk_ids, int64_t n, int num_experts, int block, int32_t* d_counts,
                 int32_t* d_offsets, int32_t* d_sorted_ids, int64_t capacity, hipStream_t stream);

/*
 * Copy of nbytes from d_in to d_out with the same launch shape, 16-byte
 * accesses and tile size (128 KiB) as the 4-byte scan: the practical
 * bandwidth ceiling the scan is measured against (the "copy, no scan" row of
 * "Day 32 -- The CUDA scan algorithm", section "Results"). nbytes must be a multiple of 16
 * and both pointers 16-byte aligned; the buffers must not overlap.
 */
int ds_copy(const void* d_in, void* d_out, int64_t nbytes, hipStream_t stream);

/* Access pattern of ds_bandwidth_pattern. */
typedef enum {
    DS_PATTERN_READ = 0,       /* read nbytes (folded on chip; nothing written) */
    DS_PATTERN_WRITE = 1,      /* write nbytes (d_in unused, may be NULL) */
    DS_PATTERN_COPY = 2,       /* read then write each tile (stores may leave as their loads arrive) */
    DS_PATTERN_READ_HALF = 3,  /* read each tile, write its first half contiguously: compaction's bytes
                                  at half kept, with no scan (stores may leave as their loads arrive) */
    DS_PATTERN_READ_HALF_HELD = 4, /* as READ_HALF, but no store leaves before the whole tile has arrived,
                                      as in a single-pass compaction, which stores only after its prefix */
    DS_PATTERN_COPY_HELD = 5   /* as COPY, held the same way: the look-back scan's structure */
} ds_pattern;

/*
 * Bandwidth probe for the ceiling table the scan and the compaction are read
 * against (the "copy, no scan" row of "Day 32 -- The CUDA scan algorithm",
 * section "Results", widened to reads, writes and tile sizes): 256-thread
 * workgroups each move vectors_per_thread (1, 2, 4, 8, 16, 20, 28 or 32) 16-byte
 * vectors per thread with non-temporal accesses. layout 0: each workgroup a
 * contiguous tile, laid out as the scan's (lane l of wave w holds vectors
 * k * 64 + l of the wave's quarter); layout 1: 4 KiB chunks at a 32 KiB
 * stride (8 consecutive workgroups share 8 * vectors_per_thread chunks, the
 * g-th taking every 8th from chunk g % 8). nbytes a multiple of 16, pointers
 * 16-byte aligned, in and out not overlapping. Returns DS_OK or a ds_status
 * error.
 */
int ds_bandwidth_pattern(int mode, int vectors_per_thread, int layout, const void* d_in, void* d_out, int64_t nbytes,
                         hipStream_t stream);

/*
 * The pages' block-scan experiment on gfx950: each 4,096-element tile of d_in
 * is scanned (exclusive) by one 1,024-thread workgroup in LDS with the given
 * ds_tile_variant, and each tile's total goes to d_tile_sums (ceil(n/4096)
 * elements, may be NULL). The tiles are independent: this is a block scan,
 * not a device scan. "Day 32 -- The CUDA scan algorithm: the tree and the
 * three kernels", sections "Two sweeps over one tree" and "The stride doubles,
 * and so does the conflict"; "Day 31 -- CUDA prefix sum, the Hillis-Steele
 * scan", section "Why one array is not enough".
 *   dtype   DS_INT32, DS_UINT32 or DS_FP32 (DS_ERR_UNSUPPORTED_DTYPE otherwise)
 *   d_out   n elements, may equal d_in, must not otherwise overlap it
 *   n       0 <= n < 2^32
 * Other arguments and errors as scan_exclusive.
 */
int ds_tile_scan(int dtype, int variant, const void* d_in, void* d_out, void* d_tile_sums, int64_t n,
                 hipStream_t stream);

/*
 * The pages' three-kernel device scan built on ds_tile_scan: scan every tile
 * and save its total, scan the totals (one workgroup, carried sum), add each
 * tile's offset to every element of the tile. Exclusive; reads and writes the
 * data twice ("Day 32", section "One block scans 4,096. Ten million needs
 * three kernels."). Arguments and errors as ds_tile_scan, without d_tile_sums.
 */
int ds_tile_pipeline(int dtype, int variant, const void* d_in, void* d_out, int64_t n, hipStream_t stream);

/*
 * Waits for `stream` and reports, in *timed_out, whether any look-back wait
 * on this (device, stream) gave up since the last query (1) or not (0), then
 * clears the record. A wait gives up only after the spin limit; the outputs of
 * such a call are not valid. After a give-up it also clears every status word
 * of the workspace (a tile that read the launch number late may have stamped
 * its word with the next one), so later calls start clean. Returns DS_OK or
 * DS_ERR_HIP.
 */
int ds_query_timeout(hipStream_t stream, int* timed_out);

/*
 * Testing hook: the next `count` workspace allocations of any entry point
 * fail with DS_ERR_OUT_OF_MEMORY without calling hipMalloc (count 0 ends
 * it). The environment variable DEVSCAN_FAIL_ALLOCS=count, read at the first
 * allocation, does the same. Returns DS_OK or DS_ERR_INVALID_VALUE (count < 0).
 */
int ds_fail_next_allocations(int count);

/*
 * Sets the number of polls a look-back wait makes before it gives up
 * (default 1 << 20; 0 restores the default). Affects later calls in this
 * process. Small values exist to test the give-up path.
 */
int ds_set_spin_limit(uint32_t polls);

/* Which entry point's tile ds_tile_elems reports. */
typedef enum {
    DS_TILE_OF_SCAN_EXCLUSIVE = 0, /* scan_exclusive, ds_scan look-back exclusive: the large tile,
                                      used past 64 MiB of input (ds_scan_tile_elems for any n) */
    DS_TILE_OF_SCAN_INCLUSIVE = 1, /* scan_inclusive, ds_scan look-back inclusive: same */
    DS_TILE_OF_THREE_PASS = 2,     /* DS_ALGO_THREE_PASS */
    DS_TILE_OF_COMPACT = 3,        /* compact_if */
    DS_TILE_OF_LDS_TILE_SCAN = 4,  /* ds_tile_scan / ds_tile_pipeline (4-byte types only) */
    DS_TILE_OF_COUNTING_SORT = 5,  /* ds_radix_pass without values (4-byte types only) */
    DS_TILE_OF_COUNTING_SORT_VALUES = 6, /* ds_radix_pass with values (4-byte types only) */
    DS_TILE_OF_MOE_ALIGN = 7       /* ds_moe_align above its one-launch size (4-byte types only) */
} ds_tile_of;

/*
 * Elements of `dtype` one workgroup of the given entry point (ds_tile_of)
 * handles: the granularity of its tiles, for callers that size work or
 * tests that aim at tile boundaries. Returns -1 for an invalid dtype or entry.
 */
int64_t ds_tile_elems(int dtype, int entry);

/*
 * Elements per workgroup tile of the look-back scan (scan_exclusive,
 * scan_inclusive, ds_scan look-back) for an input of n elements of `dtype`:
 * 8 sixteen-byte vectors per thread up to 8 MiB of data, 12 up to 32 MiB,
 * 16 up to 64 MiB (where that is below the type's large tile), the type's
 * large tile beyond (so mid-size inputs still spread over many workgroups).
 * `inclusive` 0 or 1. Returns -1 for invalid arguments.
 */
int64_t ds_scan_tile_elems(int dtype, int inclusive, int64_t n);

/* Human-readable name of a ds_status value (static storage). */
const char* ds_status_string(int status);

/* Frees every workspace the library holds, after waiting for the device. */
void ds_release_workspace(void);

/* Library ABI version (2: status values 4-8 renumbered, ds_fail_next_allocations). */
int ds_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DEVSCAN_H */
