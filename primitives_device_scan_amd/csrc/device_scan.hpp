// device_scan.hpp -- shared by the device-level kernels: tile size, the launch
// order that the look-back relies on, the launch epoch, and the exclusive
// prefix of a tile found by wave 0.
#pragma once

#include "launch.hpp"
#include "tile.hpp"

namespace ds {

// 16-byte vectors per thread (VPT); a tile is 256 threads x VPT x 16 B.
//  - look-back scan: large tiles, since resident tile bytes per CU are what
//    hide the look-back latency (several microseconds under full HBM load)
//    behind other tiles' transfers. 4-byte types: 128 KiB tiles (32 vectors
//    per thread, 204-211 VGPRs, no spill) at 2 workgroups per CU. Measured on
//    MI355X at n = 100M with the status words padded to a line each and the
//    scanned values pinned before the look-back (scan_lookback.hip): 136-138 us
//    after a cache eviction for int32 and fp32 alike, against 139-141 us for
//    80 KiB tiles at 3 per CU, the earlier choice; 112 and 144 KiB tiles took
//    141-143 us, and 112 KiB at 3 per CU spills. A held copy shows the same
//    order: 135 us at 128 KiB and 2 per CU, 143-144 us at 80-112 KiB and 3-4.
//    8-byte types take the same 128 KiB tile (16,384 elements, 166 VGPRs, no
//    spill) at 2 per CU (ScanOcc); 96-112 KiB at 3 per CU spill and were
//    slower. With the prefix added and stored one vector at a time, n = 50M
//    after a cache eviction: exclusive 136-139 us against 141-143 us for the
//    earlier 144 KiB tile, inclusive 137-138 us against 141-143 us at 112 KiB;
//  - three-pass scan and compaction: 64 KiB tiles (the three-pass scan has no
//    wait to hide; compaction's keep mask holds 64 elements).
template <typename T, bool INCLUSIVE>
struct ScanVPT {
    static constexpr int value = 32;
};
// Workgroups per CU the look-back kernel is compiled for (waves per SIMD):
// tiles past 80 KiB need up to 256 VGPRs; every other tile fits 3.
template <typename T, int VPT>
struct ScanOcc {
    static constexpr int value = (VPT > 20 && (sizeof(T) == 8 || VPT > 28)) ? 2 : 3;
};
constexpr int kVPT = 32;  // the 4-byte scan tile: the same-pattern copy (ds_copy) uses it
constexpr int kThreePassVPT = 16;
constexpr int kCompactVPT = 16;
constexpr int kCompactOcc = 4;  // workgroups per CU the ordered compaction is compiled for
constexpr int kTileBytes = kThreads * kVPT * kVecBytes;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Tile order and forward progress. Tile t is workgroup t (blockIdx.x) and
// waits only for tiles below t. Workgroups are dispatched in increasing index
// order (round-robin over the XCDs, in order within each), so the lowest
// unfinished tile is always running or next to start, and every wait ends.
// A shared atomic ticket counter would make the order explicit, but every
// workgroup's fetch-and-add on one address serialises at roughly 50 ns each
// on this GPU -- over a millisecond for 24,415 tiles -- so the order of the
// launch is used instead, and the bounded wait in `lookback` backs it up.

__device__ __forceinline__ void flag_timeout(Ctrl* ctrl)
{
    if (ctrl) __hip_atomic_store(&ctrl->timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by lane 0 of the last tile once it has published its inclusive
// prefix. Every other tile has by then published a status stamped with the
// epoch it read (the last tile's prefix depends on all of them), so the epoch
// can be advanced for the next launch.
__device__ __forceinline__ void end_of_launch(Ctrl* ctrl, uint32_t epoch)
{
    __hip_atomic_store(&ctrl->epoch, (epoch + 1u) & kEpochMask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t launch_epoch(Ctrl* ctrl)
{
    return __hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Read of the tile's own status line as the tile starts, long before the
// tile publishes into it: the line is then fetched while the tile's data
// loads, and the publish and its successors' polls find it nearby. Measured
// at n = 100M (int32 exclusive, 112 KiB tiles) the whole scan is 1-2% faster,
// most after a cache eviction. The value is unused; keep_alive() consumes it
// at the end of the kernel so the load is not dropped.
__device__ __forceinline__ uint64_t touch_status(uint64_t* status, int64_t tile)
{
    return status_load(status + tile * kStatusWords);
}

__device__ __forceinline__ void keep_alive(uint64_t v) { asm volatile("" ::"v"(v)); }

// Called by one thread as soon as the tile aggregate is known: tile 0
// publishes its inclusive prefix `first + agg` (first: 0, or the seed of a
// seeded scan), every other tile its aggregate, so successors can use it
// while this tile still scans its own elements.
template <typename T>
__device__ __forceinline__ void publish_early(uint64_t* status, int64_t tile, uint32_t epoch, T agg, T first)
{
    if (tile == 0)
        StatusCodec<T>::publish(status, 0, epoch, kFlagPrefix, first + agg);
    else
        StatusCodec<T>::publish(status, tile, epoch, kFlagAggregate, agg);
}

// The exclusive prefix of `tile`, found by wave 0 and shared through LDS.
// Tile 0's prefix is `first` (0, or the seed of a seeded scan); unless
// `published` (publish_early has run), it publishes first + aggregate as its
// inclusive prefix at once.
template <typename T>
__device__ __forceinline__ T tile_prefix(int64_t tile, int64_t num_tiles, uint32_t epoch, T agg, Ctrl* ctrl,
                                         uint64_t* status, uint32_t spin_limit, T first = T(0),
                                         bool published = false)
{
    __shared__ T s_prefix;
    if (threadIdx.x < kWave) {
        T p = T(0);
        if (tile == 0) {
            p = first;
            if (threadIdx.x == 0 && !published) StatusCodec<T>::publish(status, 0, epoch, kFlagPrefix, first + agg);
        } else {
            p = lookback<T>(status, tile, epoch, agg, spin_limit, &ctrl->timeout, published);
        }
        if (threadIdx.x == 0) {
            s_prefix = p;
            if (tile == num_tiles - 1) end_of_launch(ctrl, epoch);
        }
    }
    __syncthreads();
    return s_prefix;
}

}  // namespace ds
