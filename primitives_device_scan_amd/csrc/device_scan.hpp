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
//    behind other tiles' transfers: 112 KiB for 4-byte types (fp32 inclusive
//    104 KiB, the largest that does not spill) at 3 workgroups per CU, 144 / 112 KiB for 8-byte types
//    (exclusive / inclusive) at 2 per CU (ScanOcc). Measured at n = 100M:
//    against 96 KiB tiles at 4 per CU, the 4-byte scans 1.5-2.5% faster in all
//    four cases, though the int32 tiles spill 12 bytes per thread (as the 96
//    KiB int32 tile did 24 at 4 per CU), while 120-128 KiB tiles or 2 per CU
//    were slower; against 80 / 64 KiB at 3 per CU, int64 5-6% (exclusive) and
//    7% (inclusive) faster (144 KiB exclusive tiles 1-1.4% faster than 128);
//    8-byte tiles of 96-112 KiB at 3 per CU spill 70-430 bytes and are
//    slower, and 160 KiB at 2 per CU too;
//  - three-pass scan and compaction: 64 KiB tiles (the three-pass scan has no
//    wait to hide; compaction's keep mask holds 64 elements).
template <typename T, bool INCLUSIVE>
struct ScanVPT {
    static constexpr int value = sizeof(T) == 8 ? (INCLUSIVE ? 28 : 36)
                               : __is_same(T, float) ? (INCLUSIVE ? 26 : 28)
                                                     : 28;
};
// Workgroups per CU the look-back kernel is compiled for (waves per SIMD):
// the large 8-byte tiles need up to 256 VGPRs; every other tile fits 3.
template <typename T, int VPT>
struct ScanOcc {
    static constexpr int value = (sizeof(T) == 8 && VPT > 20) ? 2 : 3;
};
constexpr int kVPT = 28;  // largest scan tile: the same-pattern copy uses it
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
