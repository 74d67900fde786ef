// device_scan.hpp -- shared by the device-level kernels: tile size, the launch
// order that the look-back relies on, the launch epoch, and the exclusive
// prefix of a tile found by wave 0.
#pragma once

#include "launch.hpp"
#include "tile.hpp"

namespace ds {

// 16-byte vectors per thread (VPT); a tile is 256 threads x VPT x 16 B.
//  - look-back scan: the largest tile that fits its occupancy (ScanOcc
//    below) without spilling (ScanVPT), since resident tile bytes per CU are
//    what hide the look-back latency (several microseconds under full HBM
//    load) behind other tiles' transfers: 96 KiB for int32 and fp32
//    exclusive, 80 KiB inclusive, 80 / 64 KiB for 8-byte types;
//  - three-pass scan and compaction: 64 KiB tiles (the three-pass scan has no
//    wait to hide; compaction's keep mask holds 64 elements).
template <typename T, bool INCLUSIVE>
struct ScanVPT {
    static constexpr int value = sizeof(T) == 8 ? (INCLUSIVE ? 16 : 20)
                               : __is_same(T, float) ? (INCLUSIVE ? 20 : 24)
                                                     : (INCLUSIVE ? 20 : 24);
};
// Workgroups per CU the look-back kernel is compiled for (waves per SIMD):
// 4 for 4-byte integers (their tiles fit 128 VGPRs); fp32 and 8-byte scans
// need more registers per vector and hold larger tiles at 3 (measured: 1-2%
// faster for fp32, 5-6% for 8-byte than their 4-wave tiles).
template <typename T>
struct ScanOcc {
    static constexpr int value = (sizeof(T) == 8 || __is_same(T, float)) ? 3 : 4;
};
constexpr int kVPT = 24;  // largest scan tile: the same-pattern copy uses it
constexpr int kThreePassVPT = 16;
constexpr int kCompactVPT = 16;
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

// The exclusive prefix of `tile`, found by wave 0 and shared through LDS.
// Tile 0's prefix is `first` (0, or the seed of a seeded scan); it publishes
// first + aggregate as its inclusive prefix at once.
template <typename T>
__device__ __forceinline__ T tile_prefix(int64_t tile, int64_t num_tiles, uint32_t epoch, T agg, Ctrl* ctrl,
                                         uint64_t* status, uint32_t spin_limit, T first = T(0))
{
    __shared__ T s_prefix;
    if (threadIdx.x < kWave) {
        T p = T(0);
        if (tile == 0) {
            p = first;
            if (threadIdx.x == 0) StatusCodec<T>::publish(status, 0, epoch, kFlagPrefix, first + agg);
        } else {
            p = lookback<T>(status, tile, epoch, agg, spin_limit, &ctrl->timeout);
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
