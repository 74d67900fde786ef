// copy.hip -- the scan's access pattern without the scan: the same tile, the
// same 16-byte non-temporal loads and stores. These are the bandwidth
// ceilings the scan and the compaction are read against ("Day 32 -- The CUDA
// scan algorithm", section "Results", copy row).
#include "device_scan.hpp"

namespace ds {

template <int VPT>
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* in, u32x4* out, int64_t nvec)
{
    const int64_t base = (int64_t)blockIdx.x * (kThreads * VPT) +
                         (int64_t)(threadIdx.x / kWave) * (kWave * VPT) + lane_id();
    u32x4 r[VPT];
    if (base + (VPT - 1) * kWave < nvec) {  // whole wave segment: straight-line, as the scan's
#pragma unroll
        for (int k = 0; k < VPT; ++k) r[k] = __builtin_nontemporal_load(in + base + k * kWave);
#pragma unroll
        for (int k = 0; k < VPT; ++k) __builtin_nontemporal_store(r[k], out + base + k * kWave);
        return;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (base + k * kWave < nvec) r[k] = __builtin_nontemporal_load(in + base + k * kWave);
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (base + k * kWave < nvec) __builtin_nontemporal_store(r[k], out + base + k * kWave);
}

hipError_t launch_copy(const void* in, void* out, int64_t nbytes, hipStream_t stream)
{
    const int64_t nvec = nbytes / kVecBytes;
    const int64_t per_block = (int64_t)kThreads * kVPT;
    const int64_t blocks = (nvec + per_block - 1) / per_block;
    copy_kernel<kVPT><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>((const u32x4*)in, (u32x4*)out, nvec);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Access-pattern probes for the ceiling table: one workgroup of 256 threads
// moves VPT 16-byte vectors per thread (VPT * 4 KiB per workgroup).
//   MODE 0 read only (folded into one word, stored only if it equals `magic`)
//        1 write only (a pattern)
//        2 copy: all loads, then all stores (the held tile of a look-back scan)
//        3 compaction-shaped: read the whole tile, write its first half
//          contiguously at out + tile * (tile bytes / 2): the bytes
//          compact_if moves when half the elements are kept, with no scan
//        4 as 3, held: every store depends on a fold of every loaded vector,
//          so no store leaves before the whole tile has arrived (a single-pass
//          compaction cannot store before its prefix, which needs the tile)
//        5 as 2, held the same way (the look-back scan's structure)
//   LAYOUT 0 contiguous tile, lane l of wave w holding vectors k * 64 + l of
//            the wave's quarter (the scan's tile)
//          1 four-KiB chunks at a 32 KiB stride: a group of 8 consecutive
//            workgroups covers 8 * VPT chunks and workgroup g % 8 takes every
//            8th of them (with the round-robin dispatch over the 8 XCDs, each
//            XCD then touches one 4 KiB slot of every 32 KiB)
// ---------------------------------------------------------------------------
template <int MODE, int VPT, int LAYOUT, bool WHOLE>
__device__ __forceinline__ void pattern_body(const u32x4* in, u32x4* out, int64_t nvec, uint32_t magic,
                                             const int64_t (&addr)[VPT])
{
    u32x4 r[VPT];
    if constexpr (MODE == 1) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) r[k] = u32x4{(uint32_t)k, (uint32_t)threadIdx.x, magic, blockIdx.x};
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            r[k] = (WHOLE || addr[k] < nvec) ? __builtin_nontemporal_load(in + addr[k]) : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (MODE == 4 || MODE == 5) {
        // the fold of all VPT vectors gates every store; `magic` never matches real data
        // in a way that matters here (a bandwidth probe: a match flips one bit)
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            if (WHOLE || addr[k] < nvec) acc ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
        const uint32_t z = acc == magic ? 1u : 0u;
        const int64_t half = (int64_t)kThreads * VPT / 2;
        const int64_t dst0 = (int64_t)blockIdx.x * half;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            u32x4 v = r[k];
            v.x ^= z;
            if constexpr (MODE == 4) {
                const int64_t q = (int64_t)k * kThreads + threadIdx.x;
                if (q < half && (WHOLE || (dst0 + q < nvec && addr[k] < nvec)))
                    __builtin_nontemporal_store(v, out + dst0 + q);
            } else {
                if (WHOLE || addr[k] < nvec) __builtin_nontemporal_store(v, out + addr[k]);
            }
        }
        return;
    }
    if constexpr (MODE == 0 || MODE == 3) {
        // every loaded vector not stored below is folded into one word, so no load is dead
        uint32_t acc = 0;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int64_t q = (int64_t)k * kThreads + threadIdx.x;
            if (MODE == 0 || q >= (int64_t)kThreads * VPT / 2) acc ^= r[k].x ^ r[k].y ^ r[k].z ^ r[k].w;
        }
        if (acc == magic) out[0] = u32x4{acc, acc, acc, acc};
        if constexpr (MODE == 0) return;
    }
    if constexpr (MODE == 3) {
        // the first half of the tile (vector q = k * 256 + thread), in order, to the compacted position
        const int64_t half = (int64_t)kThreads * VPT / 2;
        const int64_t dst0 = (int64_t)blockIdx.x * half;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int64_t q = (int64_t)k * kThreads + threadIdx.x;
            if (q < half && (WHOLE || (dst0 + q < nvec && addr[k] < nvec)))
                __builtin_nontemporal_store(r[k], out + dst0 + q);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (WHOLE || addr[k] < nvec) __builtin_nontemporal_store(r[k], out + addr[k]);
}

template <int MODE, int VPT, int LAYOUT>
__global__ __launch_bounds__(kThreads) void pattern_kernel(const u32x4* in, u32x4* out, int64_t nvec, uint32_t magic)
{
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
    int64_t addr[VPT];
    int64_t last;  // one past the largest vector index the workgroup touches
    if constexpr (LAYOUT == 0) {
        const int64_t base = (int64_t)blockIdx.x * (kThreads * VPT) + (int64_t)wave * (kWave * VPT) + lane;
#pragma unroll
        for (int k = 0; k < VPT; ++k) addr[k] = base + (int64_t)k * kWave;
        last = ((int64_t)blockIdx.x + 1) * (kThreads * VPT);
    } else {
        const int64_t group = blockIdx.x / 8, slot = blockIdx.x % 8;
#pragma unroll
        for (int k = 0; k < VPT; ++k) addr[k] = ((group * VPT + k) * 8 + slot) * kThreads + threadIdx.x;
        last = ((group * VPT + VPT - 1) * 8 + slot + 1) * kThreads;
    }
    // whole workgroups take the straight-line path (no per-vector bounds test)
    if (last <= nvec)
        pattern_body<MODE, VPT, LAYOUT, true>(in, out, nvec, magic, addr);
    else
        pattern_body<MODE, VPT, LAYOUT, false>(in, out, nvec, magic, addr);
}

template <int MODE, int VPT>
static hipError_t pattern_launch(int layout, const void* in, void* out, int64_t nvec, hipStream_t st)
{
    const int64_t per = (int64_t)kThreads * VPT;
    int64_t blocks = (nvec + per - 1) / per;
    if (layout == 1) blocks = (blocks + 7) / 8 * 8;  // whole groups of 8 (guarded per vector)
    if (layout == 0)
        pattern_kernel<MODE, VPT, 0><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
            (const u32x4*)in, (u32x4*)out, nvec, 0x9E3779B9u);
    else
        pattern_kernel<MODE, VPT, 1><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
            (const u32x4*)in, (u32x4*)out, nvec, 0x9E3779B9u);
    return hipGetLastError();
}

template <int MODE>
static hipError_t pattern_mode(int vpt, int layout, const void* in, void* out, int64_t nvec, hipStream_t st)
{
    switch (vpt) {
    case 1: return pattern_launch<MODE, 1>(layout, in, out, nvec, st);
    case 2: return pattern_launch<MODE, 2>(layout, in, out, nvec, st);
    case 4: return pattern_launch<MODE, 4>(layout, in, out, nvec, st);
    case 8: return pattern_launch<MODE, 8>(layout, in, out, nvec, st);
    case 16: return pattern_launch<MODE, 16>(layout, in, out, nvec, st);
    case 20: return pattern_launch<MODE, 20>(layout, in, out, nvec, st);
    case 28: return pattern_launch<MODE, 28>(layout, in, out, nvec, st);
    case 32: return pattern_launch<MODE, 32>(layout, in, out, nvec, st);
    default: return hipErrorInvalidValue;
    }
}

bool pattern_vpt_ok(int vpt)
{
    return vpt == 1 || vpt == 2 || vpt == 4 || vpt == 8 || vpt == 16 || vpt == 20 || vpt == 28 || vpt == 32;
}

hipError_t launch_pattern(int mode, int vpt, int layout, const void* in, void* out, int64_t nbytes,
                          hipStream_t stream)
{
    const int64_t nvec = nbytes / kVecBytes;
    switch (mode) {
    case 0: return pattern_mode<0>(vpt, layout, in, out, nvec, stream);
    case 1: return pattern_mode<1>(vpt, layout, in, out, nvec, stream);
    case 2: return pattern_mode<2>(vpt, layout, in, out, nvec, stream);
    case 3: return pattern_mode<3>(vpt, layout, in, out, nvec, stream);
    case 4: return pattern_mode<4>(vpt, layout, in, out, nvec, stream);
    default: return pattern_mode<5>(vpt, layout, in, out, nvec, stream);
    }
}

int64_t tile_bytes() { return kTileBytes; }
int64_t three_pass_tile_elems(int elem_bytes) { return (int64_t)kThreads * kThreePassVPT * kVecBytes / elem_bytes; }
int64_t compact_tile_elems(int elem_bytes) { return (int64_t)kThreads * kCompactVPT * kVecBytes / elem_bytes; }

}  // namespace ds
