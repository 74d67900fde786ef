// copy.hip -- the scan's access pattern without the scan (same tile, same
// 16-byte non-temporal loads and stores): the bandwidth ceiling the scan is
// compared with ("Day 32 -- The CUDA scan algorithm", section "Results",
// copy row).
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

int64_t tile_bytes() { return kTileBytes; }
int64_t three_pass_tile_elems(int elem_bytes) { return (int64_t)kThreads * kThreePassVPT * kVecBytes / elem_bytes; }
int64_t compact_tile_elems(int elem_bytes) { return (int64_t)kThreads * kCompactVPT * kVecBytes / elem_bytes; }

}  // namespace ds
