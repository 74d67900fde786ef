// scan_blocked.hip -- the look-back scan with the tile transposed through LDS
// (the blocked layout): each wave loads its segment with coalesced 16-byte
// loads, writes it to LDS and reads it back so that each lane holds a
// contiguous run of elements. A lane then scans its run serially and the wave
// needs one 64-lane scan for all of it, where the striped layout of
// scan_lookback.hip needs one per 16-byte vector. The transpose moves 16-byte
// vectors, and each lane's run of VPT vectors is followed by one pad vector:
// a lane's run starts VPT + 1 vectors after its neighbour's, an odd stride,
// so eight lanes of a 16-byte access (the 128 bytes the 32 banks of 4 bytes
// serve at once) land in eight different bank groups both ways (measured:
// SQ_LDS_BANK_CONFLICT; word padding i -> i + i/32, built for the pages'
// power-of-two strides, left 768 conflict cycles per tile on this one). This
// is the tile layout the pages' block scans use ("Day 32 --
// The CUDA scan algorithm", section "The stride doubles, and so does the
// conflict"; "Parallel Prefix Sum (Scan) for NVIDIA T4 (sm_75)", section "How
// It Works"), kept as a measured alternative to the striped layout; the
// device-level part is the same decoupled look-back ("Prefix sum and other
// parallel patterns", section "A device-level scan: scan then propagate").
// 4-byte types only.
#include "device_scan.hpp"

namespace ds {

// Vectors per thread: 12 (48 KiB tiles, 3 workgroups per CU: the staging
// buffer takes 52 KiB of LDS per workgroup), 8 up to 8 MiB of input.
constexpr int kBlockedVPT = 12;
constexpr int kBlockedSmallVPT = 8;

__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// 16-byte vector v of a wave's segment (v = k * 64 + lane in the striped
// layout, v = lane * VPT + q in the blocked one) -> its slot in LDS.
template <int VPT>
__device__ __forceinline__ int slot(int v) { return v + v / VPT; }

template <typename T, bool INCLUSIVE, bool A16, int VPT>
__global__ __launch_bounds__(kThreads, 3) void lookback_blocked_kernel(const T* in, T* out, int64_t n,
                                                                       int64_t num_tiles, Ctrl* ctrl,
                                                                       uint64_t* status, uint32_t spin_limit)
{
    static_assert(sizeof(T) == 4, "4-byte types");
    using S = Shape<T, VPT>;
    constexpr int V = S::kPerVec;
    constexpr int C = S::kItems;                 // contiguous elements per lane after the transpose
    constexpr int WE = S::kWaveElems;            // elements per wave segment (64 * C)
    constexpr int WSLOTS = kWave * (VPT + 1);    // 16-byte slots per wave, pads included
    __shared__ u32x4 s_stage[kWaves * WSLOTS];
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const uint32_t epoch = (num_tiles > 1 && wave == 0) ? launch_epoch(ctrl) : 0u;
    uint64_t touched = 0;
    if (num_tiles > 1 && threadIdx.x == 0) touched = touch_status(status, tile);

    const int64_t seg = tile * S::kTile + (int64_t)wave * WE;
    const bool whole = seg + WE <= n;
    T e[C];
    if (whole)
        load_vec<T, VPT, A16>(in, seg, lane, e);
    else
        load_scalar<T, VPT>(in, seg, n, lane, e, T(0));

    // striped -> blocked through this wave's part of LDS, 16 bytes at a time
    u32x4* st = s_stage + wave * WSLOTS;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        u32x4 v;
        __builtin_memcpy(&v, &e[k * V], kVecBytes);
        st[slot<VPT>(k * kWave + lane)] = v;
    }
    wave_lds_order();
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        const u32x4 v = st[slot<VPT>(lane * VPT + q)];
        __builtin_memcpy(&e[q * V], &v, kVecBytes);
    }

    // the aggregate first (published at once), then the scan
    T sum = T(0);
#pragma unroll
    for (int c = 0; c < C; ++c) sum = sum + e[c];
    const T wsum = wave_sum(sum);
    if (lane == 0) s_wave[wave] = wsum;
    __syncthreads();
    T agg = T(0), wave_excl = T(0);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const T x = s_wave[w];
        if (w < wave) wave_excl = wave_excl + x;
        agg = agg + x;
    }
    if (num_tiles > 1 && threadIdx.x == 0) publish_early<T>(status, tile, epoch, agg, T(0));

#pragma unroll
    for (int c = 1; c < C; ++c) e[c] = e[c] + e[c - 1];
    const T lane_excl = wave_shift_right1(wave_inclusive_scan(e[C - 1]));
    const T prefix = num_tiles > 1 ? tile_prefix<T>(tile, num_tiles, epoch, agg, ctrl, status, spin_limit, T(0), true)
                                   : T(0);
    const T head = prefix + wave_excl + lane_excl;
    if constexpr (INCLUSIVE) {
#pragma unroll
        for (int c = 0; c < C; ++c) e[c] = head + e[c];
    } else {
#pragma unroll
        for (int c = C - 1; c > 0; --c) e[c] = head + e[c - 1];
        e[0] = head;
    }

    // blocked -> striped, then coalesced stores
    wave_lds_order();
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
        u32x4 v;
        __builtin_memcpy(&v, &e[q * V], kVecBytes);
        st[slot<VPT>(lane * VPT + q)] = v;
    }
    wave_lds_order();
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const u32x4 v = st[slot<VPT>(k * kWave + lane)];
        __builtin_memcpy(&e[k * V], &v, kVecBytes);
    }
    if (whole)
        store_vec<T, VPT, A16>(out, seg, lane, e);
    else
        store_scalar<T, VPT>(out, seg, n, lane, e);
    if (threadIdx.x == 0) keep_alive(touched);
}

static int blocked_vpt(int64_t n)
{
    return n * 4 <= ((int64_t)8 << 20) ? kBlockedSmallVPT : kBlockedVPT;
}

int64_t blocked_tile_elems(int64_t n) { return (int64_t)kThreads * blocked_vpt(n) * 4; }

template <typename T, bool INCL, bool A16, int VPT>
static hipError_t blocked_launch(const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin, hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, VPT>::kTile - 1) / Shape<T, VPT>::kTile;
    if (tiles > 1 && (!ws.ctrl || !ws.status)) return hipErrorInvalidValue;  // several tiles need a workspace
    lookback_blocked_kernel<T, INCL, A16, VPT><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
        (const T*)in, (T*)out, n, tiles, ws.ctrl, ws.status, spin);
    return hipGetLastError();
}

template <typename T, bool INCL, bool A16>
static hipError_t blocked_typed(const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin, hipStream_t st)
{
    return blocked_vpt(n) == kBlockedSmallVPT ? blocked_launch<T, INCL, A16, kBlockedSmallVPT>(in, out, n, ws, spin, st)
                                              : blocked_launch<T, INCL, A16, kBlockedVPT>(in, out, n, ws, spin, st);
}

template <typename T>
static hipError_t blocked_dispatch(bool incl, const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin,
                                   hipStream_t st)
{
    const bool a16 = aligned16(in) && aligned16(out);
    if (incl)
        return a16 ? blocked_typed<T, true, true>(in, out, n, ws, spin, st)
                   : blocked_typed<T, true, false>(in, out, n, ws, spin, st);
    return a16 ? blocked_typed<T, false, true>(in, out, n, ws, spin, st)
               : blocked_typed<T, false, false>(in, out, n, ws, spin, st);
}

hipError_t launch_lookback_blocked(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                   const DevWs& ws, uint32_t spin_limit, hipStream_t stream)
{
    switch (kind) {
    case kF32: return blocked_dispatch<float>(inclusive, in, out, n, ws, spin_limit, stream);
    case kU32:
    case kI32: return blocked_dispatch<uint32_t>(inclusive, in, out, n, ws, spin_limit, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ds
