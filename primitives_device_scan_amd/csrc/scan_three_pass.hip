// scan_three_pass.hip -- the device-wide scan in three launches: tile totals,
// an exclusive scan of the totals in one workgroup with a carried sum, and a
// rescan of each tile seeded with its offset ("Day 32 -- The CUDA scan
// algorithm", section "One block scans 4,096. Ten million needs three
// kernels.", in reduce-then-scan form: the first pass only reads).
#include "device_scan.hpp"

namespace ds {

template <typename T, bool A16>
__global__ __launch_bounds__(kThreads) void tile_reduce_kernel(const T* in, int64_t n, T* totals)
{
    using S = Shape<T, kThreePassVPT>;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    T e[S::kItems];
    if (seg + S::kWaveElems <= n)  // whole wave: 16-byte vectors, 16-byte aligned or not (A16)
        load_vec<T, kThreePassVPT, A16>(in, seg, lane, e);
    else
        load_scalar<T, kThreePassVPT>(in, seg, n, lane, e, T(0));
    T s = T(0);
#pragma unroll
    for (int i = 0; i < S::kItems; ++i) s = s + e[i];
    s = wave_sum(s);
    if (lane == 0) s_wave[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        T t = T(0);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t = t + s_wave[w];
        totals[tile] = t;
    }
}

// Exclusive scan of `count` tile totals in place by one workgroup of 1,024
// threads, 1,024 totals per round, the running sum carried between rounds.
constexpr int kTotalsThreads = 1024;

template <typename T>
__global__ __launch_bounds__(kTotalsThreads) void scan_totals_kernel(T* totals, int64_t count)
{
    constexpr int kW = kTotalsThreads / kWave;
    __shared__ T s_wave[kW];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    T carry = T(0);
    for (int64_t start = 0; start < count; start += kTotalsThreads) {
        const int64_t i = start + threadIdx.x;
        const T v = i < count ? totals[i] : T(0);
        const T incl = wave_inclusive_scan(v);
        if (lane == kWave - 1) s_wave[wave] = incl;
        __syncthreads();
        T before = T(0), round = T(0);
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            const T t = s_wave[w];
            if (w < wave) before = before + t;
            round = round + t;
        }
        if (i < count) totals[i] = carry + (before + wave_shift_right1(incl));
        carry = carry + round;
        __syncthreads();
    }
}

template <typename T, bool INCLUSIVE, bool A16>
__global__ __launch_bounds__(kThreads) void tile_rescan_kernel(const T* in, T* out, int64_t n,
                                                                const T* offsets)
{
    using S = Shape<T, kThreePassVPT>;
    constexpr int V = S::kPerVec;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, kThreePassVPT, A16>(in, seg, lane, e);
    else
        load_scalar<T, kThreePassVPT>(in, seg, n, lane, e, T(0));
    // The sums of the waves before this one come from a reduction first, so
    // each vector can be stored as soon as it is scanned.
    T wave_excl;
    (void)tile_reduce<T, S::kItems>(e, wave_excl, s_wave);
    const T head = offsets[tile] + wave_excl;
    if (whole) {
        scan_store_vec<T, V, kThreePassVPT, INCLUSIVE, A16>(out, seg, lane, e, head);
    } else {
        scan_in_wave<T, V, kThreePassVPT, INCLUSIVE>(e);
        add_uniform(e, head);
        store_scalar<T, kThreePassVPT>(out, seg, n, lane, e);
    }
}

template <typename T, bool A16>
static hipError_t three_pass_typed(bool incl, const void* in, void* out, int64_t n, const DevWs& ws,
                                   hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, kThreePassVPT>::kTile - 1) / Shape<T, kThreePassVPT>::kTile;
    if (!ws.totals) return hipErrorInvalidValue;
    T* totals = (T*)ws.totals;
    tile_reduce_kernel<T, A16><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>((const T*)in, n, totals);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scan_totals_kernel<T><<<dim3(1), dim3(kTotalsThreads), 0, st>>>(totals, tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (incl)
        tile_rescan_kernel<T, true, A16><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, n, totals);
    else
        tile_rescan_kernel<T, false, A16><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, n, totals);
    return hipGetLastError();
}

template <typename T>
static hipError_t three_pass_dispatch(bool incl, const void* in, void* out, int64_t n, const DevWs& ws,
                                      hipStream_t st)
{
    return (aligned16(in) && aligned16(out)) ? three_pass_typed<T, true>(incl, in, out, n, ws, st)
                                             : three_pass_typed<T, false>(incl, in, out, n, ws, st);
}

hipError_t launch_three_pass_scan(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                  const DevWs& ws, hipStream_t stream)
{
    switch (kind) {
    case kF32: return three_pass_dispatch<float>(inclusive, in, out, n, ws, stream);
    case kU64:
    case kI64: return three_pass_dispatch<uint64_t>(inclusive, in, out, n, ws, stream);
    default: return three_pass_dispatch<uint32_t>(inclusive, in, out, n, ws, stream);
    }
}

hipError_t launch_scan_totals(ElemKind kind, void* totals, int64_t count, hipStream_t stream)
{
    if (!totals) return hipErrorInvalidValue;
    const dim3 grid(1), block(kTotalsThreads);
    switch (kind) {
    case kF32: scan_totals_kernel<float><<<grid, block, 0, stream>>>((float*)totals, count); break;
    case kU64:
    case kI64: scan_totals_kernel<uint64_t><<<grid, block, 0, stream>>>((uint64_t*)totals, count); break;
    default: scan_totals_kernel<uint32_t><<<grid, block, 0, stream>>>((uint32_t*)totals, count); break;
    }
    return hipGetLastError();
}

}  // namespace ds
