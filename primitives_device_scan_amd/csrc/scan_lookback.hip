// scan_lookback.hip -- the single-pass device-wide scan: each tile sums
// itself and publishes its aggregate, scans itself in registers while that
// status travels, looks back over the status of earlier tiles for its
// exclusive prefix, publishes its inclusive prefix and writes ("Prefix sum and
// other parallel patterns", section "A device-level scan: scan then
// propagate", decoupled look-back).
#include "device_scan.hpp"

namespace ds {

template <typename T, bool INCLUSIVE, bool A16, int VPT>
__global__ __launch_bounds__(kThreads, (ScanOcc<T, VPT>::value)) void lookback_scan_kernel(const T* in, T* out, int64_t n,
                                                                  int64_t num_tiles, Ctrl* ctrl,
                                                                  uint64_t* status, uint32_t spin_limit,
                                                                  const T* seed)
{
    using S = Shape<T, VPT>;
    constexpr int V = S::kPerVec;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);

    const int64_t tile = blockIdx.x;
    // Only wave 0 publishes and looks back; its epoch load overlaps the data loads.
    const uint32_t epoch = (num_tiles > 1 && wave == 0) ? launch_epoch(ctrl) : 0u;
    uint64_t touched = 0;
    if (num_tiles > 1 && threadIdx.x == 0) touched = touch_status(status, tile);

    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    // Whole waves take 16-byte vectors whatever the alignment (A16: in and out
    // are 16-byte aligned); the ragged end goes element by element.
    const bool whole = seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, VPT, A16>(in, seg, lane, e);
    else
        load_scalar<T, VPT>(in, seg, n, lane, e, T(0));

    // The aggregate comes from a reduction and is published at once; the tile
    // then scans its elements while the status travels, and wave 0 looks back.
    // (Publishing after the full in-register scan instead made every
    // successor's look-back wait for that scan: 1.5-2.6% slower at 100M.)
    T wave_excl;
    const T agg = tile_reduce<T, S::kItems>(e, wave_excl, s_wave);
    // A seeded scan starts from *seed (the sum of everything before this
    // input, e.g. earlier shards); only tile 0 reads it, the look-back carries it on.
    const T first = (seed != nullptr && tile == 0) ? *seed : T(0);
    if (num_tiles > 1 && threadIdx.x == 0) publish_early<T>(status, tile, epoch, agg, first);
    scan_in_wave<T, V, VPT, INCLUSIVE>(e);
    // Left to itself the compiler sinks the integer scan's last additions past
    // the wait below, into the prefix add (v_add3); done after the prefix
    // arrives, they delay the stores: int32 at n = 100M took 140.0-140.6 us
    // cold that way against 136.8-138.0 us pinned. (The 8-byte exclusive tile
    // takes the same time pinned, in 166 VGPRs rather than 255.)
    pin_in_registers(e);
    const T prefix =
        num_tiles > 1 ? tile_prefix<T>(tile, num_tiles, epoch, agg, ctrl, status, spin_limit, first, true) : first;
    // The prefix is added and each vector stored in turn, so the tile's
    // stores begin after one vector's additions rather than all of them and
    // the tile is held that much less. Cold, 800 MB of input: int32 (n = 100M)
    // 138.7-140.5 -> 133.2-134.8 us, fp32 135.9-136.7 -> 133.3-134.4; int64
    // (n = 50M, with 128 KiB tiles in place of 144 / 112 KiB) exclusive
    // 141.3-143.2 -> 136.3-139.1, inclusive 140.6-142.5 -> 136.9-137.9.
    if (whole) {
        add_store_vec<T, VPT, A16>(out, seg, lane, e, prefix + wave_excl);
    } else {
        add_uniform(e, prefix + wave_excl);
        store_scalar<T, VPT>(out, seg, n, lane, e);
    }
    if (threadIdx.x == 0) keep_alive(touched);
}

// Vectors per thread for n elements: the per-type large tile (ScanVPT) from
// 64 MiB of data on, where resident bytes must hide the look-back; below, a
// large tile would leave most CUs idle (1M int32 fill 31 workgroups of 128 KiB)
// and a small last tile costs element-wise loads, so inputs up to 8 MiB take
// 8 vectors per thread, up to 32 MiB 12 and up to 64 MiB 16 (measured: one
// 4,096-int32 tile 7.9 -> 3.8 us, 1M int32 10.0 -> 5.6 us, 8M int32 14.5 ->
// 13.5 us, 12M fp32 inclusive 19.6 -> 17.7 us per launch back to back; from
// 30M int32 on the large tile is fastest).
constexpr int kSmallScanVPT = 8;
constexpr int kMidScanVPT = 12;
constexpr int kUpperScanVPT = 16;

template <typename T, bool INCL>
static int lookback_vpt(int64_t n)
{
    const int64_t bytes = n * (int64_t)sizeof(T);
    if (bytes <= ((int64_t)8 << 20)) return kSmallScanVPT;
    if (bytes <= ((int64_t)32 << 20)) return kMidScanVPT;
    if (bytes <= ((int64_t)64 << 20) && kUpperScanVPT < ScanVPT<T, INCL>::value) return kUpperScanVPT;
    return ScanVPT<T, INCL>::value;
}

template <typename T, bool INCL, bool A16, int VPT>
static hipError_t lookback_launch(const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin,
                                  const void* seed, hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, VPT>::kTile - 1) / Shape<T, VPT>::kTile;
    if (tiles > 1 && (!ws.ctrl || !ws.status)) return hipErrorInvalidValue;  // several tiles need a workspace
    lookback_scan_kernel<T, INCL, A16, VPT><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
        (const T*)in, (T*)out, n, tiles, ws.ctrl, ws.status, spin, (const T*)seed);
    return hipGetLastError();
}

template <typename T, bool INCL, bool A16>
static hipError_t lookback_typed(const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin,
                                 const void* seed, hipStream_t st)
{
    switch (lookback_vpt<T, INCL>(n)) {
    case kSmallScanVPT: return lookback_launch<T, INCL, A16, kSmallScanVPT>(in, out, n, ws, spin, seed, st);
    case kMidScanVPT: return lookback_launch<T, INCL, A16, kMidScanVPT>(in, out, n, ws, spin, seed, st);
    case kUpperScanVPT: return lookback_launch<T, INCL, A16, kUpperScanVPT>(in, out, n, ws, spin, seed, st);
    default: return lookback_launch<T, INCL, A16, ScanVPT<T, INCL>::value>(in, out, n, ws, spin, seed, st);
    }
}

template <typename T>
static hipError_t lookback_dispatch(bool incl, const void* in, void* out, int64_t n, const DevWs& ws,
                                    uint32_t spin, const void* seed, hipStream_t st)
{
    const bool a16 = aligned16(in) && aligned16(out);
    if (incl)
        return a16 ? lookback_typed<T, true, true>(in, out, n, ws, spin, seed, st)
                   : lookback_typed<T, true, false>(in, out, n, ws, spin, seed, st);
    return a16 ? lookback_typed<T, false, true>(in, out, n, ws, spin, seed, st)
               : lookback_typed<T, false, false>(in, out, n, ws, spin, seed, st);
}

hipError_t launch_lookback_scan(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                const DevWs& ws, uint32_t spin_limit, hipStream_t stream, const void* seed)
{
    switch (kind) {
    case kF32: return lookback_dispatch<float>(inclusive, in, out, n, ws, spin_limit, seed, stream);
    case kU64:
    case kI64: return lookback_dispatch<uint64_t>(inclusive, in, out, n, ws, spin_limit, seed, stream);
    default: return lookback_dispatch<uint32_t>(inclusive, in, out, n, ws, spin_limit, seed, stream);
    }
}

template <typename T>
static int64_t tile_of(bool inclusive, int64_t n)
{
    const int vpt = inclusive ? lookback_vpt<T, true>(n) : lookback_vpt<T, false>(n);
    return (int64_t)kThreads * vpt * (kVecBytes / (int)sizeof(T));
}

int64_t tile_elems(ElemKind kind, bool inclusive, int64_t n)
{
    switch (kind) {
    case kF32: return tile_of<float>(inclusive, n);
    case kU64:
    case kI64: return tile_of<uint64_t>(inclusive, n);
    default: return tile_of<uint32_t>(inclusive, n);
    }
}

}  // namespace ds
