// kernels.hip -- gfx950 kernels of the device-wide scan and compaction, and
// their host launchers.
//
//   lookback_scan_kernel   single pass: each tile scans itself in registers,
//                          publishes its aggregate, looks back over the status
//                          of earlier tiles for its exclusive prefix, publishes
//                          its inclusive prefix, writes ("Prefix sum and other
//                          parallel patterns", section "A device-level scan:
//                          scan then propagate", decoupled look-back).
//   tile_reduce_kernel,    three passes: tile totals, an exclusive scan of the
//   scan_totals_kernel,    totals in one workgroup with a carried sum, and a
//   tile_rescan_kernel     rescan of each tile seeded with its offset ("Day 32
//                          -- The CUDA scan algorithm", section "One block
//                          scans 4,096. Ten million needs three kernels.", in
//                          reduce-then-scan form: the first pass only reads).
//   compact_kernel         order-preserving compaction in one pass: keep flags
//                          counted per tile, the counts scanned with the same
//                          look-back, kept elements staged in LDS at their
//                          rank and written out contiguously ("Prefix sum and
//                          other parallel patterns", section "Stream
//                          compaction", first exercise, fused form).
//   copy_kernel            same access pattern without the scan: the
//                          bandwidth ceiling the scan is compared with.
#include "launch.hpp"
#include "tile.hpp"

namespace ds {

// 16-byte vectors per thread: a scan tile is 256 threads x 16 x 16 B = 64 KiB
// (16,384 four-byte or 8,192 eight-byte elements). Large tiles keep enough
// bytes resident per CU for the look-back latency (several microseconds
// under full HBM load) to hide behind other tiles' transfers. Compaction
// stages its kept elements in LDS, so it uses 16 KiB tiles.
constexpr int kVPT = 16;
constexpr int kCompactVPT = 4;
constexpr int kTileBytes = kThreads * kVPT * kVecBytes;

namespace {

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
// Tile 0 publishes its aggregate as its inclusive prefix at once.
template <typename T>
__device__ __forceinline__ T tile_prefix(int64_t tile, int64_t num_tiles, uint32_t epoch, T agg, Ctrl* ctrl,
                                         uint64_t* status, uint32_t spin_limit)
{
    __shared__ T s_prefix;
    if (threadIdx.x < kWave) {
        T p = T(0);
        if (tile == 0) {
            if (threadIdx.x == 0) StatusCodec<T>::publish(status, 0, epoch, kFlagPrefix, agg);
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

}  // namespace

template <typename T, bool INCLUSIVE, bool VEC, int VPT>
__global__ __launch_bounds__(kThreads) void lookback_scan_kernel(const T* in, T* out, int64_t n,
                                                                  int64_t num_tiles, Ctrl* ctrl,
                                                                  uint64_t* status, uint32_t spin_limit)
{
    using S = Shape<T, VPT>;
    constexpr int V = S::kPerVec;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);

    const int64_t tile = blockIdx.x;
    // Only wave 0 publishes and looks back; its epoch load overlaps the data loads.
    const uint32_t epoch = (num_tiles > 1 && wave == 0) ? launch_epoch(ctrl) : 0u;

    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = VEC && seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, VPT>(in, seg, lane, e);
    else
        load_scalar<T, VPT>(in, seg, n, lane, e, T(0));

    T off[VPT];
    T wave_excl;
    const T agg = tile_local_scan<T, V, VPT>(e, off, wave_excl, s_wave);
    const T prefix =
        num_tiles > 1 ? tile_prefix<T>(tile, num_tiles, epoch, agg, ctrl, status, spin_limit) : T(0);
    tile_finish<T, V, VPT, INCLUSIVE>(e, off, wave_excl, prefix);

    if (whole)
        store_vec<T, VPT>(out, seg, lane, e);
    else
        store_scalar<T, VPT>(out, seg, n, lane, e);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void tile_reduce_kernel(const T* in, int64_t n, T* totals)
{
    using S = Shape<T, kVPT>;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    T e[S::kItems];
    if (VEC && seg + S::kWaveElems <= n)
        load_vec<T, kVPT>(in, seg, lane, e);
    else
        load_scalar<T, kVPT>(in, seg, n, lane, e, T(0));
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

template <typename T, bool INCLUSIVE, bool VEC>
__global__ __launch_bounds__(kThreads) void tile_rescan_kernel(const T* in, T* out, int64_t n,
                                                                const T* offsets)
{
    using S = Shape<T, kVPT>;
    constexpr int V = S::kPerVec;
    __shared__ T s_wave[kWaves];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = VEC && seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, kVPT>(in, seg, lane, e);
    else
        load_scalar<T, kVPT>(in, seg, n, lane, e, T(0));
    T off[kVPT];
    T wave_excl;
    tile_local_scan<T, V, kVPT>(e, off, wave_excl, s_wave);
    tile_finish<T, V, kVPT, INCLUSIVE>(e, off, wave_excl, offsets[tile]);
    if (whole)
        store_vec<T, kVPT>(out, seg, lane, e);
    else
        store_scalar<T, kVPT>(out, seg, n, lane, e);
}

template <typename T>
__device__ __forceinline__ bool keep(T v, int cmp, T c)
{
    switch (cmp) {
    case 0: return v < c;
    case 1: return v <= c;
    case 2: return v > c;
    case 3: return v >= c;
    case 4: return v == c;
    default: return v != c;
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void compact_kernel(const T* in, T* out, int64_t* num_selected,
                                                            int64_t n, int64_t num_tiles, int cmp, T operand,
                                                            Ctrl* ctrl, uint64_t* status, uint32_t spin_limit)
{
    using S = Shape<T, kCompactVPT>;
    constexpr int V = S::kPerVec;
    __shared__ uint32_t s_wave[kWaves];
    __shared__ T s_stage[S::kTile];
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);

    const int64_t tile = blockIdx.x;
    const uint32_t epoch = (num_tiles > 1 && wave == 0) ? launch_epoch(ctrl) : 0u;

    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = VEC && seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, kCompactVPT>(in, seg, lane, e);
    else
        load_scalar<T, kCompactVPT>(in, seg, n, lane, e, T(0));

    uint32_t cnt[S::kItems];
    bool kept[S::kItems];
#pragma unroll
    for (int k = 0; k < kCompactVPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int i = k * V + j;
            kept[i] = (whole || elem_index<T>(seg, k, j, lane) < n) && keep(e[i], cmp, operand);
            cnt[i] = kept[i] ? 1u : 0u;
        }
    uint32_t off[kCompactVPT];
    uint32_t wave_excl;
    const uint32_t agg = tile_local_scan<uint32_t, V, kCompactVPT>(cnt, off, wave_excl, s_wave);

    // Stage kept elements at their rank inside the tile (memory order).
#pragma unroll
    for (int k = 0; k < kCompactVPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int i = k * V + j;
            const uint32_t rank = wave_excl + off[k] + (j > 0 ? cnt[i - 1] : 0u);
            if (kept[i]) s_stage[rank] = e[i];
        }

    uint32_t prefix = 0;
    if (num_tiles > 1)
        prefix = tile_prefix<uint32_t>(tile, num_tiles, epoch, agg, ctrl, status, spin_limit);
    else
        __syncthreads();

    // A prefix past n can only come from a look-back that gave up; never write past the buffer.
    const bool fits = (int64_t)prefix + agg <= n;
    if (!fits && threadIdx.x == 0) flag_timeout(ctrl);
    for (uint32_t i = threadIdx.x; fits && i < agg; i += kThreads)
        out[(int64_t)prefix + i] = s_stage[i];
    if (tile == num_tiles - 1 && threadIdx.x == 0) *num_selected = (int64_t)prefix + agg;
}

template <int VPT>
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* in, u32x4* out, int64_t nvec)
{
    const int64_t base = (int64_t)blockIdx.x * (kThreads * VPT) +
                         (int64_t)(threadIdx.x / kWave) * (kWave * VPT) + lane_id();
    u32x4 r[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (base + k * kWave < nvec) r[k] = __builtin_nontemporal_load(in + base + k * kWave);
#pragma unroll
    for (int k = 0; k < VPT; ++k)
        if (base + k * kWave < nvec) __builtin_nontemporal_store(r[k], out + base + k * kWave);
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
int64_t tile_elems(int elem_bytes) { return (int64_t)kTileBytes / elem_bytes; }
int64_t tile_bytes() { return kTileBytes; }
int64_t compact_tile_elems(int elem_bytes) { return (int64_t)kThreads * kCompactVPT * kVecBytes / elem_bytes; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <typename T, bool INCL, bool VEC>
static hipError_t lookback_typed(const void* in, void* out, int64_t n, const DevWs& ws, uint32_t spin,
                                 hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, kVPT>::kTile - 1) / Shape<T, kVPT>::kTile;
    lookback_scan_kernel<T, INCL, VEC, kVPT><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
        (const T*)in, (T*)out, n, tiles, ws.ctrl, ws.status, spin);
    return hipGetLastError();
}

template <typename T>
static hipError_t lookback_dispatch(bool incl, const void* in, void* out, int64_t n, const DevWs& ws,
                                    uint32_t spin, hipStream_t st)
{
    const bool vec = aligned16(in) && aligned16(out);
    if (incl)
        return vec ? lookback_typed<T, true, true>(in, out, n, ws, spin, st)
                   : lookback_typed<T, true, false>(in, out, n, ws, spin, st);
    return vec ? lookback_typed<T, false, true>(in, out, n, ws, spin, st)
               : lookback_typed<T, false, false>(in, out, n, ws, spin, st);
}

hipError_t launch_lookback_scan(ElemKind kind, bool inclusive, const void* in, void* out, int64_t n,
                                const DevWs& ws, uint32_t spin_limit, hipStream_t stream)
{
    switch (kind) {
    case kF32: return lookback_dispatch<float>(inclusive, in, out, n, ws, spin_limit, stream);
    case kU64:
    case kI64: return lookback_dispatch<uint64_t>(inclusive, in, out, n, ws, spin_limit, stream);
    default: return lookback_dispatch<uint32_t>(inclusive, in, out, n, ws, spin_limit, stream);
    }
}

template <typename T, bool VEC>
static hipError_t three_pass_typed(bool incl, const void* in, void* out, int64_t n, const DevWs& ws,
                                   hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, kVPT>::kTile - 1) / Shape<T, kVPT>::kTile;
    T* totals = (T*)ws.totals;
    tile_reduce_kernel<T, VEC><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>((const T*)in, n, totals);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scan_totals_kernel<T><<<dim3(1), dim3(kTotalsThreads), 0, st>>>(totals, tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (incl)
        tile_rescan_kernel<T, true, VEC><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, n, totals);
    else
        tile_rescan_kernel<T, false, VEC><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
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

template <typename T>
static hipError_t compact_typed(const void* in, void* out, int64_t* num_selected, int64_t n, int cmp,
                                uint64_t operand_bits, const DevWs& ws, uint32_t spin, hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, kCompactVPT>::kTile - 1) / Shape<T, kCompactVPT>::kTile;
    T operand;
    if constexpr (sizeof(T) == 4)
        operand = __builtin_bit_cast(T, (uint32_t)operand_bits);
    else
        operand = __builtin_bit_cast(T, operand_bits);
    if (aligned16(in))
        compact_kernel<T, true><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, num_selected, n, tiles, cmp, operand, ws.ctrl, ws.status, spin);
    else
        compact_kernel<T, false><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, num_selected, n, tiles, cmp, operand, ws.ctrl, ws.status, spin);
    return hipGetLastError();
}

hipError_t launch_compact(ElemKind kind, const void* in, void* out, int64_t* num_selected, int64_t n, int cmp,
                          uint64_t operand_bits, const DevWs& ws, uint32_t spin_limit, hipStream_t stream)
{
    switch (kind) {
    case kU32: return compact_typed<uint32_t>(in, out, num_selected, n, cmp, operand_bits, ws, spin_limit, stream);
    case kI32: return compact_typed<int32_t>(in, out, num_selected, n, cmp, operand_bits, ws, spin_limit, stream);
    case kF32: return compact_typed<float>(in, out, num_selected, n, cmp, operand_bits, ws, spin_limit, stream);
    case kU64: return compact_typed<uint64_t>(in, out, num_selected, n, cmp, operand_bits, ws, spin_limit, stream);
    default: return compact_typed<int64_t>(in, out, num_selected, n, cmp, operand_bits, ws, spin_limit, stream);
    }
}

hipError_t launch_copy(const void* in, void* out, int64_t nbytes, hipStream_t stream)
{
    const int64_t nvec = nbytes / kVecBytes;
    const int64_t per_block = (int64_t)kThreads * kVPT;
    const int64_t blocks = (nvec + per_block - 1) / per_block;
    copy_kernel<kVPT><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>((const u32x4*)in, (u32x4*)out, nvec);
    return hipGetLastError();
}

}  // namespace ds
