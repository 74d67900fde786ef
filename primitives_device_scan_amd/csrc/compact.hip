// compact.hip -- order-preserving stream compaction in one pass: keep flags
// counted per tile, the counts scanned with the same look-back as the scan,
// kept elements written contiguously at their global rank ("Prefix sum and
// other parallel patterns", section "Stream compaction", first exercise,
// fused form).
#include "device_scan.hpp"
#include "devscan.h"

namespace ds {

// The comparison, fixed at compile time (one kernel per operator): a single
// compare per element in the element type's own order. A NaN compares false
// under every operator except !=.
template <int CMP, typename T>
__device__ __forceinline__ bool keep(T v, T c)
{
    if constexpr (CMP == DS_LT) return v < c;
    if constexpr (CMP == DS_LE) return v <= c;
    if constexpr (CMP == DS_GT) return v > c;
    if constexpr (CMP == DS_GE) return v >= c;
    if constexpr (CMP == DS_EQ) return v == c;
    return v != c;
}

// Compaction over 64 KiB tiles. The keep flags live as one bit per element in
// 64-bit mask words; the per-vector keep counts go through the same
// wave/tile scan and look-back as a scan of 32-bit counts. The tile's kept
// elements leave through one LDS buffer in windows of the tile's ranks:
// every wave places the kept elements whose rank falls in the window at LDS
// index rank - window start (the first window before the look-back, while the
// tile waits for its prefix), and once the output offset is known the whole
// workgroup writes the window back as one contiguous run of 16-byte
// non-temporal stores from a 64-byte line boundary (element stores at the two
// ragged ends), each wave's store covering whole lines. At up to kWinBytes of
// kept data per tile that is one window, so a tile's output has seams only
// where it meets its neighbours.
constexpr int kWinBytes = 36 * 1024;  // LDS for one window; 4 workgroups per CU still fit

// IN_A16: `in` is 16-byte aligned (whole waves load 16-byte vectors either way).
// VPT vectors per thread, compiled for OCC workgroups per CU.
template <typename T, bool IN_A16, int CMP, int VPT = kCompactVPT, int OCC = kCompactOcc, int WIN_BYTES = kWinBytes>
__global__ __launch_bounds__(kThreads, OCC) void compact_kernel(const T* in, T* out, int64_t* num_selected,
                                                               int64_t n, int64_t num_tiles, T operand, Ctrl* ctrl,
                                                               uint64_t* status, uint32_t spin_limit)
{
    using S = Shape<T, VPT>;
    constexpr int V = S::kPerVec;
    constexpr uint32_t kWin = WIN_BYTES / sizeof(T);  // ranks per window, a multiple of V
    constexpr int kMaskWords = (S::kItems + 63) / 64;  // a vector's V bits never straddle two words
    __shared__ uint32_t s_wave[kWaves];
    constexpr uint32_t kLine = 64 / sizeof(T);  // elements per 64-byte line
    __shared__ __attribute__((aligned(16))) T s_stage[kWin + kLine];  // a window plus the alignment shift
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t tile = blockIdx.x;
    const uint32_t epoch = (num_tiles > 1 && wave == 0) ? launch_epoch(ctrl) : 0u;
    uint64_t touched = 0;
    if (num_tiles > 1 && threadIdx.x == 0) touched = touch_status(status, tile);

    const int64_t seg = tile * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = seg + S::kWaveElems <= n;
    T e[S::kItems];
    if (whole)
        load_vec<T, VPT, IN_A16>(in, seg, lane, e);
    else
        load_scalar<T, VPT>(in, seg, n, lane, e, T(0));

    uint64_t keepm[kMaskWords] = {};  // bit i % 64 of word i / 64: this lane keeps element slot i
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int i = k * V + j;
            if ((whole || elem_index<T>(seg, k, j, lane) < n) && keep<CMP>(e[i], operand))
                keepm[i / 64] |= 1ull << (i % 64);
        }
    uint32_t cnt[VPT];
    uint32_t mine = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        cnt[k] = (uint32_t)__builtin_popcountll((keepm[k * V / 64] >> (k * V % 64)) & ((1ull << V) - 1));
        mine += cnt[k];
    }
    // The tile's keep count by a reduction first, published at once, so that
    // successors can use it while this tile ranks its elements.
    const uint32_t wave_total = wave_sum(mine);
    if (lane == 0) s_wave[wave] = wave_total;
    __syncthreads();
    uint32_t agg = 0, wave_excl = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t v = s_wave[w];
        if (w < wave) wave_excl += v;
        agg += v;
    }
    if (num_tiles > 1 && threadIdx.x == 0) publish_early<uint32_t>(status, tile, epoch, agg, 0u);
    // Tile rank of each vector's first kept element in this lane.
    uint32_t off[VPT];
    uint32_t run = wave_excl;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const uint32_t incl = wave_inclusive_scan(cnt[k]);
        off[k] = run + wave_shift_right1(incl);
        run += readlane(incl, kWave - 1);
    }

    // Places this thread's kept elements whose ranks lie in [lo, lo + width) at
    // LDS index rank - lo.
    auto stage = [&](uint32_t lo, uint32_t width) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            uint32_t t = off[k] - lo;  // window slot of the vector's first kept element; wraps below the window
#pragma unroll
            for (int j = 0; j < V; ++j)
                if ((keepm[(k * V + j) / 64] >> ((k * V + j) % 64)) & 1ull) {
                    if (t < width) s_stage[t] = e[k * V + j];
                    ++t;
                }
        }
    };
    // The first window (every kept element when they fit in it) is staged
    // before the look-back: its LDS work then overlaps the wait for the prefix
    // instead of following it while the tile is held.
    stage(0u, agg < kWin ? agg : kWin);
    uint32_t prefix = 0;
    if (num_tiles > 1)
        prefix = tile_prefix<uint32_t>(tile, num_tiles, epoch, agg, ctrl, status, spin_limit, 0u, true);
    else
        __syncthreads();  // tile_prefix ends with this barrier, which the staged window needs

    // A prefix past n can only come from a look-back that gave up; never write past the buffer.
    const bool fits = (int64_t)prefix + agg <= n;
    if (!fits && threadIdx.x == 0) flag_timeout(ctrl);
    // Phase of `out` within a 64-byte line, in elements: each window is written
    // from a line boundary (a wave's 1 KiB store then writes 16 whole lines, not
    // parts of 17), reading the staged elements `shift` slots back.
    const uint32_t out_phase = (uint32_t)(((uintptr_t)out % 64) / sizeof(T));
    for (uint32_t lo = 0; lo < agg; lo += kWin) {  // agg is the same in every wave
        const uint32_t hi = agg - lo < kWin ? agg : lo + kWin;
        const uint32_t width = hi - lo;
        if (lo > 0) {
            stage(lo, width);
            __syncthreads();
        }
        const int64_t first = (int64_t)prefix + lo;  // output index of the window's first element
        const uint32_t shift = (uint32_t)((first + out_phase) % kLine);
        const uint32_t span = shift + width;
        // Output index of slot 0 of the shifted window: out + dst0 is 64-byte aligned;
        // dst0 may be below 0, and only slots from `shift` on (indices from `first`) are written.
        const int64_t dst0 = first - (int64_t)shift;
        if (fits) {
            for (uint32_t q = threadIdx.x * V; q < span; q += kThreads * V) {
                if (q >= shift && q + V <= span) {
                    T v[V];
#pragma unroll
                    for (int j = 0; j < V; ++j) v[j] = s_stage[q - shift + j];
                    u32x4 w;
                    __builtin_memcpy(&w, v, kVecBytes);
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + (dst0 + q)));
                } else {
                    for (uint32_t i = q; i < q + V && i < span; ++i)
                        if (i >= shift) out[dst0 + i] = s_stage[i - shift];
                }
            }
        }
        if (hi < agg) __syncthreads();  // the next window reuses the buffer
    }
    if (tile == num_tiles - 1 && threadIdx.x == 0) {
        // -1 when a look-back wait gave up (here or in a tile whose prefix
        // this one used): the kept elements are then not where they belong.
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool bad = !fits || (num_tiles > 1 && __hip_atomic_load(&ctrl->timeout, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT) != 0u);
        *num_selected = bad ? (int64_t)-1 : (int64_t)prefix + agg;
    }
    if (threadIdx.x == 0) keep_alive(touched);
}

__global__ void write_count_kernel(int64_t* p, int64_t v) { *p = v; }

hipError_t launch_write_count(int64_t* p, int64_t v, hipStream_t stream)
{
    write_count_kernel<<<1, 1, 0, stream>>>(p, v);
    return hipGetLastError();
}

template <typename T, int CMP>
static hipError_t compact_cmp(const void* in, void* out, int64_t* num_selected, int64_t n, T operand,
                              const DevWs& ws, uint32_t spin, hipStream_t st)
{
    const int64_t tiles = (n + Shape<T, kCompactVPT>::kTile - 1) / Shape<T, kCompactVPT>::kTile;  // compact_tile_elems
    if (tiles > 1 && (!ws.ctrl || !ws.status)) return hipErrorInvalidValue;  // several tiles need a workspace
    if (aligned16(in))
        compact_kernel<T, true, CMP><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, num_selected, n, tiles, operand, ws.ctrl, ws.status, spin);
    else
        compact_kernel<T, false, CMP><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(
            (const T*)in, (T*)out, num_selected, n, tiles, operand, ws.ctrl, ws.status, spin);
    return hipGetLastError();
}

template <typename T>
static hipError_t compact_typed(const void* in, void* out, int64_t* num_selected, int64_t n, int cmp,
                                uint64_t operand_bits, const DevWs& ws, uint32_t spin, hipStream_t st)
{
    T operand;
    if constexpr (sizeof(T) == 4)
        operand = __builtin_bit_cast(T, (uint32_t)operand_bits);
    else
        operand = __builtin_bit_cast(T, operand_bits);
    switch (cmp) {
    case DS_LT: return compact_cmp<T, DS_LT>(in, out, num_selected, n, operand, ws, spin, st);
    case DS_LE: return compact_cmp<T, DS_LE>(in, out, num_selected, n, operand, ws, spin, st);
    case DS_GT: return compact_cmp<T, DS_GT>(in, out, num_selected, n, operand, ws, spin, st);
    case DS_GE: return compact_cmp<T, DS_GE>(in, out, num_selected, n, operand, ws, spin, st);
    case DS_EQ: return compact_cmp<T, DS_EQ>(in, out, num_selected, n, operand, ws, spin, st);
    default: return compact_cmp<T, DS_NE>(in, out, num_selected, n, operand, ws, spin, st);
    }
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

}  // namespace ds
