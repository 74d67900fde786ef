// tile.hpp -- gfx950 device building blocks of the scan: per-thread register
// scans over 16-byte vectors, 64-lane wavefront scans on DPP, the workgroup
// scan of wave totals in LDS, and the per-tile status words of the
// single-pass look-back.
//
// Tile layout (all kernels): a workgroup of 256 threads (4 waves of 64) owns
// one tile of VPT sixteen-byte vectors per thread (Shape<T, VPT>; each kernel
// picks its VPT). Wave w owns the w-th quarter of the tile; in it, lane l
// holds the 16-byte vectors k*64 + l for k = 0..VPT-1. Every load and store
// instruction of a wave therefore covers 1 KiB of contiguous memory, and the
// scan order inside the wave is (vector k, lane, element in vector), which is
// the memory order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kVecBytes = 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte access
// The same 16 bytes at an address that is only 4-byte aligned (a tensor slice
// that starts mid-vector). Global 16-byte accesses need dword alignment only,
// so these still compile to one dwordx4 load or store per lane; a wave's
// 1 KiB then straddles one more 128-byte line.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
template <bool A16> struct VecOf { using type = u32x4; };
template <> struct VecOf<false> { using type = u32x4_a4; };

// VPT = 16-byte vectors per thread; the tile is kThreads * VPT * 16 bytes.
template <typename T, int VPT>
struct Shape {
    static constexpr int kPerVec = kVecBytes / (int)sizeof(T);   // elements per 16-byte vector
    static constexpr int kItems = kPerVec * VPT;                 // elements per thread
    static constexpr int kWaveElems = kWave * kItems;            // elements per wave
    static constexpr int kTile = kThreads * kItems;              // elements per tile
    static constexpr int kTileBytes = kThreads * VPT * kVecBytes;
};

// Launch-wide control words, kept in the workspace.
struct Ctrl {
    uint32_t epoch;     // 30-bit launch number stamped into status words
    uint32_t timeout;   // set to 1 when a look-back wait gave up
    uint32_t pad[62];
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// ---------------------------------------------------------------------------
// Cross-lane moves. update_dpp with old = 0: lanes whose source lane lies
// outside the pattern, or whose row is masked off, read 0 -- the identity of
// addition for every type here (+0.0 for floats).
// ---------------------------------------------------------------------------
template <int CTRL, int ROWS = 0xf, typename T>
__device__ __forceinline__ T dpp(T x)
{
    if constexpr (sizeof(T) == 4) {
        const int u = __builtin_bit_cast(int, x);
        return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, u, CTRL, ROWS, 0xf, false));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xf, false);
        const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xf, false);
        return __builtin_bit_cast(T, (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32));
    }
}

template <typename T>
__device__ __forceinline__ T readlane(T x, int src)
{
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
        return __builtin_bit_cast(T, (uint64_t)lo | ((uint64_t)hi << 32));
    }
}

// Inclusive scan over the 64 lanes of a wave: Hillis-Steele steps 1, 2, 4, 8
// inside each row of 16 lanes (row_shr), then lane 15 of rows 0 and 2 is added
// into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31). Six dependent adds; every lane must be active.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x)
{
    x = x + dpp<0x111>(x);       // row_shr:1
    x = x + dpp<0x112>(x);       // row_shr:2
    x = x + dpp<0x114>(x);       // row_shr:4
    x = x + dpp<0x118>(x);       // row_shr:8
    x = x + dpp<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
    x = x + dpp<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
    return x;
}

// Lane l receives lane l-1's value, lane 0 receives 0 (wave_shr:1): turns an
// inclusive scan into an exclusive one without a subtraction.
template <typename T>
__device__ __forceinline__ T wave_shift_right1(T x) { return dpp<0x138>(x); }

template <typename T>
__device__ __forceinline__ T wave_sum(T x) { return readlane(wave_inclusive_scan(x), kWave - 1); }

// An empty asm statement that claims to modify each value: the arithmetic
// that produced them must be done here, before whatever follows. Used after a
// tile's in-register scan so that the compiler cannot sink the scan's last
// additions past the wait for the tile's prefix (folding them into the
// prefix add), which would lengthen the time the tile is held.
template <typename T, int N>
__device__ __forceinline__ void pin_in_registers(T (&x)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// ---------------------------------------------------------------------------
// Tile loads and stores.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ int64_t elem_index(int64_t seg, int k, int j, int lane)
{
    return seg + (int64_t)(k * kWave + lane) * (kVecBytes / (int)sizeof(T)) + j;
}

// Whole wave segment in range: one 16-byte load per vector. A16: `in` is
// 16-byte aligned (else only element-aligned).
template <typename T, int VPT, bool A16 = true>
__device__ __forceinline__ void load_vec(const T* __restrict__ in, int64_t seg, int lane,
                                         T (&e)[Shape<T, VPT>::kItems])
{
    using V = typename VecOf<A16>::type;
    const V* p = reinterpret_cast<const V*>(in + seg) + lane;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const V r = __builtin_nontemporal_load(p + k * kWave);
        __builtin_memcpy(&e[k * Shape<T, VPT>::kPerVec], &r, kVecBytes);
    }
}

// Element-wise, guarded: elements at or past n read as `fill`.
template <typename T, int VPT>
__device__ __forceinline__ void load_scalar(const T* __restrict__ in, int64_t seg, int64_t n, int lane,
                                            T (&e)[Shape<T, VPT>::kItems], T fill)
{
    constexpr int V = Shape<T, VPT>::kPerVec;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int64_t i = elem_index<T>(seg, k, j, lane);
            e[k * V + j] = i < n ? in[i] : fill;
        }
}

template <typename T, int VPT, bool A16 = true>
__device__ __forceinline__ void store_vec(T* __restrict__ out, int64_t seg, int lane,
                                          const T (&e)[Shape<T, VPT>::kItems])
{
    using V = typename VecOf<A16>::type;
    V* p = reinterpret_cast<V*>(out + seg) + lane;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        V r;
        __builtin_memcpy(&r, &e[k * Shape<T, VPT>::kPerVec], kVecBytes);
        __builtin_nontemporal_store(r, p + k * kWave);
    }
}

// e + head, stored vector by vector: each vector's additions, then its
// store. After each store an empty asm with a memory clobber claims to
// touch the next vector's values, so the compiler can neither hoist the
// later additions above the store nor sink the store below them: the first
// store leaves after one vector's additions instead of the whole tile's.
template <typename T, int VPT, bool A16 = true>
__device__ __forceinline__ void add_store_vec(T* __restrict__ out, int64_t seg, int lane,
                                              T (&e)[Shape<T, VPT>::kItems], T head)
{
    using V = typename VecOf<A16>::type;
    constexpr int PV = Shape<T, VPT>::kPerVec;
    V* p = reinterpret_cast<V*>(out + seg) + lane;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
        for (int j = 0; j < PV; ++j) e[k * PV + j] = head + e[k * PV + j];
        V r;
        __builtin_memcpy(&r, &e[k * PV], kVecBytes);
        __builtin_nontemporal_store(r, p + k * kWave);
        if (k + 1 < VPT) {
#pragma unroll
            for (int j = 0; j < PV; ++j) asm volatile("" : "+v"(e[(k + 1) * PV + j])::"memory");
        }
    }
}

template <typename T, int VPT>
__device__ __forceinline__ void store_scalar(T* __restrict__ out, int64_t seg, int64_t n, int lane,
                                             const T (&e)[Shape<T, VPT>::kItems])
{
    constexpr int V = Shape<T, VPT>::kPerVec;
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int64_t i = elem_index<T>(seg, k, j, lane);
            if (i < n) out[i] = e[k * V + j];
        }
}

// ---------------------------------------------------------------------------
// Scan of one tile held in registers. V is the number of elements per 16-byte
// vector of the data (4 or 2); T is the type being summed (the data, or 32-bit
// keep counts in compaction). tile_reduce gives the tile aggregate and the
// sums of the waves before each wave; scan_in_wave (or scan_store_vec, which
// also stores) scans each wave's segment.
// ---------------------------------------------------------------------------
// The tile aggregate by a reduction (each lane's elements, then the wave, then
// the four wave totals through LDS): known before any prefix is computed, so
// the look-back scan can publish it at once. Out: wave_excl = sum of the
// waves before this one. One workgroup barrier.
template <typename T, int N>
__device__ __forceinline__ T tile_reduce(const T (&e)[N], T& wave_excl, T* s_wave)
{
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    T s = T(0);
#pragma unroll
    for (int i = 0; i < N; ++i) s = s + e[i];
    s = wave_sum(s);
    if (lane == 0) s_wave[wave] = s;
    __syncthreads();
    T agg = T(0), before = T(0);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const T v = s_wave[w];
        if (w < wave) before = before + v;
        agg = agg + v;
    }
    wave_excl = before;
    return agg;
}

// The scan within the wave, one vector at a time: each vector's serial scan,
// then a wave scan of the vector totals folded into its elements at once, so
// only the data and a few temporaries are live. Out: e = each element's
// inclusive or exclusive sum within its wave's segment.
template <typename T, int V, int VPT, bool INCLUSIVE>
__device__ __forceinline__ void scan_in_wave(T (&e)[V * VPT])
{
    T run = T(0);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
        for (int j = 1; j < V; ++j)
            e[k * V + j] = e[k * V + j] + e[k * V + j - 1];
        const T incl = wave_inclusive_scan(e[k * V + V - 1]);
        const T off = run + wave_shift_right1(incl);
        run = run + readlane(incl, kWave - 1);
        if constexpr (INCLUSIVE) {
#pragma unroll
            for (int j = 0; j < V; ++j)
                e[k * V + j] = off + e[k * V + j];
        } else {
#pragma unroll
            for (int j = V - 1; j > 0; --j)
                e[k * V + j] = off + e[k * V + j - 1];
            e[k * V] = off;
        }
    }
}

// scan_in_wave, `head` added and each vector stored as soon as its values
// are final (head: the tile's prefix plus the sums of the waves before this
// one, so every value is final once its vector is scanned). The same empty
// asm as in add_store_vec keeps each store ahead of the next vector's scan.
template <typename T, int V, int VPT, bool INCLUSIVE, bool A16 = true>
__device__ __forceinline__ void scan_store_vec(T* __restrict__ out, int64_t seg, int lane, T (&e)[V * VPT], T head)
{
    using Vec = typename VecOf<A16>::type;
    Vec* p = reinterpret_cast<Vec*>(out + seg) + lane;
    T run = head;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
#pragma unroll
        for (int j = 1; j < V; ++j)
            e[k * V + j] = e[k * V + j] + e[k * V + j - 1];
        const T incl = wave_inclusive_scan(e[k * V + V - 1]);
        const T off = run + wave_shift_right1(incl);
        run = run + readlane(incl, kWave - 1);
        if constexpr (INCLUSIVE) {
#pragma unroll
            for (int j = 0; j < V; ++j)
                e[k * V + j] = off + e[k * V + j];
        } else {
#pragma unroll
            for (int j = V - 1; j > 0; --j)
                e[k * V + j] = off + e[k * V + j - 1];
            e[k * V] = off;
        }
        Vec r;
        __builtin_memcpy(&r, &e[k * V], kVecBytes);
        __builtin_nontemporal_store(r, p + k * kWave);
        if (k + 1 < VPT) {
#pragma unroll
            for (int j = 0; j < V; ++j) asm volatile("" : "+v"(e[(k + 1) * V + j])::"memory");
        }
    }
}

// Adds the same value (the tile's exclusive prefix plus the waves before this
// one) to every element.
template <typename T, int N>
__device__ __forceinline__ void add_uniform(T (&e)[N], T head)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        e[i] = head + e[i];
}

// ---------------------------------------------------------------------------
// Status words of the single-pass look-back.
//
// A 4-byte value travels in one 64-bit word: bits 0-31 the value, bits 32-33
// the flag (0 nothing yet, 1 aggregate of this tile only, 2 inclusive prefix
// through this tile), bits 34-63 the launch epoch. A word whose epoch is not
// the current launch's reads as "nothing yet", so the array never needs
// clearing between launches. An 8-byte value travels in two such words (low
// and high halves, same flag and epoch); a reader accepts the pair only when
// both words carry the same flag and the current epoch, which rules out a
// torn read because each flag is written once per launch.
//
// Words are written and read with relaxed device-scope atomics: coherent
// across the XCDs' separate L2 caches, with no cache writeback or invalidate.
// Each word carries its own value, so no ordering with other memory is needed.
//
// Each tile's words sit alone in one 128-byte line (kStatusWords 64-bit words
// per tile; an 8-byte value uses the first two). Packed eight to a line, the
// words of neighbouring tiles share a line that is written by one tile while
// the next polls it; measured on MI355X at n = 100M int32, padding each tile
// to its own line makes the whole scan 3-4% faster (144 -> 139 us), although
// a 64-tile window read then touches 64 lines instead of 4.
// ---------------------------------------------------------------------------
constexpr uint32_t kFlagNone = 0, kFlagAggregate = 1, kFlagPrefix = 2;
constexpr uint32_t kEpochMask = 0x3FFFFFFFu;
constexpr int kStatusWords = 16;  // 64-bit words (one 128-byte line) per tile

__device__ __forceinline__ void status_store(uint64_t* p, uint64_t w)
{
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t status_load(uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t status_word(uint32_t epoch, uint32_t flag, uint32_t bits)
{
    return ((uint64_t)((epoch << 2) | flag) << 32) | bits;
}

template <typename T>
struct StatusCodec {

    static __device__ __forceinline__ void publish(uint64_t* status, int64_t tile, uint32_t epoch,
                                                   uint32_t flag, T v)
    {
        uint64_t* p = status + tile * kStatusWords;
        if constexpr (sizeof(T) == 4) {
            status_store(p, status_word(epoch, flag, __builtin_bit_cast(uint32_t, v)));
        } else {
            const uint64_t u = __builtin_bit_cast(uint64_t, v);
            status_store(p, status_word(epoch, flag, (uint32_t)u));
            status_store(p + 1, status_word(epoch, flag, (uint32_t)(u >> 32)));
        }
    }

    // Reads tile `idx`'s status; returns its flag (kFlagNone when stale or torn).
    static __device__ __forceinline__ uint32_t read(uint64_t* status, int64_t idx, uint32_t epoch, T& v)
    {
        uint64_t* p = status + idx * kStatusWords;
        if constexpr (sizeof(T) == 4) {
            const uint64_t w = status_load(p);
            const uint32_t hi = (uint32_t)(w >> 32);
            v = __builtin_bit_cast(T, (uint32_t)w);
            return (hi >> 2) == epoch ? (hi & 3u) : kFlagNone;
        } else {
            const uint64_t w0 = status_load(p);
            const uint64_t w1 = status_load(p + 1);
            const uint32_t h0 = (uint32_t)(w0 >> 32), h1 = (uint32_t)(w1 >> 32);
            v = __builtin_bit_cast(T, (uint64_t)(uint32_t)w0 | (w1 << 32));
            return (h0 == h1 && (h0 >> 2) == epoch) ? (h0 & 3u) : kFlagNone;
        }
    }
};

// Decoupled look-back, run by one whole wave for tile `tile` (> 0) once the
// tile's aggregate is known.
//  1. Publish the aggregate (unless `published`: the caller already has).
//  2. Wait, polling with lane 0 alone, until the nearest predecessor has
//     published anything: until then no window can complete, and polling one
//     word instead of 64 keeps the status traffic off the memory system.
//  3. Read the status of the 64 preceding tiles at once (lane l reads tile
//     base - l, one coalesced 512-byte access), re-read only the words that
//     still show nothing up to the nearest inclusive prefix, add the
//     aggregates and that prefix, and move 64 tiles further back when the
//     window holds no prefix.
//  4. Publish this tile's inclusive prefix; return the exclusive one.
// Every wait is bounded: after `spin_limit` polls in total the wave gives up,
// missing values count as 0 and `timeout` is set, so every wave finishes.
template <typename T>
__device__ T lookback(uint64_t* status, int64_t tile, uint32_t epoch, T agg, uint32_t spin_limit,
                      uint32_t* timeout, bool published = false)
{
    using C = StatusCodec<T>;
    const int lane = lane_id();
    if (lane == 0 && !published) C::publish(status, tile, epoch, kFlagAggregate, agg);
    uint32_t polls = 0;
    bool gave_up = false;
    auto give_up = [&]() {
        gave_up = true;
        if (lane == 0) __hip_atomic_store(timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the flag becomes visible before the (incomplete) prefix this tile publishes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    };
    uint32_t f = kFlagNone;
    T v0 = T(0);
    for (;;) {
        if (lane == 0) f = C::read(status, tile - 1, epoch, v0);
        if (__builtin_amdgcn_readfirstlane(f) != kFlagNone) break;
        if (++polls >= spin_limit) {
            give_up();
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    // The predecessor's word is already in hand: an inclusive prefix there ends
    // the look-back without a window read (one status round trip fewer on the
    // chain); an aggregate starts the sum and the window begins a tile further back.
    T acc = T(0);
    int64_t base = tile - 1;
    f = __builtin_amdgcn_readfirstlane(f);
    if (f != kFlagNone) {
        acc = readlane(v0, 0);
        if (f == kFlagPrefix) {
            if (lane == 0) C::publish(status, tile, epoch, kFlagPrefix, acc + agg);
            return acc;
        }
        base = tile - 2;
    }
    for (;;) {
        const int64_t idx = base - lane;
        T v = T(0);
        uint32_t flag = kFlagPrefix;  // before tile 0: an inclusive prefix of 0
        if (idx >= 0) flag = C::read(status, idx, epoch, v);
        for (;;) {
            const uint64_t pm = ballot(flag == kFlagPrefix);
            const uint64_t xm = ballot(flag == kFlagNone);
            const uint64_t upto = pm ? (pm ^ (pm - 1)) : ~0ull;  // lanes up to the first prefix
            const bool needed = (upto >> lane) & 1ull;
            if ((xm & upto) && !gave_up) {
                if (++polls < spin_limit) {
                    __builtin_amdgcn_s_sleep(1);
                    if (needed && flag == kFlagNone) flag = C::read(status, idx, epoch, v);
                    continue;
                }
                give_up();
            }
            acc = acc + wave_sum((needed && flag != kFlagNone) ? v : T(0));
            if (pm) {
                if (lane == 0) C::publish(status, tile, epoch, kFlagPrefix, acc + agg);
                return acc;
            }
            break;
        }
        base -= kWave;
    }
}

}  // namespace ds
