// compact_unordered.hip -- stream compaction that does not keep the input
// order: a wave ranks its kept elements with a ballot and a count of the set
// lanes below each lane, and claims room for them with one atomic add on a
// global counter ("Prefix sum and other parallel patterns", section "Stream
// compaction", the warp-aggregated atomic and its compact_positive kernel).
// One claim per wave follows the pages; one per workgroup (the four waves'
// counts summed in LDS first) takes four times fewer atomics.
//
// On this GPU a device-scope atomic on one address serialises at roughly
// 50 ns, so the claims, not the memory traffic, bound this kernel: it is the
// comparison point for the ordered single-pass compact_if.
#include "device_scan.hpp"
#include "devscan.h"

namespace ds {

template <int CMP, typename T>
__device__ __forceinline__ bool keep_u(T v, T c)
{
    if constexpr (CMP == DS_LT) return v < c;
    if constexpr (CMP == DS_LE) return v <= c;
    if constexpr (CMP == DS_GT) return v > c;
    if constexpr (CMP == DS_GE) return v >= c;
    if constexpr (CMP == DS_EQ) return v == c;
    return v != c;
}

// Lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ void zero_count_kernel(uint64_t* count) { *count = 0; }

template <typename T, bool IN_A16, int CMP, bool PER_WG>
__global__ __launch_bounds__(kThreads) void compact_unordered_kernel(const T* in, T* out, uint64_t* count,
                                                                      int64_t n, T operand)
{
    using S = Shape<T, kCompactVPT>;
    constexpr int V = S::kPerVec;
    __shared__ uint32_t s_cnt[kWaves];
    __shared__ uint64_t s_start;
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t seg = (int64_t)blockIdx.x * S::kTile + (int64_t)wave * S::kWaveElems;
    const bool whole = seg + S::kWaveElems <= n;  // 16-byte vectors, `in` 16-byte aligned or not (IN_A16)
    T e[S::kItems];
    if (whole)
        load_vec<T, kCompactVPT, IN_A16>(in, seg, lane, e);
    else
        load_scalar<T, kCompactVPT>(in, seg, n, lane, e, T(0));

    uint64_t keepm[(S::kItems + 63) / 64] = {};  // bit i % 64 of word i / 64: this lane keeps element slot i
    uint32_t total = 0;
#pragma unroll
    for (int k = 0; k < kCompactVPT; ++k)
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int i = k * V + j;
            const bool kp = (whole || elem_index<T>(seg, k, j, lane) < n) && keep_u<CMP>(e[i], operand);
            keepm[i / 64] |= (uint64_t)kp << (i % 64);
            total += (uint32_t)__builtin_popcountll(ballot(kp));
        }

    uint64_t start = 0;
    if constexpr (PER_WG) {
        if (lane == 0) s_cnt[wave] = total;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t wg = 0;
            for (int w = 0; w < kWaves; ++w) wg += s_cnt[w];
            s_start = wg ? __hip_atomic_fetch_add(count, (uint64_t)wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
        }
        __syncthreads();
        start = s_start;
        for (int w = 0; w < wave; ++w) start += s_cnt[w];
    } else {
        if (lane == 0 && total)
            start = __hip_atomic_fetch_add(count, (uint64_t)total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        start = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)start)) |
                ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(start >> 32)) << 32);
    }
#pragma unroll
    for (int i = 0; i < S::kItems; ++i) {
        const bool kp = (keepm[i / 64] >> (i % 64)) & 1ull;
        const uint64_t m = ballot(kp);  // the lanes keeping slot i
        if (kp) out[start + lanes_below(m)] = e[i];
        start += (uint64_t)__builtin_popcountll(m);
    }
}

template <typename T, int CMP>
static hipError_t unordered_cmp(const void* in, void* out, int64_t* count, int64_t n, T operand, bool per_wg,
                                hipStream_t st)
{
    const unsigned tiles = (unsigned)((n + Shape<T, kCompactVPT>::kTile - 1) / Shape<T, kCompactVPT>::kTile);
    const dim3 grid(tiles), block(kThreads);
    const bool a16 = aligned16(in);
    zero_count_kernel<<<dim3(1), dim3(1), 0, st>>>((uint64_t*)count);
    if (per_wg) {
        if (a16) compact_unordered_kernel<T, true, CMP, true><<<grid, block, 0, st>>>((const T*)in, (T*)out, (uint64_t*)count, n, operand);
        else compact_unordered_kernel<T, false, CMP, true><<<grid, block, 0, st>>>((const T*)in, (T*)out, (uint64_t*)count, n, operand);
    } else {
        if (a16) compact_unordered_kernel<T, true, CMP, false><<<grid, block, 0, st>>>((const T*)in, (T*)out, (uint64_t*)count, n, operand);
        else compact_unordered_kernel<T, false, CMP, false><<<grid, block, 0, st>>>((const T*)in, (T*)out, (uint64_t*)count, n, operand);
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t unordered_typed(const void* in, void* out, int64_t* count, int64_t n, int cmp,
                                  uint64_t operand_bits, bool per_wg, hipStream_t st)
{
    T operand;
    if constexpr (sizeof(T) == 4)
        operand = __builtin_bit_cast(T, (uint32_t)operand_bits);
    else
        operand = __builtin_bit_cast(T, operand_bits);
    switch (cmp) {
    case DS_LT: return unordered_cmp<T, DS_LT>(in, out, count, n, operand, per_wg, st);
    case DS_LE: return unordered_cmp<T, DS_LE>(in, out, count, n, operand, per_wg, st);
    case DS_GT: return unordered_cmp<T, DS_GT>(in, out, count, n, operand, per_wg, st);
    case DS_GE: return unordered_cmp<T, DS_GE>(in, out, count, n, operand, per_wg, st);
    case DS_EQ: return unordered_cmp<T, DS_EQ>(in, out, count, n, operand, per_wg, st);
    default: return unordered_cmp<T, DS_NE>(in, out, count, n, operand, per_wg, st);
    }
}

hipError_t launch_compact_unordered(ElemKind kind, const void* in, void* out, int64_t* count, int64_t n, int cmp,
                                    uint64_t operand_bits, bool per_workgroup, hipStream_t stream)
{
    switch (kind) {
    case kU32: return unordered_typed<uint32_t>(in, out, count, n, cmp, operand_bits, per_workgroup, stream);
    case kI32: return unordered_typed<int32_t>(in, out, count, n, cmp, operand_bits, per_workgroup, stream);
    case kF32: return unordered_typed<float>(in, out, count, n, cmp, operand_bits, per_workgroup, stream);
    case kU64: return unordered_typed<uint64_t>(in, out, count, n, cmp, operand_bits, per_workgroup, stream);
    default: return unordered_typed<int64_t>(in, out, count, n, cmp, operand_bits, per_workgroup, stream);
    }
}

}  // namespace ds
