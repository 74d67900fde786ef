// tile_lds.hip -- block-level scans of 4,096-element tiles held in LDS: the
// work-efficient up-sweep / down-sweep tree ("Day 32 -- The CUDA scan
// algorithm", sections "Two sweeps over one tree" and "The stride doubles,
// and so does the conflict"; "Grokking Parallel Programming", chapter 7),
// unpadded and with one- and two-term padding, and the double-buffered
// Hillis-Steele scan ("Day 31 -- CUDA prefix sum, the Hillis-Steele scan",
// section "Why one array is not enough"). Each tile is scanned on its own
// (exclusive) and its total is saved before the tree's root is cleared. With
// a scan of the totals and a uniform add they form the pages' three-kernel
// device scan (Day 32, "One block scans 4,096. Ten million needs three
// kernels.").
//
// On gfx950 a 4-byte LDS access of a wave is served 32 lanes at a time over
// 32 banks of 4 bytes (measured: stride-s word accesses cost max(1, lanes per
// bank) cycles per 32-lane half), so the tree's level with stride s puts
// gcd(2s, 32) lanes of a half-wave on one bank. Padding word i to
// i + i/32 spreads those up to stride 16; the second term i/1024 clears the
// levels above it for a 4,096-word tile.
#include "device_scan.hpp"
#include "devscan.h"

namespace ds {

constexpr int kLdsTile = 4096;
constexpr int kLdsThreads = 1024;
constexpr int kLdsPerThread = kLdsTile / kLdsThreads;

template <int PAD>
__device__ __forceinline__ int padded(int i)
{
    if constexpr (PAD == 1) return i + (i >> 5);
    if constexpr (PAD == 2) return i + (i >> 5) + (i >> 10);
    return i;
}

template <int PAD>
constexpr int padded_words()
{
    return PAD == 0 ? kLdsTile : PAD == 1 ? kLdsTile + kLdsTile / 32 : kLdsTile + kLdsTile / 32 + kLdsTile / 1024;
}

// Work-efficient tree over the 4,096 words of a tile, written by tree level
// lv = 0 .. 11. At level lv the words fall into blocks of 2^(lv+1); block a
// owns two nodes, the last word of its first half (its left node) and its
// last word (its right node), and one thread handles one block. Going up, the
// right node accumulates the left one, so each right node ends up holding the
// sum of its block. The root (word 4,095) then holds the tile total; the tile
// keeps that total and sets the root to 0, the exclusive prefix of the tile.
// Coming down, each block's right node holds the sum of everything before the
// block: the left node takes that value, and the right node adds the first
// half's sum to it. Every thread reaches every barrier, active or not.
constexpr int kLdsLevels = 12;  // 2^12 = kLdsTile

__device__ __forceinline__ int left_node(int a, int lv) { return (a << (lv + 1)) | ((1 << lv) - 1); }
__device__ __forceinline__ int right_node(int a, int lv) { return (a << (lv + 1)) | ((2 << lv) - 1); }

template <typename T, int PAD, bool UP>
__device__ __forceinline__ void tree_level(T* tile, int lv)
{
    const int blocks = kLdsTile >> (lv + 1);
    for (int a = (int)threadIdx.x; a < blocks; a += kLdsThreads) {
        const int l = padded<PAD>(left_node(a, lv)), r = padded<PAD>(right_node(a, lv));
        const T first_half = tile[l];
        const T node = tile[r];
        if constexpr (UP) {
            tile[r] = node + first_half;
        } else {
            tile[l] = node;               // everything before the block
            tile[r] = node + first_half;  // ... and its first half
        }
    }
    __syncthreads();
}

template <typename T, int PAD>
__global__ __launch_bounds__(kLdsThreads) void tree_tile_kernel(const T* in, T* out, T* tile_sums, int64_t n)
{
    __shared__ T tile[padded_words<PAD>()];
    const int tid = (int)threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * kLdsTile;
#pragma unroll
    for (int k = 0; k < kLdsPerThread; ++k) {
        const int i = tid + k * kLdsThreads;
        tile[padded<PAD>(i)] = base + i < n ? in[base + i] : T(0);
    }
    __syncthreads();
    for (int lv = 0; lv < kLdsLevels; ++lv) tree_level<T, PAD, true>(tile, lv);
    if (tid == 0) {
        T& root = tile[padded<PAD>(kLdsTile - 1)];
        if (tile_sums) tile_sums[blockIdx.x] = root;
        root = T(0);
    }
    __syncthreads();
    for (int lv = kLdsLevels - 1; lv >= 0; --lv) tree_level<T, PAD, false>(tile, lv);
#pragma unroll
    for (int k = 0; k < kLdsPerThread; ++k) {
        const int i = tid + k * kLdsThreads;
        if (base + i < n) out[base + i] = tile[padded<PAD>(i)];
    }
}

// Hillis-Steele with two buffers: at offset d every word i >= d becomes
// src[i] + src[i-d] in the other buffer and every other word is copied across,
// so nothing is read where it is being written. Inclusive after 12 steps; the
// exclusive result is the inclusive one shifted by one word, and the last
// inclusive word is the tile total.
template <typename T>
__global__ __launch_bounds__(kLdsThreads) void hs_tile_kernel(const T* in, T* out, T* tile_sums, int64_t n)
{
    __shared__ T buf[2][kLdsTile];
    const int tid = (int)threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * kLdsTile;
#pragma unroll
    for (int k = 0; k < kLdsPerThread; ++k) {
        const int i = tid + k * kLdsThreads;
        buf[0][i] = base + i < n ? in[base + i] : T(0);
    }
    __syncthreads();
    int src = 0;
    for (int d = 1; d < kLdsTile; d <<= 1) {
#pragma unroll
        for (int k = 0; k < kLdsPerThread; ++k) {
            const int i = tid + k * kLdsThreads;
            buf[1 - src][i] = i >= d ? buf[src][i] + buf[src][i - d] : buf[src][i];
        }
        __syncthreads();
        src = 1 - src;
    }
    if (tid == 0 && tile_sums) tile_sums[blockIdx.x] = buf[src][kLdsTile - 1];
#pragma unroll
    for (int k = 0; k < kLdsPerThread; ++k) {
        const int i = tid + k * kLdsThreads;
        if (base + i < n) out[base + i] = i > 0 ? buf[src][i - 1] : T(0);
    }
}

// Adds tile b's scanned total to every element of tile b (reads and writes
// the output once more: the third kernel of the pages' pipeline).
template <typename T>
__global__ __launch_bounds__(kLdsThreads) void add_offsets_kernel(T* out, const T* offsets, int64_t n)
{
    const int64_t base = (int64_t)blockIdx.x * kLdsTile;
    const T off = offsets[blockIdx.x];
#pragma unroll
    for (int k = 0; k < kLdsPerThread; ++k) {
        const int64_t i = base + threadIdx.x + k * kLdsThreads;
        if (i < n) out[i] = out[i] + off;
    }
}

template <typename T>
static hipError_t tile_scan_typed(int variant, const void* in, void* out, void* sums, int64_t n, hipStream_t st)
{
    const unsigned tiles = (unsigned)((n + kLdsTile - 1) / kLdsTile);
    const dim3 grid(tiles), block(kLdsThreads);
    switch (variant) {
    case DS_TILE_TREE: tree_tile_kernel<T, 0><<<grid, block, 0, st>>>((const T*)in, (T*)out, (T*)sums, n); break;
    case DS_TILE_TREE_PAD1: tree_tile_kernel<T, 1><<<grid, block, 0, st>>>((const T*)in, (T*)out, (T*)sums, n); break;
    case DS_TILE_TREE_PAD2: tree_tile_kernel<T, 2><<<grid, block, 0, st>>>((const T*)in, (T*)out, (T*)sums, n); break;
    default: hs_tile_kernel<T><<<grid, block, 0, st>>>((const T*)in, (T*)out, (T*)sums, n); break;
    }
    return hipGetLastError();
}

int64_t lds_tile_elems() { return kLdsTile; }

hipError_t launch_tile_scan(ElemKind kind, int variant, const void* in, void* out, void* tile_sums, int64_t n,
                            hipStream_t stream)
{
    if (kind == kF32) return tile_scan_typed<float>(variant, in, out, tile_sums, n, stream);
    return tile_scan_typed<uint32_t>(variant, in, out, tile_sums, n, stream);
}

hipError_t launch_tile_pipeline(ElemKind kind, int variant, const void* in, void* out, int64_t n,
                                const DevWs& ws, hipStream_t stream)
{
    const int64_t tiles = (n + kLdsTile - 1) / kLdsTile;
    if (!ws.totals) return hipErrorInvalidValue;
    hipError_t e = launch_tile_scan(kind, variant, in, out, ws.totals, n, stream);
    if (e != hipSuccess) return e;
    e = launch_scan_totals(kind, ws.totals, tiles, stream);
    if (e != hipSuccess) return e;
    if (kind == kF32)
        add_offsets_kernel<float><<<dim3((unsigned)tiles), dim3(kLdsThreads), 0, stream>>>(
            (float*)out, (const float*)ws.totals, n);
    else
        add_offsets_kernel<uint32_t><<<dim3((unsigned)tiles), dim3(kLdsThreads), 0, stream>>>(
            (uint32_t*)out, (const uint32_t*)ws.totals, n);
    return hipGetLastError();
}

}  // namespace ds
