// counting_sort.hip -- one stable counting-sort pass: the step a radix sort
// repeats once per digit, and the "histogram, exclusive scan, scatter" of MoE
// token dispatch. The pages name both as users of the exclusive scan ("Day 32
// -- The CUDA scan algorithm", closing section: a radix sort runs one scan per
// digit pass; "Prefix sum and other parallel patterns", section "In LLMs: MoE
// token dispatch" and exercise 2).
//
// Three launches, reduce-then-scan style:
//   1. digit_count_kernel: each group of GROUP consecutive tiles (a tile is
//      kSortThreads * ITEMS keys) counts its digits in LDS and writes
//      count[d * groups + group] -- a digit-major table -- and, for each
//      tile after the group's first, one tile-major row: the counts of the
//      group's earlier tiles;
//   2. the device-wide exclusive scan of that table (the look-back scan): the
//      entry (d, group) becomes the first output slot of the group's digit-d
//      keys; a tile's first slot is that plus its row;
//   3. digit_scatter_kernel: each tile ranks its keys in input order -- a
//      wave matches equal digits with one ballot per digit bit and counts the
//      matching lanes below each lane -- stages the tile in LDS ordered by
//      digit, and writes each digit's run to its slot, so equal digits keep
//      their input order (the pass is stable).
// One tile per scatter workgroup: the cache line two neighbouring tiles
// share at a bucket's run boundary is then written by both at the same stage
// of their lives and merges in L2 instead of going to HBM twice (a workgroup
// that took a group's tiles in turn made the radix scatter 60% slower).
// Groups of four in the count: its table writes cost far more than their
// bytes, the scattered ones most (2^28 keys in one-tile groups: 192 us;
// 4-tile groups with 32-bit rows: 183 us, with 16-bit rows 13 us less per
// pass; the table scan 14 -> 7 us).
// For MoE alignment every scatter workgroup also derives the experts' counts
// and block-rounded offsets from the scanned table and shifts each expert's
// slots to its padded start (workgroup 0 writes counts, offsets and padding
// marks); up to kMoeOneLaunchMax ids, one workgroup does all of it in a
// single launch (moe_align_one_launch_kernel).
// Bucket B (one past the last real digit) collects elements that belong to
// no bucket: the ragged end of the last tile and, for MoE, ids outside
// [0, experts). It takes part in the ranking but is never written.
#include "device_scan.hpp"
#include "launch.hpp"

namespace ds {

// Workgroups of 512 threads (8 waves): for the same tile, each wave ranks
// half as many slots in sequence as with 256, and the CU holds more waves
// to cover the latency between the tile's barriers.
constexpr int kSortThreads = 512;
constexpr int kSortWaves = kSortThreads / kWave;

// Keys per lane per tile (a tile is kSortThreads * ITEMS keys). Longer tiles
// give longer runs per digit, so fewer partly written lines, and fewer
// barriers per key, until registers and LDS cut the workgroups per CU: the
// keys-only radix pass holds 16 per lane (3 workgroups per CU), with values
// 12 (the staged values take LDS too); MoE inputs are small, and shorter
// tiles give more workgroups.
constexpr int kRadixItems = 16;                       // 8,192-key tiles
constexpr int kRadixKvItems = 12;                     // 6,144-key tiles
constexpr int kMoeItems = 4;                          // 2,048-id tiles
constexpr int kRadixGroup = 4;                        // tiles per count-table entry (MoE: 1)
constexpr int kRadixKvGroup = 4;
constexpr int kSortMaxBuckets = 512;                  // real buckets + the spare one

// digit<BITS>(k) is the same bucket as operator(), BITS = ceil(log2(buckets))
// known at compile time. kSpareKeys: whether a key itself can fall in the
// spare bucket (else only the ragged end of the last tile goes there).
struct RadixDigit {
    uint32_t shift, mask, buckets;  // buckets = 2^BITS, mask = buckets - 1
    static constexpr bool kSpareKeys = false;
    __device__ __forceinline__ uint32_t operator()(uint32_t k) const { return (k >> shift) & mask; }
    template <int BITS>
    __device__ __forceinline__ uint32_t digit(uint32_t k) const { return __builtin_amdgcn_ubfe(k, shift, BITS); }
};

// Expert ids: an id outside [0, experts) (negative ones included, as unsigned)
// goes to the spare bucket.
struct ExpertDigit {
    uint32_t buckets;
    static constexpr bool kSpareKeys = true;
    __device__ __forceinline__ uint32_t operator()(uint32_t k) const { return k < buckets ? k : buckets; }
    template <int BITS>
    __device__ __forceinline__ uint32_t digit(uint32_t k) const { return k < buckets ? k : buckets; }
};

__device__ __forceinline__ uint32_t lanes_below_mask(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Lanes whose bucket equals this lane's. For every bit b of the real bucket
// indices, the wave's ballot of that bit is kept where this lane has the bit
// and complemented where it does not, and the results are ANDed:
// same &= ~(ballot_b ^ mine_b), with mine_b = bit b of d copied into all 32
// bits -- one three-input bitwise op (v_bitop3, truth table 0x90 for
// s0 & ~(s1 ^ s2)) per 32-lane half, so a bit costs four VALU instructions.
// SPARE: some lane may hold the spare bucket, whose lanes match only each
// other (its low bits can equal a real bucket's). Every lane of the wave
// takes part.
template <int BITS, bool SPARE>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, uint32_t spare)
{
    constexpr unsigned kKeepWhereEqual = 0x90;
    constexpr int kIcmpNe = 33;  // the "not equal" integer predicate of the lane-mask compare
    uint32_t lo = ~0u, hi = ~0u;
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const uint32_t mine = (uint32_t)__builtin_amdgcn_sbfe((int32_t)d, b, 1);  // 0 or all ones
        const uint64_t set = __builtin_amdgcn_uicmp(mine, 0u, kIcmpNe);         // lanes with bit b
        lo = __builtin_amdgcn_bitop3_b32(lo, (uint32_t)set, mine, kKeepWhereEqual);
        hi = __builtin_amdgcn_bitop3_b32(hi, (uint32_t)(set >> 32), mine, kKeepWhereEqual);
    }
    const uint64_t same = ((uint64_t)hi << 32) | lo;
    if constexpr (!SPARE) {
        return same;
    } else {
        const bool is_spare = d == spare;
        const uint64_t spare_lanes = ballot(is_spare);
        return is_spare ? spare_lanes : (same & ~spare_lanes);
    }
}

// Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b mod 8).
// Renumbering them so that each XCD takes a contiguous run of tiles puts
// neighbouring tiles, which write neighbouring words, on the same XCD, whose
// L2 then merges their partial cache lines before they go to HBM: the count
// table's entries (d, tile) and (d, tile + 1), and the two halves of the line
// at each bucket's run boundary in the scatter. Any order of tiles is correct
// in both kernels: a tile's table column and its output slots follow from
// its number alone.
__device__ __forceinline__ int64_t xcd_contiguous_tile()
{
    const uint32_t G = gridDim.x, b = blockIdx.x, x = b % 8u, q = G / 8u, r = G % 8u;
    return (int64_t)(x * q + (x < r ? x : r) + b / 8u);
}

// All of a lane's keys are loaded before any is counted: the LDS atomics
// would otherwise keep the compiler from issuing the next load until the
// previous one has returned, one 16-byte load in flight per lane.
// One workgroup counts GROUP consecutive tiles (kSortThreads * ITEMS keys
// each): table[d * groups + g] = the group's count of digit d, and for
// GROUP > 1 pre[t * B + d] (16 bits) = the count of d in the tiles of t's group before
// t, for every tile t after the first of its group. A single tile keeps one
// histogram per wave; a group keeps one per tile, shared by the waves.
// A16: keys 16-byte aligned (whole groups load 16-byte vectors either way).
template <typename DIG, bool A16, int ITEMS, int GROUP>
__global__ __launch_bounds__(kSortThreads) void digit_count_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                                 DIG dig, uint32_t* __restrict__ table,
                                                                 uint16_t* __restrict__ pre, int64_t groups,
                                                                 int64_t tiles)
{
    static_assert(ITEMS % 4 == 0, "whole 16-byte vectors per lane");
    static_assert((GROUP - 1) * kSortThreads * ITEMS <= 0xFFFF, "a prefix row entry fits 16 bits");
    constexpr int kTile = kSortThreads * ITEMS, kPer = ITEMS * GROUP, kVecs = kPer / 4, kTileVecs = ITEMS / 4;
    constexpr int kSets = GROUP == 1 ? kSortWaves : 1;
    __shared__ uint32_t hist[GROUP][kSets][kSortMaxBuckets];
    const uint32_t B = dig.buckets;
    const int set = GROUP == 1 ? (int)(threadIdx.x / kWave) : 0;
    for (uint32_t i = threadIdx.x; i < GROUP * kSets * kSortMaxBuckets; i += kSortThreads) (&hist[0][0][0])[i] = 0;
    const int64_t g = xcd_contiguous_tile();
    const int64_t base = g * ((int64_t)kTile * GROUP);
    if (base + (int64_t)kTile * GROUP <= n) {
        // vector v of a lane lies in tile v / kTileVecs of the group
        using V = typename VecOf<A16>::type;
        const V* p = reinterpret_cast<const V*>(keys + base) + threadIdx.x;
        V k[kVecs];
#pragma unroll
        for (int v = 0; v < kVecs; ++v) k[v] = __builtin_nontemporal_load(p + v * kSortThreads);
        __syncthreads();  // the histograms are zero
#pragma unroll
        for (int v = 0; v < kVecs; ++v)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t d = dig(k[v][j]);
                if (!DIG::kSpareKeys || d < B) atomicAdd(&hist[v / kTileVecs][set][d], 1u);
            }
    } else {
        // the ragged last group, element by element: key i of a lane lies in tile i / ITEMS
        uint32_t k[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t at = base + threadIdx.x + (int64_t)i * kSortThreads;
            k[i] = at < n ? keys[at] : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t at = base + threadIdx.x + (int64_t)i * kSortThreads;
            const uint32_t d = dig(k[i]);
            if (at < n && d < B) atomicAdd(&hist[i / ITEMS][set][d], 1u);
        }
    }
    __syncthreads();
    for (uint32_t d = threadIdx.x; d < B; d += kSortThreads) {
        uint32_t run = 0;
#pragma unroll
        for (int i = 0; i < GROUP; ++i) {
            if (i > 0 && g * GROUP + i < tiles) pre[(g * GROUP + i) * B + d] = (uint16_t)run;
            uint32_t c = 0;
#pragma unroll
            for (int w = 0; w < kSets; ++w) c += hist[i][w][d];
            run += c;
        }
        table[(int64_t)d * groups + g] = run;
    }
}

// Exclusive scan over the workgroup of one value per thread;
// returns this thread's exclusive prefix and sets `total`.
__device__ __forceinline__ uint32_t block_exclusive_u32(uint32_t v, uint32_t* s_wave, uint32_t& total)
{
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
        const uint32_t t = s_wave[w];
        if (w < wave) before += t;
        all += t;
    }
    total = all;
    return before + incl - v;
}

// Bucket d = t of thread t: the waves' counts in `cnt` become each wave's
// first staging position for the bucket; gdelta[d] becomes (output slot of
// the tile's first bucket-d key) - (its staging position); gbase[d] moves
// past this tile's bucket-d keys.
__device__ __forceinline__ void tile_bases(uint32_t (*cnt)[kSortMaxBuckets], uint32_t* gbase, uint32_t* gdelta,
                                           uint32_t* s_wave, uint32_t* s_real, uint32_t B)
{
    static_assert(kSortThreads == kSortMaxBuckets, "one bucket per thread");
    const uint32_t d = threadIdx.x;
    uint32_t p[kSortWaves], tot = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
        p[w] = tot;
        if (d <= B) tot += cnt[w][d];
    }
    uint32_t all;
    const uint32_t start = block_exclusive_u32(tot, s_wave, all);
    if (d <= B) {
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) cnt[w][d] = start + p[w];
        if (d < B) {
            gdelta[d] = gbase[d] - start;
            gbase[d] += tot;
        } else {
            *s_real = start;  // keys of real buckets come first in the staging order
        }
    }
}

// LDS of a workgroup that ranks and scatters its tile of kSortThreads * ITEMS keys.
template <int VALS, int ITEMS>
struct SortLds {
    uint32_t cnt[kSortWaves][kSortMaxBuckets];  // per wave: running count, then staging base
    uint32_t gbase[kSortMaxBuckets];        // next output slot of each bucket
    uint32_t gdelta[kSortMaxBuckets];       // output slot - staging position
    uint32_t stage_k[kSortThreads * ITEMS];
    uint32_t stage_v[VALS ? kSortThreads * ITEMS : 1];
    uint32_t s_wave[kSortWaves];
    uint32_t s_real;
};

// This wave's 64 * ITEMS keys of the tile starting at `first`, in input order: slot s of
// lane l is element s*64 + l of the wave's segment. All loads are issued
// before any is used. Returns whether the whole segment lies below n.
template <int VALS, int ITEMS>
__device__ __forceinline__ bool load_tile(const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals_in,
                                          int64_t n, int64_t first, uint32_t (&key)[ITEMS], uint32_t (&val)[ITEMS])
{
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
    const int64_t seg = first + (int64_t)wave * (kWave * ITEMS);
    const bool whole = seg + kWave * ITEMS <= n;
    if (whole) {
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            key[s] = keys[seg + s * kWave + lane];
            if constexpr (VALS == 1) val[s] = vals_in[seg + s * kWave + lane];
        }
    } else {
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            const int64_t i = seg + s * kWave + lane;
            key[s] = i < n ? keys[i] : 0u;
            if constexpr (VALS == 1) val[s] = i < n ? vals_in[i] : 0u;
        }
    }
    return whole;
}

// Each key's rank among this wave's keys of the same bucket that come before
// it, packed with its bucket as (bucket << 16) | rank; `cnt` (this wave's
// per-bucket counts, zero on entry) ends as the wave's bucket counts. WHOLE:
// every key of the wave's segment lies below n.
template <typename DIG, int VALS, int BITS, bool WHOLE, int ITEMS>
__device__ __forceinline__ void rank_in_wave(uint32_t* cnt, const uint32_t (&key)[ITEMS], uint32_t (&val)[ITEMS],
                                             uint32_t (&dr)[ITEMS], int64_t seg,
                                             int64_t n, DIG dig)
{
    constexpr bool kSpare = !WHOLE || DIG::kSpareKeys;
    const uint32_t B = dig.buckets;
    const int lane = lane_id();
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int64_t i = seg + s * kWave + lane;
        if constexpr (VALS == 2) val[s] = (uint32_t)i;
        const uint32_t d = (WHOLE || i < n) ? dig.template digit<BITS>(key[s]) : B;
        const uint64_t peers = match_digit<BITS, kSpare>(d, B);
        const uint32_t below = lanes_below_mask(peers);
        const uint32_t run = cnt[d];
        if (below == 0) cnt[d] = run + (uint32_t)__builtin_popcountll(peers);
        dr[s] = (d << 16) | (run + below);
    }
}

// VALS: 0 keys only; 1 values from vals_in follow the keys; 2 the value is the
// element's index and only values are written (MoE: the assignment index).
// The tile's loaded keys, starting at `first` (< n): rank, then
// stage it in LDS ordered by bucket; gbase must hold each bucket's first
// output slot for this tile, and gdelta ends mapping staging positions to
// output slots. Every thread of the workgroup calls it; ends with a barrier.
template <typename DIG, int VALS, int BITS, int ITEMS>
__device__ __forceinline__ void rank_and_stage(SortLds<VALS, ITEMS>& sh, const uint32_t (&key)[ITEMS],
                                               uint32_t (&val)[ITEMS], bool whole, int64_t n, DIG dig,
                                               int64_t first)
{
    const uint32_t B = dig.buckets;  // real buckets; B itself is the spare one
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
    const int64_t seg = first + (int64_t)wave * (kWave * ITEMS);
    for (uint32_t d = lane; d <= B; d += kWave) sh.cnt[wave][d] = 0;
    uint32_t dr[ITEMS];
    // Rank among this wave's keys of the same bucket, in input order.
    if (whole)
        rank_in_wave<DIG, VALS, BITS, true, ITEMS>(sh.cnt[wave], key, val, dr, seg, n, dig);
    else
        rank_in_wave<DIG, VALS, BITS, false, ITEMS>(sh.cnt[wave], key, val, dr, seg, n, dig);
    __syncthreads();
    tile_bases(sh.cnt, sh.gbase, sh.gdelta, sh.s_wave, &sh.s_real, B);
    __syncthreads();
    // Stage the tile ordered by bucket, equal buckets in input order.
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const uint32_t p = sh.cnt[wave][dr[s] >> 16] + (dr[s] & 0xFFFFu);
        if (p < (uint32_t)(kSortThreads * ITEMS)) {
            sh.stage_k[p] = key[s];
            if constexpr (VALS != 0) sh.stage_v[p] = val[s];
        }
    }
    __syncthreads();
}

// Each bucket's run of the staged tile goes to its slots; the spare
// bucket's keys, staged last, are not written.
template <typename DIG, int VALS, int BITS, int ITEMS>
__device__ __forceinline__ void write_runs(const SortLds<VALS, ITEMS>& sh, uint32_t* __restrict__ keys_out,
                                           uint32_t* __restrict__ vals_out, DIG dig, int64_t out_cap)
{
    const uint32_t B = dig.buckets;
    const uint32_t real = sh.s_real;
    if constexpr (VALS == 0) {
        if (real == kSortThreads * ITEMS && out_cap > 0) {
            // A whole tile of keys, all in real buckets: each thread takes
            // ITEMS of them with every LDS read issued up front, where the
            // loop below waits on two dependent reads per key. (Keys only:
            // with values the same form was 7% slower at 2^28 pairs.)
            uint32_t k[ITEMS], pos[ITEMS];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) k[i] = sh.stage_k[threadIdx.x + i * kSortThreads];
#pragma unroll
            for (int i = 0; i < ITEMS; ++i)
                pos[i] = sh.gdelta[dig.template digit<BITS>(k[i])] + threadIdx.x + (uint32_t)(i * kSortThreads);
            // pos < out_cap as a 32-bit compare (pos is 32-bit)
            const uint32_t last = out_cap > (int64_t)0xFFFFFFFFu ? 0xFFFFFFFFu : (uint32_t)(out_cap - 1);
#pragma unroll
            for (int i = 0; i < ITEMS; ++i)
                if (pos[i] <= last) keys_out[pos[i]] = k[i];
            return;
        }
    }
    for (uint32_t j = threadIdx.x; j < real; j += kSortThreads) {
        const uint32_t k = sh.stage_k[j];
        const uint32_t d = dig.template digit<BITS>(k);
        const uint64_t pos = (uint64_t)(uint32_t)(sh.gdelta[d] + j);
        if (d < B && pos < (uint64_t)out_cap) {
            if constexpr (VALS != 2) keys_out[pos] = k;
            if constexpr (VALS != 0) vals_out[pos] = sh.stage_v[j];
        }
    }
}

// MoE outputs of the scatter: with hist set, every workgroup derives the
// experts' block-rounded offsets from the scanned table and places its keys
// at them; workgroup 0 also writes the counts, the offsets and the padding.
struct MoeSlots {
    const uint32_t* hist;  // the unscanned table (its last entry completes the total); null: a radix pass
    int block;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted;
};

// gbase[e] for MoE: expert e's padded start plus the keys of e in earlier
// tiles. Thread e takes expert e.
__device__ __forceinline__ void moe_bases(uint32_t* gbase, uint32_t* s_wave, const uint32_t* __restrict__ slots,
                                          int64_t tiles, int64_t tile, uint32_t E, const MoeSlots& moe, int64_t n)
{
    const uint32_t e = threadIdx.x;
    const uint32_t last = slots[(int64_t)E * tiles - 1] + moe.hist[(int64_t)E * tiles - 1];
    uint32_t lo = 0, c = 0;
    if (e < E) {
        lo = slots[(int64_t)e * tiles];
        c = (e + 1 < E ? slots[(int64_t)(e + 1) * tiles] : last) - lo;
    }
    const uint32_t b = (uint32_t)moe.block;
    const uint32_t r = (c + b - 1) / b * b;
    uint32_t total;
    const uint32_t off = block_exclusive_u32(r, s_wave, total);
    if (e < E) gbase[e] = off + (slots[(int64_t)e * tiles + tile] - lo);
    if (blockIdx.x == 0) {
        if (e < E) {
            moe.counts[e] = (int32_t)c;
            moe.offsets[e] = (int32_t)off;
            for (uint32_t j = c; j < r; ++j) moe.sorted[off + j] = (int32_t)n;
        }
        if (threadIdx.x == 0) moe.offsets[E] = (int32_t)total;
    }
}

// One tile per workgroup (neighbouring tiles, which share a cache line at
// each bucket's run boundary, are then written at the same time). Its first
// slot for bucket d is its group's entry of the scanned table plus, after
// the group's first tile, its row of the group prefixes.
template <typename DIG, int VALS, int BITS, int ITEMS, int GROUP>
__global__ __launch_bounds__(kSortThreads) void digit_scatter_kernel(
    const uint32_t* __restrict__ keys, const uint32_t* __restrict__ vals_in, uint32_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, int64_t n, DIG dig, const uint32_t* __restrict__ slots,
    const uint16_t* __restrict__ pre, MoeSlots moe, int64_t groups, int64_t out_cap)
{
    static_assert(GROUP == 1 || VALS != 2, "MoE offsets are read per tile");
    __shared__ SortLds<VALS, ITEMS> sh;
    const int64_t tile = xcd_contiguous_tile();
    const int64_t first = tile * (int64_t)(kSortThreads * ITEMS);
    if (first >= n) return;  // uniform over the workgroup
    // The tile's keys are requested first, so their latency overlaps the
    // reads of its column of the scanned table.
    uint32_t key[ITEMS], val[ITEMS];
    const bool whole = load_tile<VALS, ITEMS>(keys, vals_in, n, first, key, val);
    if (moe.hist) {
        moe_bases(sh.gbase, sh.s_wave, slots, groups, tile, dig.buckets, moe, n);
    } else {
        const int64_t g = tile / GROUP;
        const bool later = GROUP > 1 && tile % GROUP != 0;
        for (uint32_t d = threadIdx.x; d < dig.buckets; d += kSortThreads)
            sh.gbase[d] = slots[(int64_t)d * groups + g] + (later ? pre[tile * dig.buckets + d] : 0u);
    }
    __syncthreads();
    rank_and_stage<DIG, VALS, BITS, ITEMS>(sh, key, val, whole, n, dig, first);
    write_runs<DIG, VALS, BITS, ITEMS>(sh, keys_out, vals_out, dig, out_cap);
}

// MoE alignment of up to kMoeOneLaunchMax ids in one launch of one
// workgroup of 1,024 threads (16 waves). Wave w ranks the ids of its own
// contiguous segment in input order (the same ballot match and per-wave LDS
// counters as above), then thread e, for expert e, turns the 16 waves'
// counts into the expert's count, its block-rounded offset (a workgroup
// scan), the padding marks and each wave's first slot, and every lane writes
// its ids' indices straight to their slots.
constexpr int kMoeWaves = 16;
constexpr int kMoeThreadsOne = kMoeWaves * kWave;
constexpr int kMoeSlots = 8;  // ids per lane
constexpr int64_t kMoeOneLaunchMax = (int64_t)kMoeThreadsOne * kMoeSlots;

template <int BITS>
__global__ __launch_bounds__(kMoeThreadsOne) void moe_align_one_launch_kernel(const uint32_t* __restrict__ ids,
                                                                             int64_t n, ExpertDigit dig, int block,
                                                                             int32_t* __restrict__ counts,
                                                                             int32_t* __restrict__ offsets,
                                                                             int32_t* __restrict__ sorted)
{
    __shared__ uint32_t cnt[kMoeWaves][kSortMaxBuckets];
    __shared__ uint32_t s_count[kSortMaxBuckets], s_off[kSortMaxBuckets], s_round[kSortMaxBuckets];
    __shared__ uint32_t s_wave[kMoeWaves];
    const uint32_t E = dig.buckets;
    const int lane = lane_id(), wave = (int)(threadIdx.x / kWave);
    // Wave w's segment: seg_len ids from w * seg_len, seg_len a multiple of 64.
    // The ids are requested first; the counters are cleared while they load.
    const int64_t seg_len = (n + kMoeThreadsOne - 1) / kMoeThreadsOne * kWave;
    const int slots = (int)(seg_len / kWave);
    const int64_t seg = (int64_t)wave * seg_len;
    uint32_t key[kMoeSlots];
#pragma unroll
    for (int s = 0; s < kMoeSlots; ++s) {
        const int64_t i = seg + s * kWave + lane;
        key[s] = (s < slots && i < n) ? ids[i] : 0u;
    }
    for (uint32_t i = threadIdx.x; i < kMoeWaves * kSortMaxBuckets; i += kMoeThreadsOne) (&cnt[0][0])[i] = 0;
    __syncthreads();
    uint32_t dr[kMoeSlots];
#pragma unroll
    for (int s = 0; s < kMoeSlots; ++s) {
        if (s < slots) {  // uniform
            const int64_t i = seg + s * kWave + lane;
            const uint32_t d = i < n ? dig(key[s]) : E;
            const uint64_t peers = match_digit<BITS, true>(d, E);
            const uint32_t below = lanes_below_mask(peers);
            const uint32_t run = cnt[wave][d];
            if (below == 0) cnt[wave][d] = run + (uint32_t)__builtin_popcountll(peers);
            dr[s] = (d << 16) | (run + below);
        }
    }
    __syncthreads();
    // Thread e: expert e's count over the waves, its rounded offset, the
    // waves' first slots, and the padding marks.
    const uint32_t e = threadIdx.x;
    uint32_t c = 0, pw[kMoeWaves];
#pragma unroll
    for (int w = 0; w < kMoeWaves; ++w) {
        pw[w] = c;
        if (e < E) c += cnt[w][e];
    }
    const uint32_t r = (c + block - 1) / block * block;
    const uint32_t incl = wave_inclusive_scan(r);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kMoeWaves; ++w)
        if (w < wave) before += s_wave[w];
    const uint32_t off = before + incl - r;
    if (e < E) {
        counts[e] = (int32_t)c;
        offsets[e] = (int32_t)off;
#pragma unroll
        for (int w = 0; w < kMoeWaves; ++w) cnt[w][e] = off + pw[w];
        s_count[e] = c;
        s_off[e] = off;
        s_round[e] = r;
    }
    if (e == E) offsets[E] = (int32_t)off;  // r = 0 here: the padded total
    __syncthreads();
    // Padding marks: wave w takes experts w, w + 16, ...; its lanes write the
    // unused slots of the expert's rounded segment side by side.
    for (uint32_t x = wave; x < E; x += kMoeWaves) {
        const uint32_t cx = s_count[x], ox = s_off[x], rx = s_round[x];
        for (uint32_t j = cx + lane; j < rx; j += kWave) sorted[ox + j] = (int32_t)n;
    }
#pragma unroll
    for (int s = 0; s < kMoeSlots; ++s) {
        if (s < slots) {
            const uint32_t d = dr[s] >> 16;
            if (d < E) sorted[cnt[wave][d] + (dr[s] & 0xFFFFu)] = (int32_t)(seg + s * kWave + lane);
        }
    }
}

// GROUP: tiles per entry of the count table. For a radix pass hist and slots
// are the same buffer (scanned in place) and pre follows the table in it.
template <typename DIG, int VALS, int ITEMS, int GROUP>
static hipError_t counting_sort_typed(const uint32_t* keys, const uint32_t* vals_in, uint32_t* keys_out,
                                      uint32_t* vals_out, int64_t n, DIG dig, uint32_t* hist, uint32_t* slots,
                                      uint16_t* pre, const MoeSlots& moe, int64_t out_cap, const DevWs& ws,
                                      uint32_t spin_limit, hipStream_t st)
{
    const int64_t tile_elems = (int64_t)kSortThreads * ITEMS;
    const int64_t tiles = (n + tile_elems - 1) / tile_elems, groups = (tiles + GROUP - 1) / GROUP;
    if (GROUP > 1 && !pre) return hipErrorInvalidValue;
    const dim3 block(kSortThreads);
    if (aligned16(keys))
        digit_count_kernel<DIG, true, ITEMS, GROUP><<<dim3((unsigned)groups), block, 0, st>>>(keys, n, dig, hist, pre,
                                                                                           groups, tiles);
    else
        digit_count_kernel<DIG, false, ITEMS, GROUP><<<dim3((unsigned)groups), block, 0, st>>>(keys, n, dig, hist, pre,
                                                                                            groups, tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_lookback_scan(kU32, false, hist, slots, (int64_t)dig.buckets * groups, ws, spin_limit, st);
    if (e != hipSuccess) return e;
    const int bits = dig.buckets > 1 ? 32 - __builtin_clz(dig.buckets - 1) : 0;
#define DS_SCATTER(BITS)                                                                                      \
    digit_scatter_kernel<DIG, VALS, BITS, ITEMS, GROUP><<<dim3((unsigned)tiles), block, 0, st>>>(             \
        keys, vals_in, keys_out, vals_out, n, dig, slots, pre, moe, groups, out_cap);                         \
    break
    switch (bits) {
    case 0: DS_SCATTER(0);
    case 1: DS_SCATTER(1);
    case 2: DS_SCATTER(2);
    case 3: DS_SCATTER(3);
    case 4: DS_SCATTER(4);
    case 5: DS_SCATTER(5);
    case 6: DS_SCATTER(6);
    case 7: DS_SCATTER(7);
    case 8: DS_SCATTER(8);
    case 9: DS_SCATTER(9);
    default: return hipErrorInvalidValue;
    }
#undef DS_SCATTER
    return hipGetLastError();
}


int64_t moe_one_launch_max() { return kMoeOneLaunchMax; }
int64_t sort_tile_elems(bool values) { return (int64_t)kSortThreads * (values ? kRadixKvItems : kRadixItems); }
static int64_t sort_tiles(bool values, int64_t n) { return (n + sort_tile_elems(values) - 1) / sort_tile_elems(values); }
int64_t sort_table_columns(bool values, int64_t n)
{
    const int64_t group = values ? kRadixKvGroup : kRadixGroup;
    return (sort_tiles(values, n) + group - 1) / group;
}
int64_t sort_aux_words(bool values, int64_t n, int bits)
{
    return ((int64_t)1 << bits) * (sort_table_columns(values, n) + sort_tiles(values, n));
}
int64_t moe_tile_elems() { return (int64_t)kSortThreads * kMoeItems; }
int sort_max_buckets() { return kSortMaxBuckets - 1; }

hipError_t launch_radix_pass(const uint32_t* keys, const uint32_t* vals_in, uint32_t* keys_out, uint32_t* vals_out,
                             int64_t n, int shift, int bits, uint32_t* table, const DevWs& ws, uint32_t spin_limit,
                             hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    if (!table) return hipErrorInvalidValue;
    const RadixDigit dig{(uint32_t)shift, (1u << bits) - 1u, 1u << bits};
    const MoeSlots none{nullptr, 0, nullptr, nullptr, nullptr};
    // the table (buckets x groups, scanned in place), then the group prefixes (buckets x tiles)
    uint16_t* pre = reinterpret_cast<uint16_t*>(table + (int64_t)dig.buckets * sort_table_columns(vals_in != nullptr, n));
    if (vals_in)
        return counting_sort_typed<RadixDigit, 1, kRadixKvItems, kRadixKvGroup>(keys, vals_in, keys_out, vals_out, n, dig,
                                                                              table, table, pre, none, n, ws, spin_limit,
                                                                              stream);
    return counting_sort_typed<RadixDigit, 0, kRadixItems, kRadixGroup>(keys, nullptr, keys_out, nullptr, n, dig, table,
                                                                      table, pre, none, n, ws, spin_limit, stream);
}

hipError_t launch_moe_align(const int32_t* ids, int64_t n, int experts, const MoeOut& out, uint32_t* hist,
                            uint32_t* slots, const DevWs& ws, uint32_t spin_limit, hipStream_t stream)
{
    if (!hist || !slots) return hipErrorInvalidValue;
    const ExpertDigit dig{(uint32_t)experts};
    if (n <= kMoeOneLaunchMax) {
        const int bits = experts > 1 ? 32 - __builtin_clz((uint32_t)experts - 1) : 0;
#define DS_MOE_ONE(BITS)                                                                                     \
    moe_align_one_launch_kernel<BITS><<<dim3(1), dim3(kMoeThreadsOne), 0, stream>>>(                        \
        (const uint32_t*)ids, n, dig, out.block, out.counts, out.offsets, out.sorted);                     \
    break
        switch (bits) {
        case 0: DS_MOE_ONE(0);
        case 1: DS_MOE_ONE(1);
        case 2: DS_MOE_ONE(2);
        case 3: DS_MOE_ONE(3);
        case 4: DS_MOE_ONE(4);
        case 5: DS_MOE_ONE(5);
        case 6: DS_MOE_ONE(6);
        case 7: DS_MOE_ONE(7);
        case 8: DS_MOE_ONE(8);
        case 9: DS_MOE_ONE(9);
        default: return hipErrorInvalidValue;
        }
#undef DS_MOE_ONE
        return hipGetLastError();
    }
    const MoeSlots moe{hist, out.block, out.counts, out.offsets, out.sorted};
    return counting_sort_typed<ExpertDigit, 2, kMoeItems, 1>((const uint32_t*)ids, nullptr, nullptr, (uint32_t*)out.sorted,
                                                             n, dig, hist, slots, nullptr, moe, out.capacity, ws,
                                                             spin_limit, stream);
}

}  // namespace ds
