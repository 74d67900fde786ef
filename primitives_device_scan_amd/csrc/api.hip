// api.hip -- the C ABI of include/devscan.h: argument validation on the host,
// the per-(device, stream) workspace, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <map>
#include <mutex>
#include <utility>

#include "devscan.h"
#include "launch.hpp"
#include "tile.hpp"

// Scratch of ds_scan_noalloc (see below); 256-byte aligned like a HIP allocation.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

__global__ void noalloc_clear_kernel(uint64_t* p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

namespace {

using ds::Ctrl;
using ds::DevWs;

// Workspace layout: [Ctrl][status: one 128-byte line per tile][totals: 8 B per
// tile]; `aux` is a separate scratch buffer for the counting-sort tables.
struct Workspace {
    char* base = nullptr;
    int64_t tile_cap = 0;
    uint64_t lookback_launches = 0;  // launches that stamped an epoch since the last clear
    char* aux = nullptr;
    size_t aux_cap = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
uint32_t g_spin_limit = 1u << 20;
int g_fail_allocs = -1;  // workspace allocations still to refuse (testing hook); -1: not read from the environment yet

constexpr uint32_t kDefaultSpin = 1u << 20;
// Epochs are 30 bits: clear the status words well before one comes round again.
constexpr uint64_t kEpochClearPeriod = 1ull << 29;
// Largest n: the grid (tiles x 256 work-items) must stay below 2^32 work-items.
constexpr int64_t kMaxTiles = ((int64_t)1 << 32) / ds::kThreads - 1;
constexpr size_t kStatusBytes = (size_t)ds::kStatusWords * sizeof(uint64_t);  // per tile

size_t ws_bytes(int64_t tiles) { return sizeof(Ctrl) + (size_t)tiles * (kStatusBytes + 8); }

DevWs view(const Workspace& w)
{
    DevWs d;
    d.ctrl = reinterpret_cast<Ctrl*>(w.base);
    d.status = reinterpret_cast<uint64_t*>(w.base + sizeof(Ctrl));
    d.totals = w.base + sizeof(Ctrl) + (size_t)w.tile_cap * kStatusBytes;
    return d;
}

// True when `stream` is being captured into a graph: the workspace may then
// be used but not allocated, grown or cleared (those are not kernel launches).
bool capturing(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs != hipStreamCaptureStatusNone;
}

// Testing hook: DEVSCAN_FAIL_ALLOCS=k in the environment (read once) or
// ds_fail_next_allocations(k) makes the next k workspace allocations report
// DS_ERR_OUT_OF_MEMORY without calling hipMalloc.
bool refuse_allocation()
{
    if (g_fail_allocs < 0) {
        const char* s = getenv("DEVSCAN_FAIL_ALLOCS");
        g_fail_allocs = s ? atoi(s) : 0;
        if (g_fail_allocs < 0) g_fail_allocs = 0;
    }
    if (g_fail_allocs == 0) return false;
    --g_fail_allocs;
    return true;
}

// Returns the workspace of (current device, stream) with room for `tiles`;
// a new allocation is cleared on the stream before any kernel uses it.
int get_workspace(hipStream_t stream, int64_t tiles, Workspace** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    Workspace& w = g_ws[{dev, stream}];
    const bool grow = w.tile_cap < tiles;
    const bool clear = w.lookback_launches >= kEpochClearPeriod;
    if ((grow || clear) && capturing(stream)) return DS_ERR_STREAM_CAPTURING;
    if (grow) {
        int64_t cap = w.tile_cap * 2 > tiles ? w.tile_cap * 2 : tiles;
        if (cap < 1024) cap = 1024;
        if (refuse_allocation()) return DS_ERR_OUT_OF_MEMORY;
        if (w.base) {
            // The old buffer may still be in use by work queued on the stream.
            if (hipStreamSynchronize(stream) != hipSuccess) return DS_ERR_HIP;
            (void)hipFree(w.base);
            w.base = nullptr;
            w.tile_cap = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, ws_bytes(cap)) != hipSuccess) {
            (void)hipGetLastError();
            return DS_ERR_OUT_OF_MEMORY;
        }
        if (hipMemsetAsync(p, 0, ws_bytes(cap), stream) != hipSuccess) {
            (void)hipFree(p);
            return DS_ERR_HIP;
        }
        w.base = static_cast<char*>(p);
        w.tile_cap = cap;
        w.lookback_launches = 0;
    }
    if (w.lookback_launches >= kEpochClearPeriod) {
        if (hipMemsetAsync(w.base + sizeof(Ctrl), 0, (size_t)w.tile_cap * kStatusBytes, stream) != hipSuccess)
            return DS_ERR_HIP;
        w.lookback_launches = 0;
    }
    *out = &w;
    return DS_OK;
}

// Scratch of at least `bytes` for (current device, stream); its contents are
// undefined (every user writes what it reads).
int get_aux(hipStream_t stream, size_t bytes, char** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    Workspace& w = g_ws[{dev, stream}];
    if (w.aux_cap < bytes) {
        if (capturing(stream)) return DS_ERR_STREAM_CAPTURING;
        size_t cap = w.aux_cap * 2 > bytes ? w.aux_cap * 2 : bytes;
        if (cap < ((size_t)1 << 20)) cap = (size_t)1 << 20;
        if (refuse_allocation()) return DS_ERR_OUT_OF_MEMORY;
        if (w.aux) {
            if (hipStreamSynchronize(stream) != hipSuccess) return DS_ERR_HIP;
            (void)hipFree(w.aux);
            w.aux = nullptr;
            w.aux_cap = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, cap) != hipSuccess) {
            (void)hipGetLastError();
            return DS_ERR_OUT_OF_MEMORY;
        }
        w.aux = static_cast<char*>(p);
        w.aux_cap = cap;
    }
    *out = w.aux;
    return DS_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free look-back scan (ds_scan_noalloc): its control block and
// status words live in `scratch`, a fixed array in the library's own device
// memory, one copy per GPU, held until the process ends. Host code never
// passes `scratch` itself to a kernel (in host code the name is a host-side
// stand-in); it takes each device's address once with hipGetSymbolAddress and
// uses that.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocMaxTiles = (int64_t)((kNoAllocScratchBytes - sizeof(Ctrl)) / kStatusBytes);

struct NoAllocDev {
    char* ptr = nullptr;           // device address of this GPU's `scratch`
    bool cleared = false;          // the clear kernel has been enqueued once
    uint64_t launches = 0;         // launches since the last clear (epoch wrap guard)
};
std::map<int, NoAllocDev> g_noalloc;  // per device, guarded by g_mu

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

// The look-back workspace for an exclusive uint32 scan of `words` entries
// (none when it fits one tile).
int scan_workspace_u32(hipStream_t stream, int64_t words, DevWs* dws, Workspace** w)
{
    const int64_t te = ds::tile_elems(ds::kU32, false, words);
    const int64_t tiles = (words + te - 1) / te;
    *dws = DevWs{nullptr, nullptr, nullptr};
    *w = nullptr;
    if (tiles <= 1) return DS_OK;
    const int st = get_workspace(stream, tiles, w);
    if (st == DS_OK) *dws = view(**w);
    return st;
}

bool valid_dtype(int dtype) { return dtype >= DS_INT32 && dtype <= DS_UINT64; }

int elem_bytes(int dtype) { return (dtype == DS_INT64 || dtype == DS_UINT64) ? 8 : 4; }

ds::ElemKind kind_of(int dtype)
{
    switch (dtype) {
    case DS_INT32: return ds::kI32;
    case DS_UINT32: return ds::kU32;
    case DS_FP32: return ds::kF32;
    case DS_INT64: return ds::kI64;
    default: return ds::kU64;
    }
}

// Checks shared by every entry point that reads n elements and writes n.
int check_io(int dtype, const void* in, const void* out, int64_t n, bool allow_same)
{
    if (!valid_dtype(dtype)) return DS_ERR_UNSUPPORTED_DTYPE;
    if (n < 0) return DS_ERR_INVALID_VALUE;
    if (n == 0) return DS_OK;
    if (!in || !out) return DS_ERR_INVALID_VALUE;
    const int64_t sz = elem_bytes(dtype);
    const int64_t smallest_tile = ds::lds_tile_elems();  // 4,096: the most tiles any entry point launches
    if ((n + smallest_tile - 1) / smallest_tile > kMaxTiles) return DS_ERR_TOO_LARGE;
    if (((uintptr_t)in % sz) || ((uintptr_t)out % sz)) return DS_ERR_MISALIGNED;
    const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out, len = (uintptr_t)(n * sz);
    if (a == b) return allow_same ? DS_OK : DS_ERR_OVERLAP;
    if (a < b + len && b < a + len) return DS_ERR_OVERLAP;
    return DS_OK;
}

// seed (look-back only): null, or one element of dtype in device memory added
// to every prefix.
int scan_impl(int dtype, int inclusive, int algo, const void* in, void* out, int64_t n, hipStream_t stream,
              const void* seed = nullptr)
{
    if (inclusive != 0 && inclusive != 1) return DS_ERR_INVALID_VALUE;
    if (algo < DS_ALGO_DEFAULT || algo > DS_ALGO_LOOKBACK_BLOCKED) return DS_ERR_INVALID_VALUE;
    int st = check_io(dtype, in, out, n, true);
    if (st != DS_OK || n == 0) return st;
    if (algo == DS_ALGO_LOOKBACK_BLOCKED) {
        if (elem_bytes(dtype) != 4) return DS_ERR_UNSUPPORTED_DTYPE;
        const int64_t bt = ds::blocked_tile_elems(n);
        const int64_t btiles = (n + bt - 1) / bt;
        std::lock_guard<std::mutex> lock(g_mu);
        DevWs dws{nullptr, nullptr, nullptr};
        Workspace* w = nullptr;
        if (btiles > 1) {
            st = get_workspace(stream, btiles, &w);
            if (st != DS_OK) return st;
            dws = view(*w);
        }
        const hipError_t e =
            ds::launch_lookback_blocked(kind_of(dtype), inclusive != 0, in, out, n, dws, g_spin_limit, stream);
        if (w && e == hipSuccess) ++w->lookback_launches;
        return e == hipSuccess ? DS_OK : DS_ERR_HIP;
    }
    // Choose the kernel first, then size the workspace by that kernel's own
    // tiles: the look-back and three-pass tiles differ in size, and a
    // three-pass call on one tile runs the look-back kernel instead.
    const int64_t tp = ds::three_pass_tile_elems(elem_bytes(dtype));
    const bool three = algo == DS_ALGO_THREE_PASS && n > tp;
    const int64_t te = three ? tp : ds::tile_elems(kind_of(dtype), inclusive != 0, n);
    const int64_t tiles = (n + te - 1) / te;
    std::lock_guard<std::mutex> lock(g_mu);
    DevWs dws{nullptr, nullptr, nullptr};
    Workspace* w = nullptr;
    if (tiles > 1) {
        st = get_workspace(stream, tiles, &w);
        if (st != DS_OK) return st;
        dws = view(*w);
    }
    hipError_t e;
    if (three) {
        e = ds::launch_three_pass_scan(kind_of(dtype), inclusive != 0, in, out, n, dws, stream);
    } else {
        e = ds::launch_lookback_scan(kind_of(dtype), inclusive != 0, in, out, n, dws, g_spin_limit, stream, seed);
        if (w && e == hipSuccess) ++w->lookback_launches;
    }
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

}  // namespace

extern "C" {

int scan_exclusive(int dtype, const void* d_in, void* d_out, int64_t n, hipStream_t stream)
{
    return scan_impl(dtype, 0, DS_ALGO_DEFAULT, d_in, d_out, n, stream);
}

int scan_inclusive(int dtype, const void* d_in, void* d_out, int64_t n, hipStream_t stream)
{
    return scan_impl(dtype, 1, DS_ALGO_DEFAULT, d_in, d_out, n, stream);
}

int ds_scan(int dtype, int inclusive, int algo, const void* d_in, void* d_out, int64_t n, hipStream_t stream)
{
    return scan_impl(dtype, inclusive, algo, d_in, d_out, n, stream);
}

int ds_scan_seeded(int dtype, int inclusive, const void* d_in, void* d_out, int64_t n, const void* d_seed,
                   hipStream_t stream)
{
    if (inclusive != 0 && inclusive != 1) return DS_ERR_INVALID_VALUE;
    const int st = check_io(dtype, d_in, d_out, n, true);  // the input and output first, as for every scan
    if (st != DS_OK || n == 0) return st;
    if (d_seed) {
        const int64_t sz = elem_bytes(dtype);
        if ((uintptr_t)d_seed % sz) return DS_ERR_MISALIGNED;
        if (overlaps(d_seed, (size_t)sz, d_out, (size_t)(n * sz))) return DS_ERR_OVERLAP;
    }
    return scan_impl(dtype, inclusive, DS_ALGO_LOOKBACK, d_in, d_out, n, stream, d_seed);
}

int ds_scan_noalloc(int dtype, int inclusive, const void* d_in, void* d_out, int64_t n, hipStream_t stream)
{
    if (inclusive != 0 && inclusive != 1) return DS_ERR_INVALID_VALUE;
    int st = check_io(dtype, d_in, d_out, n, true);
    if (st != DS_OK || n == 0) return st;
    const int64_t te = ds::tile_elems(kind_of(dtype), inclusive != 0, n);
    const int64_t tiles = (n + te - 1) / te;
    if (tiles > kNoAllocMaxTiles) return DS_ERR_TOO_LARGE;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    NoAllocDev& d = g_noalloc[dev];
    if (!d.ptr) {
        // Once per device, with that device current: this GPU's copy of the array.
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return DS_ERR_HIP;
        }
        d.ptr = static_cast<char*>(p);
    }
    DevWs dws{nullptr, nullptr, nullptr};
    if (tiles > 1) {
        if (!d.cleared || d.launches >= kEpochClearPeriod) {
            // Zero the control block and every status word (a kernel, so that
            // a captured call records no memset node); stream-ordered before
            // the scan below.
            const int64_t words = (int64_t)(kNoAllocScratchBytes / sizeof(uint64_t));
            noalloc_clear_kernel<<<dim3(256), dim3(256), 0, stream>>>(reinterpret_cast<uint64_t*>(d.ptr), words);
            if (hipGetLastError() != hipSuccess) return DS_ERR_HIP;
            d.cleared = true;
            d.launches = 0;
        }
        dws.ctrl = reinterpret_cast<Ctrl*>(d.ptr);
        dws.status = reinterpret_cast<uint64_t*>(d.ptr + sizeof(Ctrl));
    }
    const hipError_t e =
        ds::launch_lookback_scan(kind_of(dtype), inclusive != 0, d_in, d_out, n, dws, g_spin_limit, stream);
    if (e != hipSuccess) return DS_ERR_HIP;
    if (tiles > 1) ++d.launches;
    return DS_OK;
}

int compact_if(int dtype, const void* d_in, void* d_out, int64_t* d_num_selected, int64_t n, int cmp,
               uint64_t operand_bits, hipStream_t stream)
{
    if (!valid_dtype(dtype)) return DS_ERR_UNSUPPORTED_DTYPE;
    if (cmp < DS_LT || cmp > DS_NE) return DS_ERR_INVALID_VALUE;
    if (!d_num_selected || n < 0) return DS_ERR_INVALID_VALUE;
    if (((uintptr_t)d_num_selected) % 8) return DS_ERR_MISALIGNED;
    if (n >= ((int64_t)1 << 32)) return DS_ERR_TOO_LARGE;
    int st = check_io(dtype, d_in, d_out, n, true);
    if (st != DS_OK) return st;
    if (n == 0)  // nothing to scan: the count is 0, written by a one-thread kernel (capturable)
        return ds::launch_write_count(d_num_selected, 0, stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
    const int64_t ct = ds::compact_tile_elems(elem_bytes(dtype));
    const int64_t tiles = (n + ct - 1) / ct;
    std::lock_guard<std::mutex> lock(g_mu);
    DevWs dws{nullptr, nullptr, nullptr};
    Workspace* w = nullptr;
    if (tiles > 1) {
        st = get_workspace(stream, tiles, &w);
        if (st != DS_OK) return st;
        dws = view(*w);
    }
    const hipError_t e = ds::launch_compact(kind_of(dtype), d_in, d_out, d_num_selected, n, cmp, operand_bits, dws,
                                            g_spin_limit, stream);
    if (w && e == hipSuccess) ++w->lookback_launches;
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_compact_unordered(int dtype, const void* d_in, void* d_out, int64_t* d_num_selected, int64_t n, int cmp,
                         uint64_t operand_bits, int claim, hipStream_t stream)
{
    if (!valid_dtype(dtype)) return DS_ERR_UNSUPPORTED_DTYPE;
    if (cmp < DS_LT || cmp > DS_NE) return DS_ERR_INVALID_VALUE;
    if (claim != DS_CLAIM_PER_WAVE && claim != DS_CLAIM_PER_WORKGROUP) return DS_ERR_INVALID_VALUE;
    if (!d_num_selected || n < 0) return DS_ERR_INVALID_VALUE;
    if (((uintptr_t)d_num_selected) % 8) return DS_ERR_MISALIGNED;
    if (n >= ((int64_t)1 << 32)) return DS_ERR_TOO_LARGE;
    int st = check_io(dtype, d_in, d_out, n, false);  // out is written in any order: never in place
    if (st != DS_OK) return st;
    if (n == 0)  // nothing to scan: the count is 0, written by a one-thread kernel (capturable)
        return ds::launch_write_count(d_num_selected, 0, stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
    return ds::launch_compact_unordered(kind_of(dtype), d_in, d_out, d_num_selected, n, cmp, operand_bits,
                                        claim == DS_CLAIM_PER_WORKGROUP, stream) == hipSuccess
               ? DS_OK
               : DS_ERR_HIP;
}

int ds_copy(const void* d_in, void* d_out, int64_t nbytes, hipStream_t stream)
{
    if (nbytes < 0 || (nbytes % 16)) return DS_ERR_INVALID_VALUE;
    if (nbytes == 0) return DS_OK;
    if (!d_in || !d_out) return DS_ERR_INVALID_VALUE;
    if (((uintptr_t)d_in % 16) || ((uintptr_t)d_out % 16)) return DS_ERR_MISALIGNED;
    const uintptr_t a = (uintptr_t)d_in, b = (uintptr_t)d_out, len = (uintptr_t)nbytes;
    if (a < b + len && b < a + len) return DS_ERR_OVERLAP;
    if (nbytes / ds::tile_bytes() >= kMaxTiles) return DS_ERR_TOO_LARGE;
    return ds::launch_copy(d_in, d_out, nbytes, stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_bandwidth_pattern(int mode, int vectors_per_thread, int layout, const void* d_in, void* d_out, int64_t nbytes,
                         hipStream_t stream)
{
    if (mode < 0 || mode > 5 || layout < 0 || layout > 1 || !ds::pattern_vpt_ok(vectors_per_thread))
        return DS_ERR_INVALID_VALUE;
    if (nbytes < 0 || (nbytes % 16)) return DS_ERR_INVALID_VALUE;
    if (nbytes == 0) return DS_OK;
    if (!d_out || (mode != 1 && !d_in)) return DS_ERR_INVALID_VALUE;
    if (((uintptr_t)d_in % 16) || ((uintptr_t)d_out % 16)) return DS_ERR_MISALIGNED;
    if (mode != 1) {
        const uintptr_t a = (uintptr_t)d_in, b = (uintptr_t)d_out, len = (uintptr_t)nbytes;
        if (a < b + len && b < a + len) return DS_ERR_OVERLAP;
    }
    if (nbytes / 4096 + 8 >= kMaxTiles) return DS_ERR_TOO_LARGE;
    return ds::launch_pattern(mode, vectors_per_thread, layout, d_in, d_out, nbytes, stream) == hipSuccess ? DS_OK
                                                                                                        : DS_ERR_HIP;
}

static int check_tile_args(int dtype, int variant, const void* in, void* out, int64_t n)
{
    if (!valid_dtype(dtype)) return DS_ERR_UNSUPPORTED_DTYPE;
    if (elem_bytes(dtype) != 4) return DS_ERR_UNSUPPORTED_DTYPE;
    if (variant < DS_TILE_TREE || variant > DS_TILE_HS) return DS_ERR_INVALID_VALUE;
    if (n >= ((int64_t)1 << 32)) return DS_ERR_TOO_LARGE;
    return check_io(dtype, in, out, n, true);
}

int ds_tile_scan(int dtype, int variant, const void* d_in, void* d_out, void* d_tile_sums, int64_t n,
                 hipStream_t stream)
{
    int st = check_tile_args(dtype, variant, d_in, d_out, n);
    if (st != DS_OK || n == 0) return st;
    if (((uintptr_t)d_tile_sums) % 4) return DS_ERR_MISALIGNED;
    return ds::launch_tile_scan(kind_of(dtype), variant, d_in, d_out, d_tile_sums, n, stream) == hipSuccess
               ? DS_OK
               : DS_ERR_HIP;
}

int ds_tile_pipeline(int dtype, int variant, const void* d_in, void* d_out, int64_t n, hipStream_t stream)
{
    int st = check_tile_args(dtype, variant, d_in, d_out, n);
    if (st != DS_OK || n == 0) return st;
    const int64_t tiles = (n + ds::lds_tile_elems() - 1) / ds::lds_tile_elems();
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace* w = nullptr;
    st = get_workspace(stream, tiles, &w);
    if (st != DS_OK) return st;
    return ds::launch_tile_pipeline(kind_of(dtype), variant, d_in, d_out, n, view(*w), stream) == hipSuccess
               ? DS_OK
               : DS_ERR_HIP;
}

int ds_query_timeout(hipStream_t stream, int* timed_out)
{
    if (!timed_out) return DS_ERR_INVALID_VALUE;
    *timed_out = 0;
    if (hipStreamSynchronize(stream) != hipSuccess) return DS_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_HIP;
    int from_scratch = 0;
    auto na = g_noalloc.find(dev);
    if (na != g_noalloc.end() && na->second.ptr && na->second.cleared) {
        // ds_scan_noalloc's flag: the same rule, on the device's scratch array
        Ctrl* c = reinterpret_cast<Ctrl*>(na->second.ptr);
        uint32_t flag = 0;
        if (hipMemcpy(&flag, &c->timeout, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return DS_ERR_HIP;
        if (flag) {
            na->second.cleared = false;  // the next ds_scan_noalloc clears every word first
            from_scratch = 1;
        }
    }
    auto it = g_ws.find({dev, stream});
    if (it == g_ws.end() || !it->second.base) {
        *timed_out = from_scratch;
        return DS_OK;
    }
    Workspace& w = it->second;
    Ctrl* c = reinterpret_cast<Ctrl*>(w.base);
    uint32_t flag = 0;
    if (hipMemcpy(&flag, &c->timeout, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return DS_ERR_HIP;
    if (flag) {
        // A wait that gave up may have let the last tile advance the epoch
        // before slower tiles read it, so their status words can carry the
        // next launch's epoch. The stream is idle: clear every status word
        // (and the flag) so the next launch starts from a clean array.
        if (hipMemset(w.base + sizeof(Ctrl), 0, (size_t)w.tile_cap * kStatusBytes) != hipSuccess) return DS_ERR_HIP;
        const uint32_t zero = 0;
        if (hipMemcpy(&c->timeout, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return DS_ERR_HIP;
        w.lookback_launches = 0;
    }
    *timed_out = (flag || from_scratch) ? 1 : 0;
    return DS_OK;
}

int ds_fail_next_allocations(int count)
{
    if (count < 0) return DS_ERR_INVALID_VALUE;
    std::lock_guard<std::mutex> lock(g_mu);
    g_fail_allocs = count;
    return DS_OK;
}

int ds_set_spin_limit(uint32_t polls)
{
    std::lock_guard<std::mutex> lock(g_mu);
    g_spin_limit = polls ? polls : kDefaultSpin;
    return DS_OK;
}

const char* ds_status_string(int status)
{
    switch (status) {
    case DS_OK: return "DS_OK";
    case DS_ERR_INVALID_VALUE: return "DS_ERR_INVALID_VALUE: bad argument (n < 0, null pointer, bad enum)";
    case DS_ERR_UNSUPPORTED_DTYPE: return "DS_ERR_UNSUPPORTED_DTYPE";
    case DS_ERR_OVERLAP: return "DS_ERR_OVERLAP: input and output partially overlap";
    case DS_ERR_OUT_OF_MEMORY: return "DS_ERR_OUT_OF_MEMORY: workspace allocation failed";
    case DS_ERR_HIP: return "DS_ERR_HIP: a HIP call or kernel launch failed";
    case DS_ERR_MISALIGNED: return "DS_ERR_MISALIGNED: pointer not aligned to the element size";
    case DS_ERR_TOO_LARGE: return "DS_ERR_TOO_LARGE: n beyond the entry point's limit";
    case DS_ERR_STREAM_CAPTURING:
        return "DS_ERR_STREAM_CAPTURING: the workspace would have to be allocated, grown or cleared while the "
               "stream is being captured (make one call on the stream before capturing)";
    default: return "unknown ds_status";
    }
}

int ds_radix_pass(const uint32_t* d_keys_in, uint32_t* d_keys_out, const uint32_t* d_vals_in, uint32_t* d_vals_out,
                  int64_t n, int shift, int bits, hipStream_t stream)
{
    if (n < 0 || bits < 1 || bits > 8 || shift < 0 || shift > 31 || shift + bits > 32) return DS_ERR_INVALID_VALUE;
    if ((d_vals_in == nullptr) != (d_vals_out == nullptr)) return DS_ERR_INVALID_VALUE;
    if (n == 0) return DS_OK;
    if (n >= ((int64_t)1 << 32)) return DS_ERR_TOO_LARGE;
    if (!d_keys_in || !d_keys_out) return DS_ERR_INVALID_VALUE;
    const void* ptrs[4] = {d_keys_in, d_keys_out, d_vals_in, d_vals_out};
    for (const void* p : ptrs)
        if ((uintptr_t)p % 4) return DS_ERR_MISALIGNED;
    const size_t bytes = (size_t)n * 4;
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j) {
            if (i == 0 && j == 2) continue;  // the two inputs may share memory: both are only read
            if (ptrs[i] && ptrs[j] && overlaps(ptrs[i], bytes, ptrs[j], bytes)) return DS_ERR_OVERLAP;
        }
    const int64_t words = ((int64_t)1 << bits) * ds::sort_table_columns(d_vals_in != nullptr, n);
    std::lock_guard<std::mutex> lock(g_mu);
    char* aux = nullptr;
    int st = get_aux(stream, (size_t)ds::sort_aux_words(d_vals_in != nullptr, n, bits) * 4, &aux);
    if (st != DS_OK) return st;
    DevWs dws;
    Workspace* w = nullptr;
    st = scan_workspace_u32(stream, words, &dws, &w);
    if (st != DS_OK) return st;
    const hipError_t e = ds::launch_radix_pass(d_keys_in, d_vals_in, d_keys_out, d_vals_out, n, shift, bits,
                                               reinterpret_cast<uint32_t*>(aux), dws, g_spin_limit, stream);
    if (w && e == hipSuccess) ++w->lookback_launches;
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

int ds_moe_align(const int32_t* d_topk_ids, int64_t n, int num_experts, int block, int32_t* d_counts,
                 int32_t* d_offsets, int32_t* d_sorted_ids, int64_t capacity, hipStream_t stream)
{
    if (n < 0 || block < 1 || num_experts < 1 || num_experts > ds::sort_max_buckets()) return DS_ERR_INVALID_VALUE;
    if (!d_counts || !d_offsets || !d_sorted_ids || (n > 0 && !d_topk_ids)) return DS_ERR_INVALID_VALUE;
    const int64_t worst = n + (int64_t)num_experts * (block - 1);
    if (worst >= ((int64_t)1 << 31)) return DS_ERR_TOO_LARGE;
    if (capacity < worst) return DS_ERR_INVALID_VALUE;
    const void* ptrs[4] = {d_topk_ids, d_counts, d_offsets, d_sorted_ids};
    const size_t sizes[4] = {(size_t)n * 4, (size_t)num_experts * 4, (size_t)(num_experts + 1) * 4,
                             (size_t)capacity * 4};
    for (int i = 0; i < 4; ++i) {
        if ((uintptr_t)ptrs[i] % 4) return DS_ERR_MISALIGNED;
        for (int j = i + 1; j < 4; ++j)
            if (ptrs[i] && ptrs[j] && overlaps(ptrs[i], sizes[i], ptrs[j], sizes[j])) return DS_ERR_OVERLAP;
    }
    const int64_t tiles = (n + ds::moe_tile_elems() - 1) / ds::moe_tile_elems();
    const int64_t words = (int64_t)num_experts * tiles;
    std::lock_guard<std::mutex> lock(g_mu);
    char* aux = nullptr;
    int st = get_aux(stream, (size_t)(2 * words + 1) * 4, &aux);
    if (st != DS_OK) return st;
    DevWs dws;
    Workspace* w = nullptr;
    st = scan_workspace_u32(stream, words, &dws, &w);
    if (st != DS_OK) return st;
    uint32_t* hist = reinterpret_cast<uint32_t*>(aux);
    uint32_t* slots = hist + words;
    const ds::MoeOut out{d_counts, d_offsets, d_sorted_ids, block, capacity};
    const hipError_t e = ds::launch_moe_align(d_topk_ids, n, num_experts, out, hist, slots, dws, g_spin_limit,
                                              stream);
    if (w && e == hipSuccess && n > 0) ++w->lookback_launches;
    return e == hipSuccess ? DS_OK : DS_ERR_HIP;
}

void ds_release_workspace(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ws.empty()) (void)hipDeviceSynchronize();
    for (auto& kv : g_ws) {
        if (kv.second.base) (void)hipFree(kv.second.base);
        if (kv.second.aux) (void)hipFree(kv.second.aux);
    }
    g_ws.clear();
}

int64_t ds_tile_elems(int dtype, int entry)
{
    if (!valid_dtype(dtype)) return -1;
    const int b = elem_bytes(dtype);
    switch (entry) {
    case DS_TILE_OF_SCAN_EXCLUSIVE: return ds::tile_elems(kind_of(dtype), false, INT64_MAX / 16);
    case DS_TILE_OF_SCAN_INCLUSIVE: return ds::tile_elems(kind_of(dtype), true, INT64_MAX / 16);
    case DS_TILE_OF_THREE_PASS: return ds::three_pass_tile_elems(b);
    case DS_TILE_OF_COMPACT: return ds::compact_tile_elems(b);
    case DS_TILE_OF_LDS_TILE_SCAN: return b == 4 ? ds::lds_tile_elems() : -1;
    case DS_TILE_OF_COUNTING_SORT: return b == 4 ? ds::sort_tile_elems(false) : -1;
    case DS_TILE_OF_COUNTING_SORT_VALUES: return b == 4 ? ds::sort_tile_elems(true) : -1;
    case DS_TILE_OF_MOE_ALIGN: return b == 4 ? ds::moe_tile_elems() : -1;
    default: return -1;
    }
}

int64_t ds_scan_tile_elems(int dtype, int inclusive, int64_t n)
{
    if (!valid_dtype(dtype) || (inclusive != 0 && inclusive != 1) || n < 0) return -1;
    return ds::tile_elems(kind_of(dtype), inclusive != 0, n);
}

int ds_version(void) { return 2; }

}  // extern "C"
