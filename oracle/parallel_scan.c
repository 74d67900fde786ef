/*
 * parallel_scan.c -- a plain two-pass blocked prefix sum on host threads.
 *
 * TEST AND BENCHMARK INFRASTRUCTURE ONLY, like the sequential oracle beside
 * it: the benchmark times it as a second CPU row next to the one-core oracle,
 * and a CPU test checks it against that oracle. It is not the oracle (nothing
 * is checked against it) and shares no code with the HIP library.
 *
 * The input splits into one contiguous block per thread. Pass 1: every thread
 * sums its block. Then the block sums are scanned on the calling thread, which
 * gives every block its starting offset. Pass 2: every thread scans its block
 * from that offset. This is the three-pass scheme of "Prefix sum and other
 * parallel patterns" (section "A device-level scan: scan then propagate") with
 * one block per core and the first pass reduced to a sum, so it reads the
 * input twice and writes it once.
 *
 * int32/uint32 sums wrap modulo 2^32 as in the oracle, so the result is
 * bit-identical to it. fp32 blocks accumulate in fp64 and store each prefix
 * rounded to fp32. Output may alias input (each x_i is read before y_i is
 * written, and pass 1 finishes before pass 2 starts).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define MAX_THREADS 256

typedef struct {
    const void* x;
    void* y;
    int64_t lo, hi;
    int inclusive;
    uint32_t usum, useed;
    double fsum, fseed;
} block_t;

static void* reduce_u32(void* p)
{
    block_t* b = (block_t*)p;
    const uint32_t* x = (const uint32_t*)b->x;
    uint32_t s = 0;
    for (int64_t i = b->lo; i < b->hi; ++i) s += x[i];
    b->usum = s;
    return NULL;
}

static void* scan_u32(void* p)
{
    block_t* b = (block_t*)p;
    const uint32_t* x = (const uint32_t*)b->x;
    uint32_t* y = (uint32_t*)b->y;
    uint32_t acc = b->useed;
    if (b->inclusive) {
        for (int64_t i = b->lo; i < b->hi; ++i) { acc += x[i]; y[i] = acc; }
    } else {
        for (int64_t i = b->lo; i < b->hi; ++i) { uint32_t v = x[i]; y[i] = acc; acc += v; }
    }
    return NULL;
}

static void* reduce_f32(void* p)
{
    block_t* b = (block_t*)p;
    const float* x = (const float*)b->x;
    double s = 0.0;
    for (int64_t i = b->lo; i < b->hi; ++i) s += (double)x[i];
    b->fsum = s;
    return NULL;
}

static void* scan_f32(void* p)
{
    block_t* b = (block_t*)p;
    const float* x = (const float*)b->x;
    float* y = (float*)b->y;
    double acc = b->fseed;
    if (b->inclusive) {
        for (int64_t i = b->lo; i < b->hi; ++i) { acc += (double)x[i]; y[i] = (float)acc; }
    } else {
        for (int64_t i = b->lo; i < b->hi; ++i) { float v = x[i]; y[i] = (float)acc; acc += (double)v; }
    }
    return NULL;
}

/* Runs fn on every block, blocks 1.. on their own threads and block 0 here.
 * Returns 0, or -1 if a thread could not be started (nothing is then left
 * running: the started ones are joined first). */
static int run_blocks(void* (*fn)(void*), block_t* blk, int t)
{
    pthread_t th[MAX_THREADS];
    int started = 1, rc = 0;
    for (; started < t; ++started)
        if (pthread_create(&th[started], NULL, fn, &blk[started]) != 0) { rc = -1; break; }
    if (rc == 0) fn(&blk[0]);
    for (int k = 1; k < started; ++k) pthread_join(th[k], NULL);
    return rc;
}

static int split(block_t* blk, const void* x, void* y, int64_t n, int inclusive, int threads)
{
    int t = threads < 1 ? 1 : (threads > MAX_THREADS ? MAX_THREADS : threads);
    if ((int64_t)t > n) t = n > 0 ? (int)n : 1;
    for (int k = 0; k < t; ++k) {
        blk[k].x = x;
        blk[k].y = y;
        blk[k].lo = n * k / t;
        blk[k].hi = n * (k + 1) / t;
        blk[k].inclusive = inclusive;
    }
    return t;
}

/* Returns 0 on success, -1 if threads could not be started (y is then
 * unspecified). */
int par_scan_u32(const uint32_t* x, uint32_t* y, int64_t n, int inclusive, int threads)
{
    block_t blk[MAX_THREADS];
    if (n <= 0) return 0;
    const int t = split(blk, x, y, n, inclusive, threads);
    if (run_blocks(reduce_u32, blk, t) != 0) return -1;
    uint32_t off = 0;
    for (int k = 0; k < t; ++k) { blk[k].useed = off; off += blk[k].usum; }
    return run_blocks(scan_u32, blk, t);
}

int par_scan_f32(const float* x, float* y, int64_t n, int inclusive, int threads)
{
    block_t blk[MAX_THREADS];
    if (n <= 0) return 0;
    const int t = split(blk, x, y, n, inclusive, threads);
    if (run_blocks(reduce_f32, blk, t) != 0) return -1;
    double off = 0.0;
    for (int k = 0; k < t; ++k) { blk[k].fseed = off; off += blk[k].fsum; }
    return run_blocks(scan_f32, blk, t);
}
