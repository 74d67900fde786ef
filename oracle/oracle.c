/*
 * oracle.c -- plain sequential CPU reference for device-wide prefix sums and
 * order-preserving stream compaction.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the product path never
 * does, and this file shares no code, header, table or helper with the HIP
 * library.
 *
 * What it computes (the plain definitions, written out):
 *   inclusive  y_i = x_0 + x_1 + ... + x_i
 *   exclusive  y_0 = 0,  y_i = x_0 + ... + x_{i-1}
 * "Prefix sum and other parallel patterns" (ai-infra-handbooks), section
 * "Definitions", and "Day 31 -- CUDA prefix sum, the Hillis-Steele scan",
 * section "Two scans, and which one hands you the total".
 *
 * Integers accumulate in unsigned arithmetic, so a sum that leaves the range
 * wraps modulo 2^32 (int32/uint32) or 2^64 (int64/uint64); the result bits are
 * then read back in the caller's signed or unsigned type. fp32 inputs
 * accumulate in fp64 and the fp64 prefix is returned unrounded, together with
 * S_i = |x_0| + ... + |x_i| for the tolerance |gpu_i - y_i| <= 1e-5 * S_i.
 *
 * Compaction keeps, in input order, every x_i with (x_i OP operand), and
 * returns how many it kept ("Prefix sum and other parallel patterns",
 * section "Stream compaction" and its first exercise).
 *
 * A counting-sort pass (the step a radix sort repeats once per digit, which
 * the pages name as a user of the exclusive scan: "Day 32", closing section,
 * and "Prefix sum and other parallel patterns", opening paragraph) orders
 * 32-bit keys stably by one digit: count each digit, take the exclusive scan
 * of the counts as each digit's first output slot, then place the elements in
 * input order.
 *
 * MoE alignment ("Prefix sum and other parallel patterns", section "In LLMs:
 * MoE token dispatch" and exercise 2): the number of assignments per expert,
 * each expert's start as the exclusive scan of those counts rounded up to a
 * multiple of the block size, and the assignment indices grouped by expert.
 *
 * The scans accept y == x (in place): each x_i is read before y_i is
 * written. The counting-sort and MoE functions need distinct buffers.
 */
#include <stdint.h>

void oracle_scan_u32(const uint32_t* x, uint32_t* y, int64_t n, int inclusive)
{
    uint32_t acc = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint32_t v = x[i];
        if (inclusive) {
            acc += v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc += v;
        }
    }
}

void oracle_scan_u64(const uint64_t* x, uint64_t* y, int64_t n, int inclusive)
{
    uint64_t acc = 0;
    for (int64_t i = 0; i < n; ++i) {
        uint64_t v = x[i];
        if (inclusive) {
            acc += v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc += v;
        }
    }
}

/* y and s_abs are fp64 arrays of n elements; s_abs may be NULL. */
void oracle_scan_f32(const float* x, double* y, double* s_abs, int64_t n, int inclusive)
{
    double acc = 0.0;
    double acc_abs = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = (double)x[i];
        acc_abs += v < 0.0 ? -v : v;
        if (inclusive) {
            acc += v;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc += v;
        }
        if (s_abs)
            s_abs[i] = acc_abs;
    }
}

/* Comparison codes: 0 '<', 1 '<=', 2 '>', 3 '>=', 4 '==', 5 '!='. */
#define ORACLE_KEEP(v, op, c)                                   \
    ((op) == 0 ? (v) < (c) : (op) == 1 ? (v) <= (c)             \
   : (op) == 2 ? (v) > (c) : (op) == 3 ? (v) >= (c)             \
   : (op) == 4 ? (v) == (c) : (v) != (c))

int64_t oracle_compact_u32(const uint32_t* x, uint32_t* out, int64_t n, int op, uint32_t c)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ORACLE_KEEP(x[i], op, c))
            out[k++] = x[i];
    return k;
}

int64_t oracle_compact_i32(const int32_t* x, int32_t* out, int64_t n, int op, int32_t c)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ORACLE_KEEP(x[i], op, c))
            out[k++] = x[i];
    return k;
}

int64_t oracle_compact_f32(const float* x, float* out, int64_t n, int op, float c)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ORACLE_KEEP(x[i], op, c))
            out[k++] = x[i];
    return k;
}

int64_t oracle_compact_i64(const int64_t* x, int64_t* out, int64_t n, int op, int64_t c)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ORACLE_KEEP(x[i], op, c))
            out[k++] = x[i];
    return k;
}

int64_t oracle_compact_u64(const uint64_t* x, uint64_t* out, int64_t n, int op, uint64_t c)
{
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ORACLE_KEEP(x[i], op, c))
            out[k++] = x[i];
    return k;
}

/*
 * Stable counting-sort pass over the digit d(k) = (k >> shift) & (2^bits - 1),
 * 1 <= bits <= 8, 0 <= shift <= 31: keys_out holds the keys ordered by digit,
 * equal digits in input order; vals (may be NULL) follow their keys.
 */
void oracle_radix_pass_u32(const uint32_t* keys, const uint32_t* vals, uint32_t* keys_out, uint32_t* vals_out,
                           int64_t n, int shift, int bits)
{
    int64_t count[256] = {0};
    int64_t next[256];
    const uint32_t mask = (1u << bits) - 1u;
    for (int64_t i = 0; i < n; ++i)
        count[(keys[i] >> shift) & mask]++;
    int64_t run = 0;
    for (int d = 0; d < 256; ++d) {
        next[d] = run;
        run += count[d];
    }
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t d = (keys[i] >> shift) & mask;
        const int64_t p = next[d]++;
        keys_out[p] = keys[i];
        if (vals)
            vals_out[p] = vals[i];
    }
}

/*
 * ids: n expert indices (token-major, top_k per token); an id outside
 * [0, num_experts) belongs to no expert. counts[e] = assignments of expert e;
 * offsets[0] = 0 and offsets[e+1] = offsets[e] + counts[e] rounded up to a
 * multiple of block; sorted[offsets[e] ...] = the indices i with ids[i] == e
 * in increasing order, and the rest of expert e's block-rounded segment is n
 * (the padding mark). Writes sorted[0 .. offsets[E]) and returns offsets[E],
 * or -1 if that exceeds capacity. num_experts <= 1024.
 */
int64_t oracle_moe_align(const int32_t* ids, int64_t n, int num_experts, int block, int32_t* counts,
                         int32_t* offsets, int32_t* sorted, int64_t capacity)
{
    int64_t next[1024];
    for (int e = 0; e < num_experts; ++e)
        counts[e] = 0;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] >= 0 && ids[i] < num_experts)
            counts[ids[i]]++;
    int64_t run = 0;
    for (int e = 0; e < num_experts; ++e) {
        offsets[e] = (int32_t)run;
        next[e] = run;
        run += (counts[e] + block - 1) / block * block;
    }
    offsets[num_experts] = (int32_t)run;
    if (run > capacity)
        return -1;
    for (int64_t p = 0; p < run; ++p)
        sorted[p] = (int32_t)n;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] >= 0 && ids[i] < num_experts)
            sorted[next[ids[i]]++] = (int32_t)i;
    return run;
}
