"""Checks that tie the CPU oracle to what the pages and the mathematics fix.

Each check takes an oracle instance (oracle.Oracle) and raises AssertionError
on a mismatch. test_oracle.py runs them on the real oracle and on copies of
oracle.c with planted mistakes, which every mistake must fail.

Pins, none of which re-types the oracle's own loop:
  * worked examples printed on the pages (tests/golden/worked_examples.txt);
  * brute force: every y_i summed on its own, in Python integers or with
    math.fsum (exactly rounded), for all n <= 300;
  * closed forms for all-ones, the period-4 "every fourth element is 2"
    input and the (i % 8) + 1 input;
  * invariants: inclusive_i = exclusive_i + x_i, exclusive_0 = 0, the last
    inclusive value equals the total, monotone for non-negative input;
  * wraparound: closed form for constant 2^30 int32 input, brute force mod
    2^64 for raw 64-bit draws;
  * compaction: brute-force filtering, count = excl(flags)[n-1] + flags[n-1].
  * counting-sort pass: hand-worked case (tests/golden/counting_sort_examples.txt),
    numpy's stable argsort of the digits, brute-force output positions on
    tiny inputs, and four 8-bit passes from the low digit up = np.sort;
  * MoE alignment: hand-worked cases, np.bincount of the valid ids, the
    offsets' defining properties (multiples of the block, the smallest that
    hold each expert's count), np.nonzero per expert, the padding mark, and
    block = 1 reducing to numpy's stable argsort of the ids.
"""
from __future__ import annotations

import math
import os

import numpy as np

import datagen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_golden_examples(path=os.path.join(GOLDEN, "worked_examples.txt")):
    blocks, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = {"name": line.strip("[]")}
            blocks.append(cur)
            continue
        key, _, val = line.partition(":")
        cur[key.strip()] = val.strip() if key == "source" else [int(v) for v in val.split()]
    return blocks


def _mod(w):
    return 1 << w


def brute_int(x, inclusive, w):
    m = _mod(w)
    xs = [int(v) % m for v in x]
    return [sum(xs[: i + (1 if inclusive else 0)]) % m for i in range(len(xs))]


def brute_fsum(x, inclusive):
    xs = [float(v) for v in x]
    y = [math.fsum(xs[: i + (1 if inclusive else 0)]) for i in range(len(xs))]
    s = [math.fsum(abs(v) for v in xs[: i + 1]) for i in range(len(xs))]
    return y, s


BRUTE_NS = list(range(0, 34)) + [63, 64, 65, 127, 128, 129, 255, 256, 257, 300]


def check_worked_examples(orc):
    for ex in parse_golden_examples():
        for dt in (np.int32, np.uint32, np.int64, np.uint64, np.float32):
            x = np.array(ex["input"], dtype=dt)
            for kind in ("inclusive", "exclusive"):
                if kind not in ex:
                    continue
                got = orc.scan(x, kind == "inclusive")
                if dt == np.float32:
                    got = got[0]
                assert [int(v) for v in got] == ex[kind], (ex["name"], dt, kind, got)


def check_brute_int(orc):
    for n in BRUTE_NS:
        for dt, w, gen in ((np.int32, 32, lambda s, n: datagen.uniform_int(s, n, -(1 << 31), (1 << 31) - 1)),
                           (np.uint32, 32, lambda s, n: datagen.keys_u32(s, n)),
                           (np.int64, 64, lambda s, n: datagen.uniform_i64(s, n, 62)),
                           (np.uint64, 64, lambda s, n: datagen.raw_u64(s, n))):
            x = gen(100 + n, n).astype(dt)
            for inc in (True, False):
                got = orc.scan(x, inc)
                want = brute_int(x, inc, w)
                assert [int(v) % _mod(w) for v in got] == want, (n, dt, inc)


def check_brute_fp32(orc):
    for n in BRUTE_NS:
        # multiples of 2^-24 below 1: every fp64 prefix is exact, so fp64 == fsum bit for bit
        x = datagen.uniform01_f32(200 + n, n)
        for inc in (True, False):
            y, s = orc.scan(x, inc)
            by, bs = brute_fsum(x, inc)
            assert list(y) == by, (n, inc)
            assert list(s) == bs, (n, inc)
        # normals: fp64 sequential sum within n * 2^-53 * S_i of the exactly rounded sum
        x = datagen.normal_f32(300 + n, n)
        for inc in (True, False):
            y, s = orc.scan(x, inc)
            by, bs = brute_fsum(x, inc)
            for i in range(n):
                assert abs(y[i] - by[i]) <= (n + 1) * 2.0 ** -53 * bs[i], (n, inc, i)
                assert abs(s[i] - bs[i]) <= (n + 1) * 2.0 ** -53 * bs[i], (n, inc, i)


def check_closed_forms(orc):
    n = 1_000_003
    i = np.arange(n, dtype=np.int64)
    # all ones
    for dt in (np.int32, np.int64, np.float32):
        x = np.ones(n, dtype=dt)
        ex = orc.scan(x, False)
        inc = orc.scan(x, True)
        if dt == np.float32:
            ex, inc = ex[0], inc[0]
        assert np.array_equal(np.asarray(ex, dtype=np.int64), i)
        assert np.array_equal(np.asarray(inc, dtype=np.int64), i + 1)
    # 1.0 with 2.0 at i % 4 == 3: exclusive_i = i + floor(i / 4)
    y, _ = orc.scan(datagen.quarter_twos_f32(n), False)
    assert np.array_equal(y, (i + i // 4).astype(np.float64))
    # (i % 8) + 1: exclusive_i = 36 * floor(i / 8) + r (r + 1) / 2, r = i % 8
    r = i % 8
    want = 36 * (i // 8) + r * (r + 1) // 2
    for dt in (np.int32, np.float32):
        y = orc.scan(datagen.mod8_plus1(n, dt), False)
        y = y[0] if dt == np.float32 else y
        assert np.array_equal(np.asarray(y, dtype=np.int64), want)


def check_invariants(orc):
    n = 1_000_000
    for dt, w in ((np.int32, 32), (np.uint32, 32), (np.int64, 64)):
        if dt == np.int64:
            x = datagen.uniform_i64(7, n, 40)
        else:
            x = datagen.uniform_int(7, n, -1000, 1000).astype(dt)
        inc = orc.scan(x, True).astype(np.uint64)
        exc = orc.scan(x, False).astype(np.uint64)
        mask = np.uint64((1 << w) - 1) if w < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
        with np.errstate(over="ignore"):
            assert np.array_equal((exc + x.astype(np.uint64)) & mask, inc & mask)
        assert exc[0] == 0
        total = sum(int(v) for v in x[:1000]) + int(x[1000:].astype(np.int64).sum())
        assert int(inc[-1]) & int(mask) == total % (1 << w)
    x = datagen.uniform01_f32(8, n)
    inc, s = orc.scan(x, True)
    exc, s2 = orc.scan(x, False)
    assert exc[0] == 0.0 and np.all(np.diff(inc) >= 0) and np.all(np.diff(exc) >= 0)
    assert np.array_equal(exc + x.astype(np.float64), inc)  # exact: multiples of 2^-24 below 2^29
    assert np.array_equal(s, s2) and np.array_equal(s, inc)
    assert inc[-1] == math.fsum(float(v) for v in x)


def check_wraparound(orc):
    n = 1000
    x = np.full(n, 1 << 30, dtype=np.int32)
    i = np.arange(n, dtype=np.int64)
    want = ((i * (1 << 30)) % (1 << 32)).astype(np.uint32).view(np.int32)
    assert np.array_equal(orc.scan(x, False), want)
    assert np.array_equal(orc.scan(x, True), ((i + 1) * (1 << 30) % (1 << 32)).astype(np.uint32).view(np.int32))
    assert list(orc.scan(x, True)[:4]) == [1 << 30, -(1 << 31), -(1 << 30), 0]
    x = datagen.raw_u64(9, 300).view(np.int64)
    for inc in (True, False):
        got = orc.scan(x, inc).view(np.uint64)
        assert [int(v) for v in got] == brute_int(x.view(np.uint64), inc, 64)


COMPACT_CASES = [
    # dtype, generator, operands
    (np.uint32, lambda s, n: datagen.keys_u32(s, n), [0, 1, 1 << 31, 0xFFFFFFFF]),
    (np.int32, lambda s, n: datagen.uniform_int(s, n, -5, 5), [-5, 0, 3, 5]),
    (np.int64, lambda s, n: datagen.uniform_int(s, n, -5, 5, np.int64) * np.int64(1 << 40), [0, 3 << 40, -(1 << 62)]),
    (np.uint64, lambda s, n: datagen.raw_u64(s, n) >> np.uint64(61), [0, 3, 7]),
    (np.float32, lambda s, n: np.round(datagen.normal_f32(s, n) * 2) / 2, [0.0, -0.5, 1.0]),
]


def brute_compact(x, op, c):
    f = {"<": lambda v: v < c, "<=": lambda v: v <= c, ">": lambda v: v > c,
         ">=": lambda v: v >= c, "==": lambda v: v == c, "!=": lambda v: v != c}[op]
    return [v for v in x.tolist() if f(v)]


def check_compact(orc):
    for dt, gen, operands in COMPACT_CASES:
        for n in (0, 1, 7, 64, 257, 1000):
            x = gen(400 + n, n).astype(dt)
            for c in operands:
                c = dt(c).item()
                for op in ("<", "<=", ">", ">=", "==", "!="):
                    got = orc.compact(x, op, c)
                    assert got.tolist() == brute_compact(x, op, c), (dt, n, op, c)
    # NaN compares false except under !=
    x = np.array([1.0, np.nan, -2.0, np.nan, 0.0], dtype=np.float32)
    assert orc.compact(x, "<", 5.0).tolist() == [1.0, -2.0, 0.0]
    assert len(orc.compact(x, "!=", 0.0)) == 4
    assert orc.compact(x, "==", np.nan).size == 0
    # count = exclusive(flags)[n-1] + flags[n-1] (the pages' stream-compaction exercise)
    x = datagen.keys_u32(5, 100_003)
    flags = (x < np.uint32(1 << 31)).astype(np.uint32)
    pos = orc.scan(flags, False)
    k = orc.compact(x, "<", 1 << 31)
    assert k.size == int(pos[-1]) + int(flags[-1])
    assert np.array_equal(k, x[flags.astype(bool)])


def parse_counting_sort_examples(path=os.path.join(GOLDEN, "counting_sort_examples.txt")):
    blocks, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = {"name": line.strip("[]")}
            blocks.append(cur)
            continue
        key, _, val = line.partition(":")
        cur[key.strip()] = [int(v, 0) for v in val.split()]
    return blocks


RADIX_DIGITS = [(0, 8), (8, 8), (24, 8), (28, 4), (31, 1), (5, 3), (0, 1)]


def check_radix_pass(orc):
    for ex in parse_counting_sort_examples():
        if "keys" not in ex:
            continue
        keys = np.array(ex["keys"], dtype=np.uint32)
        ko, vo = orc.radix_pass(keys, ex["shift"][0], ex["bits"][0], np.arange(keys.size, dtype=np.uint32))
        assert ko.tolist() == ex["keys_out"] and vo.tolist() == ex["order"], (ex["name"], ko, vo)
    for n in (0, 1, 2, 7, 100, 1000, 4097):
        for gen in ("uniform", "few"):
            keys = datagen.keys_u32(800 + n, n) if gen == "uniform" else \
                (datagen.uniform_int(900 + n, n, 0, 3).astype(np.uint32) * np.uint32(0x01010101))
            vals = datagen.keys_u32(850 + n, n)
            for shift, bits in RADIX_DIGITS:
                d = (keys >> np.uint32(shift)) & np.uint32((1 << bits) - 1)
                perm = np.argsort(d, kind="stable")
                ko, vo = orc.radix_pass(keys, shift, bits, vals)
                assert np.array_equal(ko, keys[perm]) and np.array_equal(vo, vals[perm]), (n, gen, shift, bits)
                ko2, none = orc.radix_pass(keys, shift, bits)
                assert none is None and np.array_equal(ko2, ko)
    # brute force: element i lands after every smaller digit and every earlier equal digit
    for n in range(0, 41):
        keys = datagen.uniform_int(950 + n, n, 0, 5).astype(np.uint32) << np.uint32(3)
        ko, vo = orc.radix_pass(keys, 3, 2, np.arange(n, dtype=np.uint32))
        d = [(int(k) >> 3) & 3 for k in keys]
        for i in range(n):
            pos = sum(1 for j in range(n) if d[j] < d[i]) + sum(1 for j in range(i) if d[j] == d[i])
            assert ko[pos] == keys[i] and vo[pos] == i, (n, i)
    # least significant digit first: four stable 8-bit passes sort the keys
    keys = datagen.keys_u32(977, 5000)
    keys[::7] = keys[3]  # repeated keys: stability decides the order of their values
    k, v = keys, np.arange(keys.size, dtype=np.uint32)
    for shift in (0, 8, 16, 24):
        k, v = orc.radix_pass(k, shift, 8, v)
    assert np.array_equal(k, np.sort(keys)) and np.array_equal(v, np.argsort(keys, kind="stable"))


def check_moe_align(orc):
    for ex in parse_counting_sort_examples():
        if "ids" not in ex:
            continue
        c, o, srt = orc.moe_align(np.array(ex["ids"], dtype=np.int32), ex["experts"][0], ex["block"][0])
        assert c.tolist() == ex["counts"] and o.tolist() == ex["offsets"] and srt.tolist() == ex["sorted"], ex["name"]
    cases = [(1, 1, 1, 1), (3, 2, 4, 4), (100, 2, 8, 16), (1000, 8, 64, 64), (513, 4, 256, 64), (2000, 1, 5, 3),
             (257, 8, 511, 32)]
    for t, k, e, block in cases:
        for drop in (False, True):
            ids = datagen.moe_topk_ids(60 + t, t, k, e).ravel()
            if drop:  # ids that name no expert
                ids = ids.copy()
                ids[::5] = -1
                ids[1::7] = e
                ids[2::11] = 1 << 30
            n = ids.size
            counts, offsets, srt = orc.moe_align(ids, e, block)
            valid = (ids >= 0) & (ids < e)
            assert np.array_equal(counts, np.bincount(ids[valid], minlength=e)), (t, k, e)
            span = np.diff(offsets.astype(np.int64))
            assert offsets[0] == 0 and np.all(span % block == 0)
            assert np.all(span >= counts) and np.all(span < counts.astype(np.int64) + block)
            assert srt.size == offsets[-1]
            for x in range(e):
                seg = srt[offsets[x]:offsets[x + 1]]
                assert np.array_equal(seg[:counts[x]], np.nonzero(ids == x)[0]), (t, k, e, x)
                assert np.all(seg[counts[x]:] == n)
            if block == 1:
                assert np.array_equal(srt, np.nonzero(valid)[0][np.argsort(ids[valid], kind="stable")])


ALL = [check_worked_examples, check_brute_int, check_brute_fp32, check_closed_forms,
       check_invariants, check_wraparound, check_compact, check_radix_pass, check_moe_align]
