"""The CPU oracle against its pins, and the pins against planted mistakes.

CPU only. A planted mistake is made in a temporary copy of oracle.c, never in
the oracle itself; each must make at least one pin fail.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)


def test_golden_has_all_examples():
    names = [b["name"] for b in pins.parse_golden_examples()]
    assert names == ["definitions_8", "two_sweeps_4", "two_scans_4", "blelloch_figures_8"]
    for b in pins.parse_golden_examples():
        assert b["source"], b


def test_in_place(orc):
    x = np.array([3, 1, 7, 0, 4, 1, 6, 3], dtype=np.int32)
    orc.lib.oracle_scan_u32(x.ctypes.data, x.ctypes.data, x.size, 0)
    assert x.tolist() == [0, 3, 4, 11, 11, 15, 16, 22]
    y = np.array([3, 1, 4, 1], dtype=np.int64)
    orc.lib.oracle_scan_u64(y.ctypes.data, y.ctypes.data, y.size, 1)
    assert y.tolist() == [3, 4, 8, 9]


def test_empty(orc):
    for dt in (np.int32, np.int64, np.float32):
        r = orc.scan(np.zeros(0, dtype=dt), True)
        r = r[0] if dt == np.float32 else r
        assert r.size == 0


# (description, text in oracle.c, replacement). Each is a plausible slip.
MUTANTS = [
    ("exclusive adds before it writes",
     "            y[i] = acc;\n            acc += v;\n        }\n    }\n}\n\nvoid oracle_scan_u64",
     "            acc += v;\n            y[i] = acc;\n        }\n    }\n}\n\nvoid oracle_scan_u64"),
    ("u32 loop skips element 0", "uint32_t acc = 0;\n    for (int64_t i = 0;", "uint32_t acc = 0;\n    for (int64_t i = 1;"),
    ("u64 reads the neighbour", "        uint64_t v = x[i];", "        uint64_t v = x[i > 0 ? i - 1 : 0];"),
    ("u64 accumulates in 32 bits", "    uint64_t acc = 0;", "    uint32_t acc = 0;"),
    ("fp32 accumulates in fp32", "    double acc = 0.0;", "    float acc = 0.0f;"),
    ("|x| sum loses the sign flip", "acc_abs += v < 0.0 ? -v : v;", "acc_abs += v;"),
    ("inclusive fp32 drops the last term",
     "        if (inclusive) {\n            acc += v;\n            y[i] = acc;\n        } else {\n            y[i] = acc;\n            acc += v;\n        }\n        if (s_abs)",
     "        if (inclusive) {\n            y[i] = acc + (i + 1 < n ? v : 0.0);\n            acc += v;\n        } else {\n            y[i] = acc;\n            acc += v;\n        }\n        if (s_abs)"),
    ("'<=' read as '<'", "(op) == 1 ? (v) <= (c)", "(op) == 1 ? (v) < (c)"),
    ("'>' and '>=' swapped", "(op) == 2 ? (v) > (c) : (op) == 3 ? (v) >= (c)", "(op) == 2 ? (v) >= (c) : (op) == 3 ? (v) > (c)"),
    ("compaction keeps the wrong element", "            out[k++] = x[i];\n    return k;\n}\n\nint64_t oracle_compact_i32",
     "            out[k++] = x[i > 0 ? i - 1 : i];\n    return k;\n}\n\nint64_t oracle_compact_i32"),
    ("signed compare done unsigned", "int64_t oracle_compact_i32(const int32_t* x, int32_t* out, int64_t n, int op, int32_t c)",
     "int64_t oracle_compact_i32(const int32_t* x0, int32_t* out, int64_t n, int op, int32_t c0)\n"
     "#define x ((const uint32_t*)x0)\n#define c ((uint32_t)c0)"),
    ("counting sort ignores the shift", "const uint32_t mask = (1u << bits) - 1u;",
     "const uint32_t mask = (1u << bits) - 1u;\n    shift = 0;"),
    ("counting sort places equal digits last-first",
     "    for (int64_t i = 0; i < n; ++i) {\n        const uint32_t d = (keys[i] >> shift) & mask;",
     "    for (int64_t i = n - 1; i >= 0; --i) {\n        const uint32_t d = (keys[i] >> shift) & mask;"),
    ("values stay where they were", "vals_out[p] = vals[i];", "vals_out[p] = vals[p];"),
    ("digit mask one bit short", "const uint32_t mask = (1u << bits) - 1u;", "const uint32_t mask = (1u << (bits - 1)) - 1u;"),
    ("MoE offsets not rounded to the block", "run += (counts[e] + block - 1) / block * block;", "run += counts[e];"),
    ("MoE rounds a full block up once more", "run += (counts[e] + block - 1) / block * block;", "run += (counts[e] + block) / block * block;"),
    ("MoE padding marked 0", "sorted[p] = (int32_t)n;", "sorted[p] = 0;"),
    ("MoE expert 0 takes the invalid ids", "        if (ids[i] >= 0 && ids[i] < num_experts)\n            counts[ids[i]]++;",
     "        counts[ids[i] >= 0 && ids[i] < num_experts ? ids[i] : 0]++;"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, desc, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/absent: {desc}"
    mutated = src.replace(old, new)
    if "#define x" in new:  # keep the macro local to that one function
        mutated = mutated.replace("int64_t oracle_compact_f32", "#undef x\n#undef c\nint64_t oracle_compact_f32")
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(path), so)
    bad = oracle.Oracle(so)
    failed = []
    for check in pins.ALL:
        try:
            check(bad)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake: {desc}"
