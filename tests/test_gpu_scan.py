"""Parity of the HIP scans (through the C ABI) with the CPU oracle.

Integers: bit-exact, wrapping modulo 2^32 / 2^64. fp32: |gpu_i - y_i| <=
1e-5 * S_i with y the fp64 oracle and S_i = sum_{j<=i} |x_j|; bit-exact on the
inputs whose every prefix is exact in fp32.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import pins
from gpu_util import (assert_fp32_close, assert_int_equal, cached_workload, check_scan, gpu_compact, gpu_scan, say,
                      scan_tile, stream_handle, tile_of, to_dev)

pytestmark = pytest.mark.gpu

ALGOS = ["lookback", "three_pass"]
DTYPES = [np.int32, np.uint32, np.float32, np.int64, np.uint64]


def _input(dt, n, seed):
    dt = np.dtype(dt)
    if dt == np.float32:
        return datagen.normal_f32(seed, n)
    if dt == np.int32:
        return datagen.uniform_int(seed, n, -1000, 1000)
    if dt == np.uint32:
        return datagen.keys_u32(seed, n)
    if dt == np.int64:
        return datagen.uniform_i64(seed, n, 40)
    return datagen.raw_u64(seed, n)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_worked_examples(dt, algo):
    for ex in pins.parse_golden_examples():
        x = np.array(ex["input"], dtype=dt)
        for kind in ("inclusive", "exclusive"):
            if kind in ex:
                got = gpu_scan(x, kind == "inclusive", algo)
                assert [int(v) for v in got] == ex[kind], (ex["name"], kind, got)


def test_one_tile_int32_exclusive():
    x = cached_workload("one_tile")
    assert x.size <= scan_tile(np.int32, False, x.size)  # one workgroup, no look-back
    say("one_tile int32 exclusive n=4096 (single workgroup)")
    check_scan(x, False, gpu_scan(x, False), "one_tile")
    check_scan(x, False, gpu_scan(x, False, entry="scan_exclusive"), "one_tile via scan_exclusive")


@pytest.mark.parametrize("algo", ALGOS)
def test_mid_int32_both(algo):
    x = cached_workload("mid")
    for inc in (False, True):
        say(f"mid int32 n=1048576 inclusive={inc} {algo}")
        check_scan(x, inc, gpu_scan(x, inc, algo), f"mid {algo} inc={inc}")


@pytest.mark.parametrize("algo", ALGOS)
def test_fp32_10m_inclusive(algo):
    x = cached_workload("fp32_10m")
    say(f"fp32_10m inclusive {algo}")
    r = check_scan(x, True, gpu_scan(x, True, algo), f"fp32_10m {algo}")
    say(f"  max |err|/S = {r:.3e}")


def test_fp32_exact_patterns_bit_exact():
    n = 10_000_000
    x = datagen.quarter_twos_f32(n)
    i = np.arange(n, dtype=np.int64)
    for algo in ALGOS:
        say(f"quarter_twos fp32 exclusive n={n} {algo}")
        got = gpu_scan(x, False, algo)
        assert_int_equal(got.astype(np.int64), i + i // 4, "every fourth 2.0, exclusive")
        got = gpu_scan(x, True, algo)
        assert_int_equal(got.astype(np.int64), (i + 1) + (i + 1) // 4, "every fourth 2.0, inclusive")
    n = 3_700_000  # totals stay below 2^24
    x = datagen.mod8_plus1(n)
    i = np.arange(n, dtype=np.int64)
    r = i % 8
    want = 36 * (i // 8) + r * (r + 1) // 2
    got = gpu_scan(x, False)
    assert np.all(got == want.astype(np.float32)), "(i % 8) + 1 exclusive not bit-exact"


@pytest.mark.parametrize("algo", ALGOS)
def test_int32_100m_exclusive(algo):
    x = cached_workload("int32_100m")
    say(f"int32_100m exclusive {algo}")
    check_scan(x, False, gpu_scan(x, False, algo), f"int32_100m {algo}")


@pytest.mark.parametrize("n", [1_048_576, 100_000_007])
def test_int64_large(n):
    # 64-bit values in [-2^40, 2^40]: two status words per tile carry the halves
    x = datagen.uniform_i64(64, n, 40)
    for inc in (False, True):
        say(f"int64 n={n} inclusive={inc}")
        assert_int_equal(gpu_scan(x, inc), oracle.scan(x, inc), f"int64 n={n} inc={inc}")


def test_fp32_100m_exclusive():
    x = cached_workload("fp32_100m")
    for algo in ALGOS:
        say(f"fp32_100m exclusive {algo}")
        r = check_scan(x, False, gpu_scan(x, False, algo), f"fp32_100m {algo}")
        say(f"  max |err|/S = {r:.3e}")


def _edge_sizes(T):
    return sorted({1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, T - 1, T, T + 1, 2 * T - 1,
                   2 * T + 1, 3 * T + 7, 64 * T, 64 * T + 5, 65 * T + 1, 130 * T + 3})


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_edge_sizes(dt, algo):
    T = tile_of(dt)
    for n in _edge_sizes(T):
        x = _input(dt, n, 1000 + n)
        for inc in (False, True):
            check_scan(x, inc, gpu_scan(x, inc, algo), f"{np.dtype(dt).name} n={n} inc={inc} {algo}")


def _regime_sizes(dt, inc):
    """Sizes at the tile boundaries of each look-back tile regime (8 vectors per thread up to
    8 MiB of data, 12 up to 32 MiB, 16 up to 64 MiB, the large tile beyond) and at the regime
    boundaries."""
    esz = np.dtype(dt).itemsize
    small_max, mid_max, upper_max = (8 << 20) // esz, (32 << 20) // esz, (64 << 20) // esz
    ts, tm = scan_tile(dt, inc, 1), scan_tile(dt, inc, small_max + 1)
    tu, tl = scan_tile(dt, inc, mid_max + 1), scan_tile(dt, inc, upper_max + 1)
    assert ts < tm < tu <= tl, (ts, tm, tu, tl)
    km, ku, kl = small_max // tm + 2, mid_max // tu + 1, upper_max // tl + 1
    return [ts - 1, ts, ts + 1, 7 * ts + 3, small_max, small_max + 1, km * tm - 1, km * tm, km * tm + 1,
            mid_max, mid_max + 1, ku * tu - 1, ku * tu, ku * tu + 1,
            upper_max, upper_max + 1, kl * tl - 1, kl * tl, kl * tl + 1]


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.int64], ids=lambda d: np.dtype(d).name)
def test_tile_regimes(dt):
    for inc in (False, True):
        for n in _regime_sizes(dt, inc):
            x = _input(dt, n, 3000 + n % 997)
            check_scan(x, inc, gpu_scan(x, inc), f"{np.dtype(dt).name} n={n} inc={inc} tile {scan_tile(dt, inc, n)}")


def test_wraparound():
    n = 100_003
    x = np.full(n, 1 << 30, dtype=np.int32)
    for algo in ALGOS:
        for inc in (False, True):
            assert_int_equal(gpu_scan(x, inc, algo), oracle.scan(x, inc), f"2^30 wrap {algo} inc={inc}")
    x = datagen.raw_u64(77, 300_007).view(np.int64)
    for algo in ALGOS:
        for inc in (False, True):
            assert_int_equal(gpu_scan(x, inc, algo), oracle.scan(x, inc), f"int64 wrap {algo} inc={inc}")
    x = datagen.keys_u32(78, 200_001)
    assert_int_equal(gpu_scan(x, True), oracle.scan(x, True), "uint32 wrap")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_in_place(dt):
    n = 3 * tile_of(dt) + 11
    x = _input(dt, n, 55)
    for algo in ALGOS:
        for inc in (False, True):
            check_scan(x, inc, gpu_scan(x, inc, algo, in_place=True), f"in place {algo} inc={inc}")


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_misaligned(dt):
    T = tile_of(dt)
    for n in (5, T + 3, 5 * T + 1):
        x = _input(dt, n, 66 + n)
        for off in (1, 3):
            for algo in ALGOS:
                check_scan(x, False, gpu_scan(x, False, algo, offset=off), f"offset {off} n={n} {algo}")
                check_scan(x, True, gpu_scan(x, True, algo, offset=off), f"offset {off} n={n} {algo}")


def _scan_at(x, inclusive, algo, in_off, out_off, guard=37):
    """Scan with the input `in_off` and the output `out_off` elements past a
    16-byte boundary; the output buffer's elements around the result keep
    their sentinel."""
    import primitives_device_scan_amd as ds
    from gpu_util import CODE, STORAGE, from_dev, sentinel_fill, stream_handle, to_dev
    n, esz = x.size, x.dtype.itemsize
    xin = to_dev(x, extra=in_off + guard, offset=in_off)
    out = torch.empty(n + out_off + guard, dtype=STORAGE[x.dtype][1], device="cuda")
    sentinel_fill(out)
    st = ds.lib.ds_scan(CODE[x.dtype], int(inclusive), ds.ALGO[algo], xin.data_ptr() + in_off * esz,
                        out.data_ptr() + out_off * esz, n, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    raw = out.view(torch.uint8).cpu().numpy()
    assert np.all(raw[:out_off * esz] == 0xA5), "written below the output"
    assert np.all(raw[(out_off + n) * esz:] == 0xA5), "written past the output"
    return from_dev(out, x.dtype, out_off, n)


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_misaligned_phases(dt):
    # input and output at different offsets from 16-byte alignment (one of them
    # aligned, or both off by different amounts): whole waves use 16-byte
    # vectors at 4- or 8-byte alignment; several tiles and a ragged end
    T = tile_of(dt)
    per_vec = 16 // np.dtype(dt).itemsize
    n = 7 * T + 5
    x = _input(dt, n, 123)
    phases = [(a, b) for a in range(per_vec) for b in range(per_vec) if a != b]
    for in_off, out_off in phases:
        for algo in ALGOS:
            for inc in (False, True):
                check_scan(x, inc, _scan_at(x, inc, algo, in_off, out_off), f"in +{in_off} out +{out_off} {algo} inc={inc}")


@pytest.mark.parametrize("dt", [np.int32, np.float32, np.int64], ids=lambda d: np.dtype(d).name)
def test_misaligned_largest_tiles(dt):
    # past 64 MiB the look-back takes its largest tile; one element off alignment on both sides,
    # then the input alone off alignment
    n = (80 << 20) // np.dtype(dt).itemsize + 3
    x = _input(dt, n, 321)
    say(f"misaligned largest tile {np.dtype(dt).name} n={n}")
    for inc in (False, True):
        check_scan(x, inc, _scan_at(x, inc, "lookback", 1, 1), f"both +1 inc={inc}")
    check_scan(x, False, _scan_at(x, False, "lookback", 1, 0), "input +1, output aligned")


def test_misaligned_in_place():
    n = 9 * tile_of(np.int32) + 11
    x = datagen.uniform_int(5, n, -1000, 1000)
    for off in (1, 2, 3):
        for inc in (False, True):
            check_scan(x, inc, gpu_scan(x, inc, in_place=True, offset=off), f"in place +{off} inc={inc}")


def test_int_repeat_determinism():
    x = datagen.uniform_int(99, 5_000_011, -1000, 1000)
    first = gpu_scan(x, False)
    for _ in range(10):
        assert np.array_equal(gpu_scan(x, False), first)
    assert_int_equal(first, oracle.scan(x, False), "repeat")


def test_workspace_growth_and_reuse():
    # small -> large -> small on one stream: the workspace grows once and stays valid
    for n in (10_000, 3_000_000, 50_000, 7_000_000, 4097):
        x = datagen.uniform_int(n, n, 0, 100)
        check_scan(x, False, gpu_scan(x, False), f"growth n={n}")


def test_two_streams():
    import primitives_device_scan_amd as ds
    n = 2_000_003
    xs = [datagen.uniform_int(s, n, -50, 50) for s in (1, 2)]
    ins = [torch.from_numpy(x).cuda() for x in xs]
    outs = [torch.empty_like(t) for t in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(5):
        for t, o, s in zip(ins, outs, streams):
            with torch.cuda.stream(s):
                ds.scan_exclusive(t, o)
        torch.cuda.synchronize()
        for x, o in zip(xs, outs):
            assert_int_equal(o.cpu().numpy(), oracle.scan(x, False), f"two streams rep {rep}")


def test_binding_entry_points():
    import primitives_device_scan_amd as ds
    x = torch.tensor([3, 1, 7, 0, 4, 1, 6, 3], dtype=torch.int32, device="cuda")
    assert ds.scan_inclusive(x).tolist() == [3, 4, 11, 11, 15, 16, 22, 25]
    assert ds.scan_exclusive(x).tolist() == [0, 3, 4, 11, 11, 15, 16, 22]
    assert ds.scan(x, False, algo="three_pass").tolist() == [0, 3, 4, 11, 11, 15, 16, 22]
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    assert ds.scan_exclusive(e).numel() == 0
    buf = torch.zeros(100, dtype=torch.int32, device="cuda")
    with pytest.raises(ds.DevscanError):  # partial overlap is refused before any launch
        ds.scan_exclusive(buf[1:], buf[:99])
    with pytest.raises(TypeError):
        ds.scan_exclusive(torch.zeros(8, dtype=torch.float16, device="cuda"))


def test_give_up_path_then_recovery():
    """A tiny spin limit makes look-back waits give up (outputs invalid, flag
    set) while every kernel still finishes; compact_if then writes -1 as its
    count; after ds_query_timeout (which clears the status words) later calls
    are correct again."""
    import torch

    import primitives_device_scan_amd as ds
    n = 300 * tile_of(np.int32) + 9
    x = datagen.uniform_int(5, n, 0, 9)
    xin = to_dev(x)
    out = torch.empty_like(xin)
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    h = stream_handle()
    assert ds.query_timeout() is False
    ds.set_spin_limit(1)
    try:
        for _ in range(3):
            assert ds.lib.ds_scan(0, 0, 0, xin.data_ptr(), out.data_ptr(), n, h) == 0
        gave_up = ds.query_timeout()
        say(f"spin limit 1, scans: gave up = {gave_up}")
        assert ds.lib.compact_if(0, xin.data_ptr(), out.data_ptr(), cnt.data_ptr(), n, ds.CMP[">"], 4, h) == 0
        gave_up_c = ds.query_timeout()
        k = int(cnt.item())
        say(f"spin limit 1, compact_if: gave up = {gave_up_c}, count = {k}")
        want_k = int(np.count_nonzero(x > 4))
        assert k == -1 if gave_up_c else k == want_k
    finally:
        ds.set_spin_limit(0)
    for _ in range(3):
        check_scan(x, False, gpu_scan(x, False), "after give-up")
    got, k = gpu_compact(x, ">", 4)
    want = oracle.compact(x, ">", 4)
    assert k == want.size and np.array_equal(got[:k], want)
    assert ds.query_timeout() is False


@pytest.mark.parametrize("dt", DTYPES, ids=lambda d: np.dtype(d).name)
def test_three_pass_on_one_tile_runs_the_lookback_kernel(dt):
    """Sizes around both tile sizes: a three-pass call whose input fits one
    three-pass tile runs the look-back kernel, whose tiles can be smaller
    (a regression test for a workspace that was sized by the wrong tile)."""
    sizes = set()
    tiles = [tile_of(dt, entry=entry) for entry in ("scan_exclusive", "scan_inclusive", "three_pass")]
    tiles += [scan_tile(dt, inc, 1) for inc in (False, True)]  # the look-back tile of small inputs
    for t in tiles:
        sizes |= {t - 1, t, t + 1, 2 * t - 1, 2 * t + 1}
    for n in sorted(sizes):
        x = _input(dt, n, 5000 + n)
        for inc in (False, True):
            check_scan(x, inc, gpu_scan(x, inc, "three_pass"), f"three_pass n={n} inc={inc}")
            check_scan(x, inc, gpu_scan(x, inc, "lookback"), f"lookback n={n} inc={inc}")
