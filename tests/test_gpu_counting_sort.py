"""Parity of the counting-sort pass (ds_radix_pass) and MoE alignment
(ds_moe_align), called through the C ABI, with the oracle: bit-exact keys,
values, counts, offsets and grouped indices (the pass is stable, so the
result is unique), and buffers past what the call defines left untouched."""
import numpy as np
import pytest
import torch

import datagen
import oracle
import primitives_device_scan_amd as ds
from gpu_util import assert_int_equal, cached_workload, from_dev, say, sentinel_fill, stream_handle, to_dev

pytestmark = pytest.mark.gpu

_TILES = {}


def sort_tile(entry: str = "counting_sort") -> int:
    """Keys per workgroup tile of the radix pass ("counting_sort", or with values
    "counting_sort_values") or of multi-launch MoE alignment ("moe_align")."""
    if entry not in _TILES:
        _TILES[entry] = int(ds.lib.ds_tile_elems(1, ds._binding.TILE_OF[entry]))
    return _TILES[entry]


def gpu_radix_pass(keys: np.ndarray, shift: int, bits: int, vals: np.ndarray | None = None, offset: int = 0):
    n = keys.size
    kin = to_dev(keys, extra=offset, offset=offset)[offset:]
    kout = torch.empty(max(n, 1) + 64, dtype=torch.int32, device="cuda")
    sentinel_fill(kout)
    vin = vout = None
    if vals is not None:
        vin = to_dev(vals)
        vout = torch.empty(max(n, 1) + 64, dtype=torch.int32, device="cuda")
        sentinel_fill(vout)
    st = ds.lib.ds_radix_pass(kin.data_ptr(), kout.data_ptr(), None if vin is None else vin.data_ptr(),
                              None if vout is None else vout.data_ptr(), n, shift, bits, stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    ko = from_dev(kout, np.uint32)
    assert np.all(ko[n:] == 0xA5A5A5A5), "written past n"
    vo = None
    if vout is not None:
        vo = from_dev(vout, np.uint32)
        assert np.all(vo[n:] == 0xA5A5A5A5)
        vo = vo[:n]
    return ko[:n], vo


def check_radix(keys, shift, bits, vals, what):
    ko, vo = gpu_radix_pass(keys, shift, bits, vals)
    wk, wv = oracle.radix_pass(keys, shift, bits, vals)
    assert_int_equal(ko, wk, what + " keys")
    if vals is not None:
        assert_int_equal(vo, wv, what + " values")


DIGITS = [(0, 8), (8, 8), (24, 8), (28, 4), (31, 1), (5, 3)]


def around_tiles(T: int):
    # also around groups of 2 and 4 tiles (a workgroup may take several tiles in turn)
    return (1, 7, 64, 4095, 4096, 4097, T - 1, T, T + 1, 2 * T, 3 * T + 5, 4 * T - 1, 4 * T, 4 * T + 1, 8 * T + 5,
            9 * T, 70 * T + 3)


@pytest.mark.parametrize("shift,bits", DIGITS)
def test_radix_pass_sizes(shift, bits):
    # sizes around the tile of each form: keys only, and keys with values
    for n in around_tiles(sort_tile("counting_sort")):
        keys = datagen.keys_u32(1000 + n, n)
        check_radix(keys, shift, bits, None, f"n={n} shift={shift} bits={bits} keys only")
    for n in around_tiles(sort_tile("counting_sort_values")):
        keys = datagen.keys_u32(1000 + n, n)
        vals = datagen.keys_u32(2000 + n, n)
        check_radix(keys, shift, bits, vals, f"n={n} shift={shift} bits={bits}")


def test_tiles_are_whole_waves():
    # every lane of a tile's four waves holds the same number of keys
    for entry in ("counting_sort", "counting_sort_values", "moe_align"):
        T = sort_tile(entry)
        assert T > 0 and T % 256 == 0, (entry, T)


def test_radix_pass_values_alias_keys():
    # the two inputs may be one buffer (both are only read): each key carries itself as its value
    T = sort_tile("counting_sort_values")
    n = 7 * T + 13
    keys = datagen.keys_u32(91, n)
    kin = to_dev(keys)
    kout = torch.empty(n + 64, dtype=torch.int32, device="cuda")
    vout = torch.empty(n + 64, dtype=torch.int32, device="cuda")
    sentinel_fill(kout)
    sentinel_fill(vout)
    st = ds.lib.ds_radix_pass(kin.data_ptr(), kout.data_ptr(), kin.data_ptr(), vout.data_ptr(), n, 4, 8,
                              stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    wk, wv = oracle.radix_pass(keys, 4, 8, keys)
    ko, vo = from_dev(kout, np.uint32), from_dev(vout, np.uint32)
    assert_int_equal(ko[:n], wk, "aliased inputs: keys")
    assert_int_equal(vo[:n], wv, "aliased inputs: values")
    assert np.all(ko[n:] == 0xA5A5A5A5) and np.all(vo[n:] == 0xA5A5A5A5), "written past n"
    assert np.array_equal(from_dev(kin, np.uint32), keys), "input changed"


def test_radix_pass_misaligned_keys():
    # keys one element off 16-byte alignment: the count kernel's element-wise path
    T = sort_tile()
    for n in (T + 5, 9 * T + 77):
        keys = datagen.keys_u32(33 + n, n)
        ko, _ = gpu_radix_pass(keys, 0, 8, None, offset=1)
        wk, _ = oracle.radix_pass(keys, 0, 8)
        assert_int_equal(ko, wk, f"n={n} misaligned keys")


def test_radix_pass_skewed_digits():
    T = sort_tile()
    n = 5 * T + 77
    few = (datagen.uniform_int(31, n, 0, 3).astype(np.uint32) * np.uint32(0x01010101))
    same = np.full(n, 0xDEADBEEF, dtype=np.uint32)
    one_hot = np.where(datagen.uniform_int(32, n, 0, 999) == 0, np.uint32(7), np.uint32(200))
    for name, keys in (("four digits", few), ("all equal", same), ("one digit in 1000", one_hot)):
        check_radix(keys, 0, 8, np.arange(n, dtype=np.uint32), name)


@pytest.mark.parametrize("n", [33_546_239, 33_554_433, 40_000_003])
def test_radix_pass_large_ragged(n):
    # thousands of tiles, the last one ragged; keys only and with values
    keys = datagen.keys_u32(n % 1000, n)
    check_radix(keys, 8, 8, None, f"n={n}")
    check_radix(keys, 16, 8, np.arange(n, dtype=np.uint32), f"n={n} with values")


def test_radix_pass_256m_keys():
    keys = cached_workload("compact_256m")
    say("radix pass: 268,435,456 uint32 keys, low 8-bit digit, with values")
    vals = datagen.keys_u32(8, keys.size)
    ko, vo = gpu_radix_pass(keys, 0, 8, vals)
    wk, wv = oracle.radix_pass(keys, 0, 8, vals)
    assert_int_equal(ko, wk, "256m keys")
    assert_int_equal(vo, wv, "256m values")


def test_four_passes_sort():
    # least significant digit first: four stable 8-bit passes sort 32-bit keys
    n = 1_000_003
    keys = datagen.keys_u32(44, n)
    keys[::5] = keys[1]
    k, v = keys, np.arange(n, dtype=np.uint32)
    for shift in (0, 8, 16, 24):
        k, v = gpu_radix_pass(k, shift, 8, v)
    assert_int_equal(k, np.sort(keys), "four passes: keys")
    assert_int_equal(v, np.argsort(keys, kind="stable").astype(np.uint32), "four passes: values")


def gpu_moe_align(ids: np.ndarray, experts: int, block: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32).ravel()
    n = ids.size
    cap = n + experts * (block - 1)
    d_ids = to_dev(ids) if n else torch.zeros(1, dtype=torch.int32, device="cuda")
    counts = torch.empty(experts, dtype=torch.int32, device="cuda")
    offsets = torch.empty(experts + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
    for t in (counts, offsets, srt):
        sentinel_fill(t)
    st = ds.lib.ds_moe_align(d_ids.data_ptr(), n, experts, block, counts.data_ptr(), offsets.data_ptr(),
                             srt.data_ptr(), max(cap, 1), stream_handle())
    assert st == 0, ds.lib.ds_status_string(st)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), offsets.cpu().numpy(), srt.cpu().numpy()


def check_moe(ids, experts, block, what):
    c, o, s = gpu_moe_align(ids, experts, block)
    wc, wo, ws = oracle.moe_align(ids, experts, block)
    assert_int_equal(c, wc, what + " counts")
    assert_int_equal(o, wo, what + " offsets")
    total = int(wo[-1])
    assert_int_equal(s[:total], ws, what + " sorted ids")
    assert np.all(s[total:].view(np.uint32) == 0xA5A5A5A5), what + ": written past offsets[E]"


@pytest.mark.parametrize("name", sorted(datagen.MOE_WORKLOADS))
def test_moe_workloads(name):
    t, k, e, block, _, _ = datagen.MOE_WORKLOADS[name]
    say("moe", name, t, "tokens x top", k, "of", e, "experts, block", block)
    check_moe(datagen.moe_workload(name), e, block, name)


@pytest.mark.parametrize("experts,top_k,block", [(1, 1, 1), (8, 2, 16), (64, 6, 64), (256, 8, 128), (511, 8, 32),
                                                  (100, 3, 7)])
def test_moe_shapes(experts, top_k, block):
    T = sort_tile("moe_align")
    # one-launch sizes (up to 8,192 ids), then past the one-launch size by about one and three tiles
    for tokens in (1, 5, 1000, (8192 + T) // top_k + 1, (8192 + 3 * T) // top_k + 11):
        ids = datagen.moe_topk_ids(70 + tokens, tokens, top_k, experts)
        check_moe(ids, experts, block, f"E={experts} k={top_k} block={block} tokens={tokens}")


@pytest.mark.parametrize("n", [4095, 4096, 4097, 8191, 8192, 8193, 12289])
def test_moe_one_launch_boundary(n):
    # up to 8,192 ids one single-workgroup launch aligns everything; above, three launches
    ids = datagen.moe_topk_ids(n, n, 1, 100).ravel().copy()
    ids[::13] = -3
    check_moe(ids, 100, 16, f"n={n}")


def test_moe_large():
    # about a million ids (512 tiles and beyond), an eighth of them dropped
    T = sort_tile("moe_align")
    for n in (512 * T - 5, 512 * T, 512 * T + 1, 600 * T + 3):
        ids = (datagen.keys_u32(n, n) % 257).astype(np.int32)  # 256: dropped
        say("moe", n, "ids")
        check_moe(ids, 256, 64, f"n={n}")


def test_moe_dropped_ids_and_empty():
    ids = datagen.moe_topk_ids(5, 4099, 8, 64).ravel().copy()
    ids[::5] = -1
    ids[1::7] = 64
    ids[2::11] = 1 << 30
    check_moe(ids, 64, 16, "dropped ids")
    check_moe(np.full(3000, -1, dtype=np.int32), 16, 8, "all dropped")
    c, o, _ = gpu_moe_align(np.zeros(0, dtype=np.int32), 16, 8)
    assert np.all(c == 0) and np.all(o == 0)


def test_radix_pass_two_streams():
    # each (device, stream) has its own table and look-back workspace: two passes in flight at once
    T = sort_tile()
    n = 300 * T + 11
    ka, kb = datagen.keys_u32(71, n), datagen.keys_u32(72, n)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for keys, st in ((ka, s1), (kb, s2)):
        kin = to_dev(keys)
        kout = torch.empty_like(kin)
        outs.append((keys, kin, kout, st))
    torch.cuda.synchronize()
    for _ in range(3):
        for keys, kin, kout, st in outs:
            assert ds.lib.ds_radix_pass(kin.data_ptr(), kout.data_ptr(), None, None, n, 16, 8, st.cuda_stream) == 0
    torch.cuda.synchronize()
    for keys, kin, kout, st in outs:
        wk, _ = oracle.radix_pass(keys, 16, 8)
        assert_int_equal(from_dev(kout, np.uint32), wk, "two streams")


def test_bindings():
    x = torch.from_numpy(datagen.keys_u32(9, 100_000).view(np.int32)).cuda()
    ko, vo = ds.radix_pass(x, 8, 8, vals=torch.arange(x.numel(), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    wk, wv = oracle.radix_pass(x.cpu().numpy().view(np.uint32), 8, 8, np.arange(x.numel(), dtype=np.uint32))
    assert_int_equal(ko.cpu().numpy().view(np.uint32), wk, "binding keys")
    assert_int_equal(vo.cpu().numpy().view(np.uint32), wv, "binding values")
    ids = torch.from_numpy(datagen.moe_topk_ids(3, 500, 4, 32)).cuda()
    c, o, s = ds.moe_align(ids, 32, 16)
    torch.cuda.synchronize()
    wc, wo, ws = oracle.moe_align(ids.cpu().numpy(), 32, 16)
    assert np.array_equal(c.cpu().numpy(), wc) and np.array_equal(o.cpu().numpy(), wo)
    assert np.array_equal(s.cpu().numpy()[:int(wo[-1])], ws)
