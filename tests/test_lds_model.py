"""The LDS bank-conflict model against the tile model the pages print, and
the tree's index formula against the pages' worked tree states (CPU only)."""
import os

import pytest

from primitives_device_scan_amd import lds_model as m

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden():
    tiles, levels, one = {}, [], None
    for line in open(os.path.join(GOLDEN, "tile_model_day32.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        key, _, val = line.partition(":")
        f = val.split()
        if key == "tile":
            tiles[f[0]] = (int(f[1]), int(f[2]))
        elif key == "level":
            levels.append([int(v) for v in f])
        elif key == "one-term":
            one = int(f[0])
    return tiles, levels, one


def test_adds_and_requests_per_tile():
    tiles, _, one = _golden()
    assert (m.hs_adds(), m.hs_requests()) == tiles["hillis-steele"]
    assert (m.tree_adds(), m.tree_requests(m.pad_none)) == tiles["blelloch-plain"]
    assert (m.tree_adds(), m.tree_requests(m.pad_two)) == tiles["blelloch-padded"]
    assert m.tree_requests(m.pad_one) == one


def test_per_level_degrees():
    _, levels, _ = _golden()
    plain = m.tree_levels(pad=m.pad_none)
    one = m.tree_levels(pad=m.pad_one)
    two = m.tree_levels(pad=m.pad_two)
    assert len(plain) == len(levels) == 12
    for row, p, o, t in zip(levels, plain, one, two):
        stride, lanes, warps, dp, do, dt = row
        assert (p["stride"], p["lanes"], p["groups"]) == (stride, lanes, warps)
        assert (p["degree"], o["degree"], t["degree"]) == (dp, do, dt), stride


def test_padding_is_a_permutation_into_the_padded_array():
    for pad, words in ((m.pad_none, 4096), (m.pad_one, 4096 + 128), (m.pad_two, 4096 + 128 + 4)):
        img = [pad(i) for i in range(4096)]
        assert len(set(img)) == 4096 and max(img) < words


def _tree_states(x):
    """Runs the tree with the model's index formula, recording the buffer after every round."""
    n = len(x)
    buf = list(x)
    states = {}
    s, r = 1, 1
    while s < n:
        for a in range(n // (2 * s)):
            lo, hi = (2 * a + 1) * s - 1, (2 * a + 2) * s - 1
            buf[hi] += buf[lo]
        states[f"up{r}"] = list(buf)
        s, r = s * 2, r + 1
    buf[n - 1] = 0
    states["seed"] = list(buf)
    s, r = n // 2, 1
    while s >= 1:
        for a in range(n // (2 * s)):
            lo, hi = (2 * a + 1) * s - 1, (2 * a + 2) * s - 1
            left, right = buf[lo], buf[hi]
            buf[lo], buf[hi] = right, right + left
        states[f"down{r}"] = list(buf)
        s, r = s // 2, r + 1
    return states


def test_tree_index_formula_reproduces_the_worked_rounds():
    want = {}
    for line in open(os.path.join(GOLDEN, "blelloch_states.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, _, v = line.partition(":")
            want[k.strip()] = [int(t) for t in v.split()]
    got = _tree_states(want.pop("input"))
    assert got == want


@pytest.mark.parametrize("pad,expect_zero", [(m.pad_none, False), (m.pad_one, False), (m.pad_two, True)])
def test_conflict_cycles(pad, expect_zero):
    c = m.tree_conflict_cycles(pad=pad)
    assert (c == 0) == expect_zero
    assert c >= 0
